/*
 * fi_profile.h -- the phase-timing build of the library (hipcc -DFI_PROFILE=1,
 * built as libfi_prof.so; the product libfi.so carries none of this).
 *
 * In that build every persistent pass (fi_run_closed_loop, fi_run_prompted)
 * records, per team (workgroup) of its grid, the cycle sums of its chain
 * wavefront's phases, and for the first team's first channel the timeline of
 * every block of 256 positions (the cumulative time per
 * token of [FI] "Tempo di Risposta per Token (Figura 2c)", [FI] = the page
 * "Flash Inference: Inferenza in Tempo Quasi-Lineare per Modelli di Sequenza
 * a Convoluzione Lunga e Oltre").  Cycles are the shader clock.
 *
 * Layout of the record (uint64 elements):
 *   [0] grid G of the last pass, [1] slots per team S, [2] blocks N in the
 *   series, [3] clock source (0 = shader clock);
 *   [4 + g*S + k]  team g's sum k: 0 total, 1 per-channel setup, 2..5 chain
 *                  segments 0..3 (64 positions each), 6 the rest of the chain
 *                  wavefront's block work, 7 the team barrier after the chain,
 *                  8 the block stores after its tile, 9 blocks, 10 channels,
 *                  16 + q the block-boundary tiles of side 2^q (barriers
 *                  included), 40 + q their count;
 *   [4 + G*S + 8n + j]  block n of the first team's first channel, its chain
 *                  wavefront's clock at: j = 0 the block's start, 1 its first
 *                  chain step, 2 the end of its last chain step (1 and 2 are 0
 *                  for a block without a chain), 3 the end of the wait for the
 *                  block's loads, 4 the team barrier after the chain, 5 the
 *                  end of that barrier, 6 the end of the block-boundary tile,
 *                  7 the end of the block's stores.
 */
#ifndef FI_PROFILE_H_
#define FI_PROFILE_H_

#include <stdint.h>

#include "fi.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Synchronises the handle's stream and copies up to cap elements of the last
 * pass's record to the host array out.  Returns the record's full length,
 * 0 when the handle has none, FI_ERR_INVALID for a NULL handle or out or a
 * negative cap, FI_ERR_HIP when the copy fails. */
int64_t fi_profile_read(fi_handle *s, uint64_t *out, int64_t cap);

#ifdef __cplusplus
}
#endif
#endif /* FI_PROFILE_H_ */
