// fi_internal.h -- declarations shared by the host API (fi_api.cpp) and the
// kernel launchers (fi_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fi {

constexpr int kMaxLevels = 40;

// Phase-timing build (hipcc -DFI_PROFILE=1, a separate library; the product
// build leaves it 0 and carries none of it): each team of the persistent pass
// sums the cycles (s_memtime) of its chain wavefront's phases and writes them
// once at the end, plus, for the first team's first channel, the cycle count
// at the start of every block of 256 positions.
#ifndef FI_PROFILE
#define FI_PROFILE 0
#endif
constexpr bool kProfile = FI_PROFILE != 0;
constexpr int kProfSlots = 64;   // cycle sums per team
constexpr int kProfHeader = 4;   // grid, kProfSlots, blocks in the series, clock source (0 = s_memtime)
constexpr int kProfSeriesW = 8;  // timestamps per block in the series (see fi_profile.h)
enum {
    kPfTotal = 0,      // the team's whole run
    kPfSetup = 1,      // per channel: LDS tables before the first block
    kPfSeg = 2,        // + k: segment k of the chain (64 positions each), k < 4
    kPfChainRest = 6,  // chain wavefront's block work around the segments (loads, recompute, LDS writes)
    kPfWait = 7,       // the team barrier after the chain
    kPfStore = 8,      // the block's y / x stores after its tile
    kPfBlocks = 9,     // blocks run (a count)
    kPfChannels = 10,  // channels run (a count)
    kPfPrologue = 11,  // chain wavefront: block start to its first chain step (part of kPfChainRest)
    kPfEpilogue = 12,  // chain wavefront: last chain step to the barrier (part of kPfChainRest)
    kPfLoadWait = 13,  // the wait for the block's loads after its chain (part of kPfEpilogue)
    kPfHwChain = 14,   // where the chain wavefront runs: XCC id << 32 | HW_ID register
    kPfHwHelper = 15,  // the same for the team's other wavefront
    kPfTile = 16,      // + q: the block-boundary tile of side 2^q, barriers included
    kPfTileCount = 40  // + q: how many such tiles
};
constexpr int kRunBlock = 256;     // positions per block of the persistent pass (= its LDS ring W)
constexpr int kLdsFftMax = 4096;  // largest complex FFT held in LDS (32 KiB in fp32)
constexpr int kTwLds = 132;       // LDS twiddle table: w_64^a, w_4096^b (64 each), w_16384^r (4)
// The run kernel's chain taps as 16-byte entries (four consecutive taps in
// reverse order), at the top of its FFT region: 64 + kRunBlock + 4 entries.
constexpr int kTapTableBytes = (64 + kRunBlock + 4) * 16;
// LDS FFT buffers hold one spare slot per 8 points (bank spreading).
constexpr int lds_fft_elems(int M) { return M + M / 8; }
// The run kernel keeps in its FFT region, above every staging area of the
// tiles up to 2048 points, the block's inputs zero-padded (15 zeros before,
// 65 after; the open loop's block triangle on the matrix cores reads them,
// and the other wavefront stores them as x_out), then the block's outputs y
// (handed to the other wavefront, which stores them during the next block).
constexpr int kMmXFloats = 15 + kRunBlock + 65;
constexpr int kMmBytes = (kMmXFloats + kRunBlock) * 4;
// The block products on the matrix cores in fp16 halves (hi + lo of each
// operand, scaled by powers of two) -- the tiles of side kRunBlock and
// 2 kRunBlock, and (TRI: runs with blocks whose inputs are all given) those
// blocks' own triangles -- keep, at the bottom of the FFT region above its
// first KiB (the two wavefronts' hand-over area), the filter table -- lags
// lo .. lo + n - 1, the hi parts then the lo parts -- and the slots of input
// blocks, each two reversed copies (the second shifted by one position) of hi
// and of lo parts.  FFT tiles of side >= 4 kRunBlock and their staging
// overwrite the area; it is rebuilt after them.  A triangle is a product at
// lag offset 0, so TRI adds 256 zero lags below the table (lag 0 included)
// and a fourth slot, placed first so that it lies below the staging area of
// the FFT tile that follows its block; without TRI the table starts at lag 1
// (lags below 16 are never read) and the three slots are the blocks at 0,
// 256 and 512 mod 1024.
constexpr int kX16N = 304;
constexpr int kH16Off = 1024;
constexpr int kX16Slot = 4 * kX16N;   // halfs per slot
template <bool TRI>
struct F16Area {
    static constexpr int kLo = TRI ? -272 : -16;       // the table's lowest lag
    static constexpr int kN = TRI ? 1296 : 1040;       // lags in the table
    static constexpr int kFirst = TRI ? 0 : 1;         // the lowest nonzero lag
    static constexpr int kSlots = TRI ? 4 : 3;
    static constexpr int kXOff = kH16Off + 2 * kN * 2;   // bytes
    // slot s (the block at 256 s mod 1024), in halfs from kXOff
    static constexpr int slot_off(int s) { return (TRI ? ((s + 1) & 3) : s) * kX16Slot; }
    static constexpr int kEnd = kXOff + kSlots * kX16Slot * 2;
};
static_assert(F16Area<true>::kXOff + kX16Slot * 2 <= lds_fft_elems(1024) * 8,
              "slot 3 lies below the staging of the 1024-point tile");
// The run kernel's FFT / staging region has one fixed layout (compile-time
// offsets, whatever L is): the staging area of the largest staged tile (side
// 2048: its transform buffer and input block; smaller tiles also stage their
// spectrum, which fits below), then the matrix-core tile's data, then the
// chain's tap table at the top.  Tiles of side >= 4096 transform across all
// of it (their data and the taps are rebuilt afterwards).
constexpr int kRunMmOff = (lds_fft_elems(2048) * 8 + 4 * 2048 + 15) / 16 * 16;
constexpr int kRunFftReg = lds_fft_elems(kLdsFftMax) * 8 > kRunMmOff + kMmBytes + kTapTableBytes
                               ? lds_fft_elems(kLdsFftMax) * 8
                               : kRunMmOff + kMmBytes + kTapTableBytes;
static_assert(lds_fft_elems(1024) * 8 + 4 * 1024 + 8 * (1024 + 2) <= kRunMmOff, "staging of the tiles up to 1024 fits");
static_assert(F16Area<true>::kEnd <= kRunMmOff && F16Area<false>::kEnd <= kRunMmOff && kH16Off % 16 == 0 &&
                  F16Area<true>::kXOff % 16 == 0 && F16Area<false>::kXOff % 16 == 0,
              "the fp16 tile area fits below the matrix-core data");

// Device state of one handle.  Layouts (rows padded to LS = L rounded up to 64):
//   hT[D][LS]      filter, one contiguous row per channel c, fp32
//   state[C][LS]   per channel (b, c), ch = b*D + c: positions below the
//                  current one hold x (the input history), the others hold the
//                  accumulated tile contributions (the two share one slot per
//                  position, as the activation buffer is reused for the mixer
//                  output in the pages' memory optimisation)
//   spec           per FFT level q (U = 2^q): [D][U + 2] float2, G[k] / (4U) with
//                  G the 2U-point DFT of the tile's filter segment, entry p < U
//                  holding frequency brev(p) (the forward FFT's position
//                  order), entry U holding G[U]
//   twf            twiddles, twf[S + m] = exp(-2 pi i m / S), S = 1 .. 2^smax
//                  (spectra in bit-reversed frequency order: entry p is
//                  frequency brev(p))
//   scratch        [slots][sc_stride] complex fp32 for FFTs larger than LDS
struct DevState {
    int64_t B, D, L, C, LS;
    // Channels are (set, b, c): `fset` batch rows share one set of D filter
    // rows.  The single mixer has one set (fset = B, DF = D); the layer stack
    // has one per layer (DF = M D filter rows).
    int64_t fset, DF;
    int T;                 // largest tile side done directly
    int W;                 // LDS accumulator window (positions) of the run kernel
    int XR;                // LDS ring of recent inputs (positions)
    int F;                 // LDS FFT buffer (complex points) of the run kernel
    int fftreg;            // bytes of the run kernel's LDS FFT / staging region (kRunFftReg)
    int mm_off;            // bytes: its matrix-core tile data (kRunMmOff)
    int io_bf16;
    float *hT;
    float *pre;            // [D][kRunBlock]: prefix sums of the closed-loop chain's scaled taps
    float *state;
    void *spec;            // float2
    int64_t spec_off[kMaxLevels];  // element (float2) offset of level q, -1 if none
    void *twf;             // Cx<float>
    void *scratch;         // Cx<float>
    int64_t sc_stride;     // complex elements per scratch slot
    int64_t sc_slots;
    int umax_fft;          // largest FFT tile side (0 if none)
    unsigned long long *prof;   // phase-timing build only (else NULL): header, per-team sums, series
    int64_t prof_n;             // its length in elements
};

// The fixed device workspace of fi_conv_static (per device, never freed):
// its device address on the current device, looked up once per device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void **ptr, size_t *bytes);

// fi_create helpers (synchronous work on `st`)
hipError_t launch_transpose(const DevState &d, const void *h, hipStream_t st);
hipError_t launch_twiddles(void *twd, void *twf, int smax, hipStream_t st);
hipError_t launch_spectra(const DevState &d, int q, void *scd, int64_t scd_stride, int64_t slots,
                          const void *twd, hipStream_t st);
hipError_t launch_zero(float *p, int64_t n, hipStream_t st);
hipError_t launch_prefix(const DevState &d, hipStream_t st);

// online pieces
hipError_t launch_step(const DevState &d, int64_t t, const void *x_t, float *y_t, hipStream_t st);
hipError_t launch_tile(const DevState &d, int64_t i, hipStream_t st);   // FFT tiles (side > T)
// the red cell of position t fused with the direct tile of side U <= T that
// position t+1 completes
hipError_t launch_step_tile(const DevState &d, int64_t t, const void *x_t, float *y_t, int U, hipStream_t st);

// the layer stack: one position of every layer's red cell and block for
// every batch row over P workgroups that pass tagged partial products, then
// (fused when its side is <= kChainFuseMax) the tile all layers' channels
// need at t + 1
#ifndef FI_CHAIN_FUSE
#define FI_CHAIN_FUSE 16
#endif
#ifndef FI_CHAIN_WORKGROUPS
#define FI_CHAIN_WORKGROUPS 16
#endif
constexpr int kChainFuseMax = FI_CHAIN_FUSE;
constexpr int kChainMaxWorkgroups = FI_CHAIN_WORKGROUPS;
constexpr int kChainStageBytes = 96 * 1024;   // LDS for the vectors and the staged accumulators
constexpr int64_t kChainMaxD = 8192;           // a D-vector of a block in LDS
constexpr int64_t kChainMaxTags = (int64_t)1 << 30;   // L M per run: tags of two runs never meet
struct StackChain {
    int64_t B, M;
    int act, P;
    const float *w1, *w2t;
    float *xnext, *hist;
    unsigned long long *part;
    int *fail;
};
int stack_chain_lds_bytes(int64_t B, int64_t D, int64_t M, int P, int *pre);
hipError_t launch_stack_chain(const DevState &d, const StackChain &sc, const float *x0, const float *noise,
                              float sigma, float *y, float *x_out, int64_t t, unsigned tag0, int fuse_u,
                              hipStream_t st);
hipError_t launch_tile_direct(const DevState &d, int64_t i, int U, hipStream_t st);
// a plain fp32 transpose: dst[c][r] = src[r][c], r < rows, c < cols (row
// stride of dst: ld >= rows, entries [rows, ld) zeroed)
hipError_t launch_transpose_f32(const float *src, float *dst, int64_t rows, int64_t cols, int64_t ld,
                                hipStream_t st);

// the persistent pass over all positions: open loop, closed loop, or a
// prompt of `prompt` given inputs followed by the closed loop
enum { kRunOpen = 0, kRunClosed = 1, kRunPrompted = 2, kRunModes = 3 };
hipError_t launch_run(const DevState &d, const void *x_in, int mode, int64_t prompt, float *y, void *x_out,
                      int grid, hipStream_t st);
int run_lds_bytes(const DevState &d);
int run_max_blocks_per_cu(const DevState &d, int mode);
int tile_fft_lds_bytes();

}  // namespace fi
