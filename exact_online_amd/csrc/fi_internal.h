// fi_internal.h -- declarations shared by the host API (fi_api.cpp) and the
// kernel launchers (fi_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fi {

constexpr int kMaxLevels = 40;
constexpr int kRunBlock = 256;     // positions per block of the persistent pass (= its LDS ring W)
constexpr int kLdsFftMax = 4096;  // largest complex FFT held in LDS (32 KiB in fp32)
constexpr int kTwLds = 132;       // LDS twiddle table: w_64^a, w_4096^b (64 each), w_16384^r (4)
// The run kernel's chain taps as 16-byte entries (four consecutive taps in
// reverse order), at the top of its FFT region: 64 + kRunBlock + 4 entries.
constexpr int kTapTableBytes = (64 + kRunBlock + 4) * 16;
// LDS FFT buffers hold one spare slot per 8 points (bank spreading).
constexpr int lds_fft_elems(int M) { return M + M / 8; }
// The run kernel's tile of side kRunBlock on the matrix cores keeps in its
// FFT region, above every staging area of the tiles up to 2048 points, the
// input block zero-padded (15 zeros before, 65 after) and the filter
// h[-64, 2 kRunBlock) (zero at negative lags) with one spare slot per 16
// (bank spreading), then the block's outputs y (handed to the other
// wavefronts, which store them during that tile).
constexpr int kMmXFloats = 15 + kRunBlock + 65;
constexpr int kMmHSlots = (64 + 2 * kRunBlock) + (64 + 2 * kRunBlock) / 16 + 4;
constexpr int kMmBytes = (kMmXFloats + kMmHSlots + kRunBlock) * 4;

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
    int T;                 // largest tile side done directly
    int W;                 // LDS accumulator window (positions) of the run kernel
    int XR;                // LDS ring of recent inputs (positions)
    int F;                 // LDS FFT buffer (complex points) of the run kernel
    int fftreg;            // bytes of the run kernel's LDS FFT / staging region
    int mm_off;            // bytes: its matrix-core tile data (above the staging areas)
    int io_bf16;
    float *hT;
    float *state;
    void *spec;            // float2
    int64_t spec_off[kMaxLevels];  // element (float2) offset of level q, -1 if none
    void *twf;             // Cx<float>
    void *scratch;         // Cx<float>
    int64_t sc_stride;     // complex elements per scratch slot
    int64_t sc_slots;
    int umax_fft;          // largest FFT tile side (0 if none)
};

// fi_create helpers (synchronous work on `st`)
hipError_t launch_transpose(const DevState &d, const void *h, hipStream_t st);
hipError_t launch_twiddles(void *twd, void *twf, int smax, hipStream_t st);
hipError_t launch_spectra(const DevState &d, int q, void *scd, int64_t scd_stride, int64_t slots,
                          const void *twd, hipStream_t st);
hipError_t launch_zero(float *p, int64_t n, hipStream_t st);

// online pieces
hipError_t launch_step(const DevState &d, int64_t t, const void *x_t, float *y_t, hipStream_t st);
hipError_t launch_tile(const DevState &d, int64_t i, hipStream_t st);   // FFT tiles (side > T)
// the red cell of position t fused with the direct tile of side U <= T that
// position t+1 completes
hipError_t launch_step_tile(const DevState &d, int64_t t, const void *x_t, float *y_t, int U, hipStream_t st);

// the persistent pass over all positions: open loop, closed loop, or a
// prompt of `prompt` given inputs followed by the closed loop
enum { kRunOpen = 0, kRunClosed = 1, kRunPrompted = 2, kRunModes = 3 };
hipError_t launch_run(const DevState &d, const void *x_in, int mode, int64_t prompt, float *y, void *x_out,
                      int grid, hipStream_t st);
int run_lds_bytes(const DevState &d);
int run_max_blocks_per_cu(const DevState &d, int mode);
int tile_fft_lds_bytes();

}  // namespace fi
