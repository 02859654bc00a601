// fi_kernels.hip -- gfx950 kernels of the exact online causal long convolution.
//
// [FI] = the page "Flash Inference: Inferenza in Tempo Quasi-Lineare per
// Modelli di Sequenza a Convoluzione Lunga e Oltre" (lowest.today summary of
// arXiv 2410.12982).
//
// Per channel (b, c): y[t] = sum_{s<=t} h[t-s] x[s], computed online with the
// relaxed tiling of [FI] "Strategia di Tiling (Algoritmo 1)": after position
// i-1, the tile of side U = lowbit(i) adds the contribution of x[i-U, i) to
// y[i, i+U) ([FI] "Definizione di Aggregazione di Contribuzione", tau).
//
// Kernels:
//   k_transpose / k_twiddles / k_spectra   fi_create: filter rows, twiddle
//       tables, and the per-level filter spectra ([FI] "Ottimizzazione della
//       Memoria": the filter DFT is precomputed for each block size).
//   k_step, k_tile_direct, k_tile_fft       one online step (fi_step).
//   k_run                                   all L steps in one persistent pass:
//       one wavefront per channel; no grid-wide synchronisation is ever needed
//       because channels are independent ([FI] "Definizione Specifica di
//       LCSM": the mixer is a per-channel Hadamard convolution).
#include "fi_device.hpp"
#include "fi_internal.h"

namespace fi {

// ------------------------------------------------------------------ io
template <bool BF16>
__device__ __forceinline__ float load_io(const void* p, int64_t idx) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[idx]);
    else return static_cast<const float*>(p)[idx];
}
template <bool BF16>
__device__ __forceinline__ void store_io(void* p, int64_t idx, float v) {
    if constexpr (BF16) static_cast<uint16_t*>(p)[idx] = f32_to_bf16_bits(v);
    else static_cast<float*>(p)[idx] = v;
}

__device__ __forceinline__ int ilog2(int64_t v) { return 63 - __builtin_clzll((unsigned long long)v); }

// ================================================================ fi_create
// h[L][D] -> hT[D][LS] (fp32), zero padding in [L, LS).  64x64 tiles via LDS.
template <bool BF16>
__global__ __launch_bounds__(256) void k_transpose(const void* h, float* hT, int64_t L, int64_t D, int64_t LS) {
    __shared__ float tile[64][65];
    const int64_t c0 = (int64_t)blockIdx.x * 64, j0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    for (int r = ty; r < 64; r += 4) {
        const int64_t j = j0 + r, c = c0 + tx;
        tile[r][tx] = (j < L && c < D) ? load_io<BF16>(h, j * D + c) : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t c = c0 + r, j = j0 + tx;
        if (c < D && j < LS) hT[c * LS + j] = tile[tx][r];
    }
}

// twd[S + m] = exp(-2 pi i m / S) in fp64 (sincospi of an exact dyadic
// argument), twf its fp32 rounding; S = 1, 2, 4, ..., 2^smax.
__global__ void k_twiddles(Cx<double>* twd, Cx<float>* twf, int smax) {
    const int64_t n = (int64_t)2 << smax;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        if (idx == 0) {
            twd[0] = {1.0, 0.0};
            twf[0] = {1.f, 0.f};
            continue;
        }
        const int s = ilog2(idx);
        const int64_t S = (int64_t)1 << s, m = idx - S;
        double sn, cs;
        sincospi(2.0 * (double)m / (double)S, &sn, &cs);
        twd[idx] = {cs, -sn};
        twf[idx] = {(float)cs, (float)-sn};
    }
}

// Filter spectra of level q (U = 2^q = M complex points): with the tile's
// length-2U filter segment g[n] = h[n] for 1 <= n < 2U (g[0] = 0: lag 0 never
// reaches the outputs [U, 2U) that are kept, [FI] "Trucco di Convoluzione
// Circolare"), z[n] = g[2n] + i g[2n+1], Z = DFT_M(z) in fp64, and per
// position p (frequency k, partner frequency M-k at p'):
//   E = (Z[p] + conj Z[p'])/2,  d = Z[p] - conj Z[p'],  w = exp(-2 pi i k/M)
//   alpha = (E + d/4 (1 - w)) / M,   beta = d/4 (1 + w) / M
// so that the tile's packed output spectrum is W = alpha Z_x + beta conj(Z_x').
__global__ __launch_bounds__(64) void k_spectra(const float* hT, int64_t LS, int64_t L, int64_t D, int M,
                                                float4* spec, Cx<double>* scd, int64_t scd_stride,
                                                const Cx<double>* twd) {
    extern __shared__ __align__(16) unsigned char smem[];
    Cx<double>* lbuf = reinterpret_cast<Cx<double>*>(smem);
    const int lane = threadIdx.x;
    const int F = M < kLdsFftMax ? M : kLdsFftMax;
    const int P = M / F, nb = ilog2(P);
    for (int64_t c = blockIdx.x; c < D; c += gridDim.x) {
        const float* hr = hT + c * LS;
        auto g = [&](int64_t n) -> double { return (n >= 1 && n < L) ? (double)hr[n] : 0.0; };
        Cx<double>* Z;
        if (P == 1) {
            for (int n = lane; n < M; n += kWave) lbuf[n] = {g(2 * n), g(2 * n + 1)};
            __syncthreads();
            fft_lds_any<false>(M, lbuf, twd);
            Z = lbuf;
        } else {
            Cx<double>* sc = scd + (int64_t)blockIdx.x * scd_stride;
            for (int n = lane; n < M; n += kWave) sc[n] = {g(2 * n), g(2 * n + 1)};
            __syncthreads();
            for (int S = M; S > F; S >>= 1) dif_pass(sc, M, S, twd);
            blocks_via_lds<false>(sc, M, F, lbuf, twd);
            Z = sc;
        }
        float4* out = spec + c * (int64_t)M;
        const double inv = 1.0 / (double)M;
        for (int p = lane; p < M; p += kWave) {
            const int blk = p / F, q = p % F;
            const int kl = brev_bits(blk, nb);
            const int k = kl + P * q;
            int pp;
            if (P == 1) pp = (M - p) & (M - 1);
            else if (kl == 0) pp = (F - q) & (F - 1);
            else pp = brev_bits(P - kl, nb) * F + (F - 1 - q);
            const Cx<double> z1 = Z[p], z2c = cconj(Z[pp]);
            const Cx<double> E = {(z1.x + z2c.x) * 0.5, (z1.y + z2c.y) * 0.5};
            const Cx<double> d4 = {(z1.x - z2c.x) * 0.25, (z1.y - z2c.y) * 0.25};
            const Cx<double> w = twd[M + k];
            const Cx<double> a = cadd(E, cmul(d4, Cx<double>{1.0 - w.x, -w.y}));
            const Cx<double> bb = cmul(d4, Cx<double>{1.0 + w.x, w.y});
            out[p] = make_float4((float)(a.x * inv), (float)(a.y * inv), (float)(bb.x * inv), (float)(bb.y * inv));
        }
        __syncthreads();
    }
}

__global__ void k_zero(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// ============================================================== FFT tile
// Where a tile's outputs go: positions below `wend` into the LDS ring `accw`
// (slot = position & wmask), the others into the channel's global row.
struct TileSink {
    float* row;
    float* accw;
    int64_t wend;
    int wmask;
    int64_t L;
};

// Adds (a, b) to positions (o, o+1); o is even and wend is even.
__device__ __forceinline__ void sink_pair(const TileSink& s, int64_t o, float a, float b) {
    if (o >= s.L) return;
    if (o < s.wend) {
        s.accw[o & s.wmask] += a;
        if (o + 1 < s.L) s.accw[(o + 1) & s.wmask] += b;
    } else if (o + 1 < s.L) {
        float2* pp = reinterpret_cast<float2*>(s.row + o);
        float2 v = *pp;
        v.x += a;
        v.y += b;
        *pp = v;
    } else {
        s.row[o] += a;
    }
}

__device__ __forceinline__ void untangle_pair(Cx<float>* Z, const float4* spec, int pa, int pb) {
    const Cx<float> z1 = Z[pa], z2 = Z[pb];
    const float4 s1 = spec[pa], s2 = spec[pb];
    // W = alpha Z + beta conj(Z_partner)
    const Cx<float> w1 = cadd(cmul(Cx<float>{s1.x, s1.y}, z1), cmul(Cx<float>{s1.z, s1.w}, cconj(z2)));
    const Cx<float> w2 = cadd(cmul(Cx<float>{s2.x, s2.y}, z2), cmul(Cx<float>{s2.z, s2.w}, cconj(z1)));
    Z[pa] = w1;
    Z[pb] = w2;
}

// The tile tau(x, [i-U, i), h, [i, i+U)) as the circular convolution of
// length 2U of [x[i-U..i), 0_U] with the segment h[1..2U) ([FI] "Trucco di
// Convoluzione Circolare": outputs U..2U-1 are free of wrap-around; the input
// block is padded on the right, [FI] "Dettagli di Implementazione").  The real
// sequences are packed in pairs into M = U complex points; the per-level
// (alpha, beta) fold the packing, the filter spectrum and the 1/M scale.
// `row` holds the channel's input history (row[s] = x[s] for s < i).
__device__ __noinline__ void fft_tile(int U, int64_t i, const float* row, const float4* spec,
                                      Cx<float>* lbuf, Cx<float>* sc, const Cx<float>* tw,
                                      TileSink out) {
    const int M = U;
    const int lane = threadIdx.x & (kWave - 1);
    const float2* xs = reinterpret_cast<const float2*>(row + (i - U));
    if (M <= kLdsFftMax) {
        for (int n = lane; n < M; n += kWave) {
            Cx<float> z = {0.f, 0.f};
            if (n < (M >> 1)) {
                const float2 v = xs[n];
                z = {v.x, v.y};
            }
            lbuf[n] = z;
        }
        __syncthreads();
        fft_lds_any<false>(M, lbuf, tw);
        for (int q = lane; q <= (M >> 1); q += kWave) untangle_pair(lbuf, spec, q, (M - q) & (M - 1));
        __syncthreads();
        fft_lds_any<true>(M, lbuf, tw);
        for (int m = lane; m < (M >> 1); m += kWave) {
            const Cx<float> w = lbuf[(M >> 1) + m];
            sink_pair(out, i + 2 * m, w.x, w.y);
        }
        __syncthreads();
        return;
    }
    const int F = kLdsFftMax, P = M / F, nb = ilog2(P);
    const int half = M >> 1;
    // first decimation-in-frequency pass fused with the load (upper half is 0)
    for (int j = lane; j < half; j += kWave) {
        const float2 v = xs[j];
        const Cx<float> z = {v.x, v.y};
        sc[j] = z;
        sc[j + half] = cmul(z, twiddle<false>(tw, M, j));
    }
    __syncthreads();
    for (int S = half; S > F; S >>= 1) dif_pass(sc, M, S, tw);
    blocks_via_lds<false>(sc, M, F, lbuf, tw);
    for (int p = 0; p < P; ++p) {
        const int pp = partner_block(p, P, nb);
        if (pp < p) continue;
        if (pp == p) {
            const int kl = brev_bits(p, nb);
            for (int q = lane; q < F; q += kWave) {
                const int q2 = kl == 0 ? ((F - q) & (F - 1)) : (F - 1 - q);
                if (q2 >= q) untangle_pair(sc, spec, p * F + q, p * F + q2);
            }
        } else {
            for (int q = lane; q < F; q += kWave) untangle_pair(sc, spec, p * F + q, pp * F + (F - 1 - q));
        }
    }
    __syncthreads();
    blocks_via_lds<true>(sc, M, F, lbuf, tw);
    for (int S = 2 * F; S < M; S <<= 1) dit_pass(sc, M, S, tw);
    // last inverse pass (size M) fused with the output; only the upper half
    // (outputs U..2U-1 of the circular convolution) is needed
    for (int j = lane; j < half; j += kWave) {
        const Cx<float> v0 = sc[j];
        const Cx<float> v1 = cmul(sc[j + half], twiddle<true>(tw, M, j));
        const Cx<float> w = csub(v0, v1);
        sink_pair(out, i + 2 * j, w.x, w.y);
    }
    __syncthreads();
}

// ================================================================ fi_step
template <bool BF16>
__global__ void k_step(float* state, const float* hT, int64_t LS, int64_t D, int64_t C, int64_t t,
                       const void* x_t, float* y_t) {
    const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (ch >= C) return;
    const int64_t c = ch % D;
    const float xv = load_io<BF16>(x_t, ch);
    float* slot = state + ch * LS + t;
    y_t[ch] = __builtin_fmaf(hT[c * LS], xv, *slot);  // accumulated tiles + red cell
    *slot = xv;                                        // the slot now holds x[t]
}

// Direct Toeplitz tile: acc[i+r] += sum_{j<U} x[i-U+j] h[U+r-j], r in [0, U).
__global__ void k_tile_direct(float* state, const float* hT, int64_t LS, int64_t L, int64_t D, int64_t C,
                              int64_t i, int U) {
    const int64_t n = C * (int64_t)U;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ch = idx / U;
        const int r = (int)(idx % U);
        if (i + r >= L) continue;
        const float* xr = state + ch * LS + (i - U);
        const float* hr = hT + (ch % D) * LS + U + r;
        float acc = 0.f;
        for (int j = 0; j < U; ++j) acc = __builtin_fmaf(xr[j], hr[-j], acc);
        state[ch * LS + i + r] += acc;
    }
}

__global__ __launch_bounds__(64) void k_tile_fft(DevState d, int64_t i, int U) {
    extern __shared__ __align__(16) unsigned char smem[];
    Cx<float>* lbuf = reinterpret_cast<Cx<float>*>(smem);
    const int q = ilog2(U);
    const float4* spec = static_cast<const float4*>(d.spec) + d.spec_off[q];
    for (int64_t ch = blockIdx.x; ch < d.C; ch += gridDim.x) {
        float* row = d.state + ch * d.LS;
        Cx<float>* sc = static_cast<Cx<float>*>(d.scratch) + (int64_t)blockIdx.x * d.sc_stride;
        TileSink s{row, nullptr, i, 0, d.L};
        fft_tile(U, i, row, spec + (ch % d.D) * (int64_t)U, lbuf, sc, static_cast<const Cx<float>*>(d.twf), s);
    }
}

// ============================================================ persistent run
// One wavefront per channel runs all L positions.  Positions are processed in
// blocks of 64, lane m holding position t0+m:
//  * the red cells and the tiles of side < 64 -- which all lie inside one
//    64-position block and together cover its lower triangle -- run in
//    registers: each new x is pushed into the accumulators of the later
//    positions of its block (a DPP lane shift slides the filter taps), so the
//    same products reach the same outputs as those tiles;
//  * at each block boundary i = t0+64 the tile of side U = lowbit(i) >= 64
//    runs: a direct Toeplitz product from LDS when U <= T, else the FFT tile.
// Accumulators of positions [t0, t0+W) live in an LDS ring; tiles add their
// outputs beyond it to the channel's global row, which is read back when the
// position enters the ring.  The global row holds x below the current
// position, so the FFT tiles read their input blocks from it.
struct RunArgs {
    DevState d;
    const void* x_in;
    float* y;
    void* x_out;
};

__device__ __forceinline__ void direct_tile_lds(int64_t i, int U, const float* xring, int xmask,
                                                const float* htap, float* accw, int wmask, int64_t L) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int r = lane; r < U; r += kWave) {
        float acc = 0.f;
        const float* hp = htap + U + r;
#pragma unroll 8
        for (int j = 0; j < U; ++j) acc = __builtin_fmaf(xring[(i - U + j) & xmask], hp[-j], acc);
        if (i + r < L) accw[(i + r) & wmask] += acc;
    }
}

template <bool CLOSED, bool BF16>
__global__ __launch_bounds__(64) void k_run(RunArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const DevState& d = a.d;
    Cx<float>* lbuf = reinterpret_cast<Cx<float>*>(smem);
    float* accw = reinterpret_cast<float*>(smem + (size_t)d.F * sizeof(Cx<float>));
    float* xring = accw + d.W;
    float* htap = xring + d.XR;  // h[0 .. 2T)
    const int lane = threadIdx.x;
    const int wmask = d.W - 1, xmask = d.XR - 1;
    const int64_t L = d.L, D = d.D;
    const int G = gridDim.x, bid = blockIdx.x;
    // consecutive channels on the same XCD (workgroups go round-robin over
    // the 8 XCDs), so their strided y / x_out rows meet in one L2
    const int64_t ch0 = (G % 8 == 0) ? (int64_t)(bid % 8) * (G / 8) + bid / 8 : bid;
    const Cx<float>* tw = static_cast<const Cx<float>*>(d.twf);
    Cx<float>* sc = static_cast<Cx<float>*>(d.scratch) + (int64_t)bid * d.sc_stride;

    for (int64_t ch = ch0; ch < d.C; ch += G) {
        const int64_t b = ch / D, c = ch % D;
        float* row = d.state + ch * d.LS;
        const float* hrow = d.hT + c * d.LS;
        for (int64_t q = 4 * lane; q < d.LS; q += 4 * kWave) *reinterpret_cast<float4*>(row + q) = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q = lane; q < d.W; q += kWave) accw[q] = 0.f;
        for (int q = lane; q < 2 * d.T; q += kWave) htap[q] = q < L ? hrow[q] : 0.f;
        const float h0 = hrow[0];
        const float hlane = (lane >= 1 && lane < L) ? hrow[lane] : 0.f;  // taps h[1..63] for the in-block push
        __syncthreads();

        float xcur = 0.f;   // closed loop: x at the next position (uniform)
        float xb_next = 0.f;  // open loop: inputs of the next block, lane m -> position t0+64+m
        if constexpr (CLOSED) {
            xcur = load_io<BF16>(a.x_in, b * D + c);
        } else {
            xb_next = lane < L ? load_io<BF16>(a.x_in, (b * L + lane) * D + c) : 0.f;
        }
        for (int64_t t0 = 0; t0 < L; t0 += kWave) {
            const int64_t tl = t0 + lane;
            const float xb = xb_next;
            if constexpr (!CLOSED) {
                const int64_t tn = tl + kWave;
                xb_next = tn < L ? load_io<BF16>(a.x_in, (b * L + tn) * D + c) : 0.f;
            }
            const int64_t pin = t0 + d.W + lane;  // position entering the LDS window at this block's end
            const float in_acc = pin < L ? row[pin] : 0.f;
            float pend = accw[tl & wmask];
            float hs = hlane;
            float ykeep = 0.f;
            const float xfirst = xcur;
#pragma unroll
            for (int m = 0; m < kWave; ++m) {
                if constexpr (CLOSED) {
                    const float ya = __builtin_fmaf(h0, xcur, pend);  // red cell: acc[t] + h[0] x[t]
                    ykeep = (lane == m) ? ya : ykeep;
                    const float ym = readlane(ya, m);
                    pend = __builtin_fmaf(hs, xcur, pend);           // push x[t0+m] into later positions
                    hs = wave_shr1(hs);
                    float xn = tanh_fast(ym);
                    if constexpr (BF16) xn = round_bf16(xn);
                    xcur = xn;
                } else {
                    const float xm = readlane(xb, m);
                    pend = __builtin_fmaf(hs, xm, pend);
                    hs = wave_shr1(hs);
                }
            }
            // Lane m's accumulator stopped changing at step m (later pushes
            // carry a zero tap there), so pend now holds what step m saw.
            float xkeep;
            if constexpr (CLOSED) {
                // x[t0+m] for m >= 1 is the feedback of y[t0+m-1]: the same
                // instructions on the same values as in the chain above
                float tx = tanh_fast(ykeep);
                if constexpr (BF16) tx = round_bf16(tx);
                xkeep = wave_shr1(tx);
                if (lane == 0) xkeep = xfirst;
            } else {
                xkeep = xb;
                ykeep = __builtin_fmaf(h0, xb, pend);
            }
            if (tl < L) {
                const int64_t o = (b * L + tl) * D + c;
                a.y[o] = ykeep;
                if (a.x_out) store_io<BF16>(a.x_out, o, xkeep);
                row[tl] = xkeep;  // the slot of a consumed accumulator now holds x
            }
            xring[tl & xmask] = xkeep;
            accw[tl & wmask] = in_acc;  // slot of position tl now holds position tl + W
            __syncthreads();
            const int64_t i = t0 + kWave;
            if (i < L) {
                const int U = (int)(i & -i);
                if (U <= d.T) {
                    direct_tile_lds(i, U, xring, xmask, htap, accw, wmask, L);
                } else {
                    TileSink s{row, accw, i + d.W, wmask, L};
                    const float4* spec = static_cast<const float4*>(d.spec) + d.spec_off[ilog2(U)] + c * (int64_t)U;
                    fft_tile(U, i, row, spec, lbuf, sc, tw, s);
                }
            }
            __syncthreads();
        }
    }
}

// ================================================================ launchers
static int grid_for(int64_t n, int block, int cap = 65536) {
    int64_t g = (n + block - 1) / block;
    if (g < 1) g = 1;
    return (int)(g < cap ? g : cap);
}

hipError_t launch_transpose(const DevState& d, const void* h, hipStream_t st) {
    dim3 grid((unsigned)((d.D + 63) / 64), (unsigned)((d.LS + 63) / 64));
    if (d.io_bf16) hipLaunchKernelGGL((k_transpose<true>), grid, dim3(256), 0, st, h, d.hT, d.L, d.D, d.LS);
    else hipLaunchKernelGGL((k_transpose<false>), grid, dim3(256), 0, st, h, d.hT, d.L, d.D, d.LS);
    return hipGetLastError();
}

hipError_t launch_twiddles(void* twd, void* twf, int smax, hipStream_t st) {
    const int64_t n = (int64_t)2 << smax;
    hipLaunchKernelGGL(k_twiddles, dim3(grid_for(n, 256, 4096)), dim3(256), 0, st, static_cast<Cx<double>*>(twd),
                       static_cast<Cx<float>*>(twf), smax);
    return hipGetLastError();
}

hipError_t launch_spectra(const DevState& d, int q, void* scd, int64_t scd_stride, int64_t slots,
                          const void* twd, hipStream_t st) {
    const int M = 1 << q;
    const int F = M < kLdsFftMax ? M : kLdsFftMax;
    const size_t lds = (size_t)F * sizeof(Cx<double>);
    const int grid = (int)(d.D < slots ? d.D : slots);
    float4* spec = static_cast<float4*>(d.spec) + d.spec_off[q];
    hipLaunchKernelGGL(k_spectra, dim3(grid), dim3(64), lds, st, d.hT, d.LS, d.L, d.D, M, spec,
                       static_cast<Cx<double>*>(scd), scd_stride, static_cast<const Cx<double>*>(twd));
    return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(k_zero, dim3(grid_for(n, 256, 8192)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_step(const DevState& d, int64_t t, const void* x_t, float* y_t, hipStream_t st) {
    const int grid = grid_for(d.C, 256, 1 << 30);
    if (d.io_bf16) hipLaunchKernelGGL((k_step<true>), dim3(grid), dim3(256), 0, st, d.state, d.hT, d.LS, d.D, d.C, t, x_t, y_t);
    else hipLaunchKernelGGL((k_step<false>), dim3(grid), dim3(256), 0, st, d.state, d.hT, d.LS, d.D, d.C, t, x_t, y_t);
    return hipGetLastError();
}

int tile_fft_lds_bytes() { return kLdsFftMax * (int)sizeof(Cx<float>); }

hipError_t launch_tile(const DevState& d, int64_t i, hipStream_t st) {
    const int U = (int)(i & -i);
    if (U <= d.T) {
        hipLaunchKernelGGL(k_tile_direct, dim3(grid_for(d.C * (int64_t)U, 256)), dim3(256), 0, st, d.state, d.hT,
                           d.LS, d.L, d.D, d.C, i, U);
    } else {
        const int F = U < kLdsFftMax ? U : kLdsFftMax;
        const int grid = (int)(d.C < d.sc_slots ? d.C : d.sc_slots);
        hipLaunchKernelGGL(k_tile_fft, dim3(grid), dim3(64), (size_t)F * sizeof(Cx<float>), st, d, i, U);
    }
    return hipGetLastError();
}

int run_lds_bytes(const DevState& d) {
    return d.F * (int)sizeof(Cx<float>) + (d.W + d.XR + 2 * d.T) * (int)sizeof(float);
}

int run_max_blocks_per_cu(const DevState& d, int closed) {
    int nb = 0;
    const void* fn;
    if (closed) fn = d.io_bf16 ? (const void*)k_run<true, true> : (const void*)k_run<true, false>;
    else fn = d.io_bf16 ? (const void*)k_run<false, true> : (const void*)k_run<false, false>;
    const int lds = run_lds_bytes(d);
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 64, lds) != hipSuccess) return 0;
    return nb;
}

hipError_t launch_run(const DevState& d, const void* x_in, int closed, float* y, void* x_out, int grid,
                      hipStream_t st) {
    RunArgs a{d, x_in, y, x_out};
    const size_t lds = (size_t)run_lds_bytes(d);
    if (closed) {
        if (d.io_bf16) hipLaunchKernelGGL((k_run<true, true>), dim3(grid), dim3(64), lds, st, a);
        else hipLaunchKernelGGL((k_run<true, false>), dim3(grid), dim3(64), lds, st, a);
    } else {
        if (d.io_bf16) hipLaunchKernelGGL((k_run<false, true>), dim3(grid), dim3(64), lds, st, a);
        else hipLaunchKernelGGL((k_run<false, false>), dim3(grid), dim3(64), lds, st, a);
    }
    return hipGetLastError();
}

}  // namespace fi
