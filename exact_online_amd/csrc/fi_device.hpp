// fi_device.hpp -- device building blocks for the gfx950 kernels: complex
// arithmetic, small in-register DFTs, wave-level Stockham FFTs in LDS and
// radix-2 passes over a global scratch buffer.
//
// Citations name the page "Flash Inference: Inferenza in Tempo Quasi-Lineare
// per Modelli di Sequenza a Convoluzione Lunga e Oltre" (lowest.today summary
// of arXiv 2410.12982), written [FI].  The FFT is the tool of [FI] "Definizione
// di Aggregazione di Contribuzione" (Lemma 1: an FFT evaluates a tile's
// contribution in O(n log n)); the algorithms below are the textbook ones:
// Stockham autosort (natural order in and out, twiddle before the butterfly)
// and decimation in frequency / in time for the passes outside LDS.
//
// Every routine here is executed by ONE wavefront (64 lanes) that owns the
// buffers it touches; workgroups are one wavefront wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_internal.h"

namespace fi {

constexpr int kWave = 64;

// ------------------------------------------------------------------ complex
template <typename R>
struct alignas(2 * sizeof(R)) Cx {
    R x, y;
};

template <typename R>
__device__ __forceinline__ Cx<R> cadd(Cx<R> a, Cx<R> b) { return {a.x + b.x, a.y + b.y}; }
template <typename R>
__device__ __forceinline__ Cx<R> csub(Cx<R> a, Cx<R> b) { return {a.x - b.x, a.y - b.y}; }
template <typename R>
__device__ __forceinline__ Cx<R> cmul(Cx<R> a, Cx<R> b) {
    return {a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x};
}
// a * conj(b)
template <typename R>
__device__ __forceinline__ Cx<R> cmulc(Cx<R> a, Cx<R> b) {
    return {a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y};
}
template <typename R>
__device__ __forceinline__ Cx<R> cconj(Cx<R> a) { return {a.x, -a.y}; }
// multiply by -i (forward) or +i (inverse)
template <bool INV, typename R>
__device__ __forceinline__ Cx<R> cmul_mi(Cx<R> a) {
    if constexpr (INV) return {-a.y, a.x};
    else return {a.y, -a.x};
}

// Twiddle tables: tw[S + m] = exp(-2*pi*i*m/S) for every power of two S and
// m in [0, S); the inverse transforms use the conjugate.
template <bool INV, typename R>
__device__ __forceinline__ Cx<R> twiddle(const Cx<R>* tw, int S, int m) {
    Cx<R> w = tw[S + m];
    if constexpr (INV) w.y = -w.y;
    return w;
}

// ------------------------------------------------------- in-register DFT_R
// Unnormalised DFT of R points: v_k <- sum_r v_r exp(-+2 pi i r k / R).
template <int R, bool INV, typename T>
__device__ __forceinline__ void dft(Cx<T>* v) {
    if constexpr (R == 2) {
        Cx<T> a = v[0], b = v[1];
        v[0] = cadd(a, b);
        v[1] = csub(a, b);
    } else if constexpr (R == 4) {
        Cx<T> s02 = cadd(v[0], v[2]), d02 = csub(v[0], v[2]);
        Cx<T> s13 = cadd(v[1], v[3]), d13 = cmul_mi<INV>(csub(v[1], v[3]));
        v[0] = cadd(s02, s13);
        v[2] = csub(s02, s13);
        v[1] = cadd(d02, d13);
        v[3] = csub(d02, d13);
    } else if constexpr (R == 8) {
        Cx<T> e[4] = {v[0], v[2], v[4], v[6]};
        Cx<T> o[4] = {v[1], v[3], v[5], v[7]};
        dft<4, INV>(e);
        dft<4, INV>(o);
        const T s = T(0.70710678118654752440);
        // o[k] *= w8^k, w8 = exp(-+ i pi / 4)
        Cx<T> o1 = INV ? Cx<T>{s * (o[1].x - o[1].y), s * (o[1].x + o[1].y)}
                       : Cx<T>{s * (o[1].x + o[1].y), s * (o[1].y - o[1].x)};
        Cx<T> o2 = cmul_mi<INV>(o[2]);
        Cx<T> o3 = INV ? Cx<T>{-s * (o[3].x + o[3].y), s * (o[3].x - o[3].y)}
                       : Cx<T>{s * (o[3].y - o[3].x), -s * (o[3].x + o[3].y)};
        v[0] = cadd(e[0], o[0]);
        v[4] = csub(e[0], o[0]);
        v[1] = cadd(e[1], o1);
        v[5] = csub(e[1], o1);
        v[2] = cadd(e[2], o2);
        v[6] = csub(e[2], o2);
        v[3] = cadd(e[3], o3);
        v[7] = csub(e[3], o3);
    }
}

// ------------------------------------------------ Stockham FFT in LDS
// One radix-R pass over M points held in LDS, current sub-transform length LS:
// butterfly j takes v_r = buf[j + r*M/R], multiplies by w_{LS*R}^{r*k}
// (k = j mod LS), applies DFT_R and stores at (j-k)*R + k + r*LS.  All reads of
// a pass complete before its writes (register staging), so it runs in place.
template <int M, int R, int LS, bool INV, typename T>
__device__ __forceinline__ void stockham_pass(Cx<T>* buf, const Cx<T>* tw) {
    constexpr int NBF = M / R;
    constexpr int PER = (NBF + kWave - 1) / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    Cx<T> v[PER][R];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int j = lane + kWave * u;
        if (NBF % kWave == 0 || j < NBF) {
            const int k = j & (LS - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) v[u][r] = buf[j + r * NBF];
            if constexpr (LS > 1) {
#pragma unroll
                for (int r = 1; r < R; ++r) v[u][r] = cmul(v[u][r], twiddle<INV>(tw, LS * R, r * k));
            }
            dft<R, INV>(v[u]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int j = lane + kWave * u;
        if (NBF % kWave == 0 || j < NBF) {
            const int k = j & (LS - 1);
            const int i0 = (j - k) * R + k;
#pragma unroll
            for (int r = 0; r < R; ++r) buf[i0 + r * LS] = v[u][r];
        }
    }
    __syncthreads();
}

template <int M, int LS, bool INV, typename T>
__device__ __forceinline__ void stockham_from(Cx<T>* buf, const Cx<T>* tw) {
    if constexpr (LS < M) {
        constexpr int R = (M / LS >= 8) ? 8 : ((M / LS >= 4) ? 4 : 2);
        stockham_pass<M, R, LS, INV>(buf, tw);
        stockham_from<M, LS * R, INV>(buf, tw);
    }
}

// Unnormalised M-point FFT of buf (LDS), natural order in and out.
template <int M, bool INV, typename T>
__device__ __forceinline__ void fft_lds(Cx<T>* buf, const Cx<T>* tw) {
    stockham_from<M, 1, INV>(buf, tw);
}

// Runtime-size dispatch for 2 <= M <= kLdsFftMax.
template <bool INV, typename T>
__device__ __noinline__ void fft_lds_any(int M, Cx<T>* buf, const Cx<T>* tw) {
    switch (M) {
        case 2: fft_lds<2, INV>(buf, tw); break;
        case 4: fft_lds<4, INV>(buf, tw); break;
        case 8: fft_lds<8, INV>(buf, tw); break;
        case 16: fft_lds<16, INV>(buf, tw); break;
        case 32: fft_lds<32, INV>(buf, tw); break;
        case 64: fft_lds<64, INV>(buf, tw); break;
        case 128: fft_lds<128, INV>(buf, tw); break;
        case 256: fft_lds<256, INV>(buf, tw); break;
        case 512: fft_lds<512, INV>(buf, tw); break;
        case 1024: fft_lds<1024, INV>(buf, tw); break;
        case 2048: fft_lds<2048, INV>(buf, tw); break;
        case 4096: fft_lds<4096, INV>(buf, tw); break;
        default: break;
    }
}

// ---------------------------------------------- passes over global scratch
// Radix-2 decimation in frequency on every sub-problem of size S of sc[0..M):
// (v0, v1) = (sc[b+j], sc[b+j+S/2]) -> (v0+v1, (v0-v1) w_S^j).  After the
// passes down to size F, the block of F points at p*F holds the DFT inputs of
// frequencies k = brev(p) + (M/F)*q (bit reversal over log2(M/F) bits).
template <typename T>
__device__ __forceinline__ void dif_pass(Cx<T>* sc, int M, int S, const Cx<T>* tw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int half = S >> 1;
    for (int n = lane; n < (M >> 1); n += kWave) {
        const int b = (n / half) * S, j = n % half;
        Cx<T> v0 = sc[b + j], v1 = sc[b + j + half];
        sc[b + j] = cadd(v0, v1);
        sc[b + j + half] = cmul(csub(v0, v1), twiddle<false>(tw, S, j));
    }
    __syncthreads();
}

// Inverse of dif_pass (unnormalised): (v0, v1 w_S^-j) -> (v0+., v0-.).
template <typename T>
__device__ __forceinline__ void dit_pass(Cx<T>* sc, int M, int S, const Cx<T>* tw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int half = S >> 1;
    for (int n = lane; n < (M >> 1); n += kWave) {
        const int b = (n / half) * S, j = n % half;
        Cx<T> v0 = sc[b + j];
        Cx<T> v1 = cmul(sc[b + j + half], twiddle<true>(tw, S, j));
        sc[b + j] = cadd(v0, v1);
        sc[b + j + half] = csub(v0, v1);
    }
    __syncthreads();
}

// FFT of each F-point block of sc[0..M) through the LDS buffer.
template <bool INV, typename T>
__device__ __forceinline__ void blocks_via_lds(Cx<T>* sc, int M, int F, Cx<T>* lbuf, const Cx<T>* tw) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int base = 0; base < M; base += F) {
        for (int q = lane; q < F; q += kWave) lbuf[q] = sc[base + q];
        __syncthreads();
        fft_lds_any<INV>(F, lbuf, tw);
        for (int q = lane; q < F; q += kWave) sc[base + q] = lbuf[q];
        __syncthreads();
    }
}

__device__ __forceinline__ int brev_bits(int v, int nb) {
    return nb == 0 ? 0 : (int)(__brev((unsigned)v) >> (32 - nb));
}

// Position of the partner frequency M-k for the layout above
// (P = M/F blocks, nb = log2 P): block p with klow = brev(p) pairs with block
// brev(P - klow) reversed; block 0 pairs with itself as q -> (F-q) mod F.
__device__ __forceinline__ int partner_block(int p, int P, int nb) {
    const int kl = brev_bits(p, nb);
    return kl == 0 ? 0 : brev_bits(P - kl, nb);
}

// ------------------------------------------------------------- scalar math
// tanh(y) = 1 - 2 / (1 + e^{2y}) with the hardware exp2 and reciprocal
// (absolute error a few 1e-7; exact limits +-1 for large |y|).
__device__ __forceinline__ float tanh_fast(float y) {
    const float e = __builtin_amdgcn_exp2f(y * 2.8853900817779268f);  // 2*log2(e)
    return __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
}

// fp32 -> nearest bf16 value (ties to even), kept in an fp32 register.
__device__ __forceinline__ float round_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return __uint_as_float(u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    uint32_t u = __float_as_uint(v);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Wavefront shift by one lane towards higher lanes; lane 0 receives 0.
__device__ __forceinline__ float wave_shr1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
}

__device__ __forceinline__ float readlane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

}  // namespace fi
