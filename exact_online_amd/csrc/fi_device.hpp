// fi_device.hpp -- device building blocks for the gfx950 kernels: complex
// arithmetic, small in-register DFTs, wave-level in-place FFT stages in LDS
// and radix-2 passes over a global scratch buffer.
//
// Citations name the page "Flash Inference: Inferenza in Tempo Quasi-Lineare
// per Modelli di Sequenza a Convoluzione Lunga e Oltre" (lowest.today summary
// of arXiv 2410.12982), written [FI].  The FFT is the tool of [FI] "Definizione
// di Aggregazione di Contribuzione" (Lemma 1: an FFT evaluates a tile's
// contribution in O(n log n)); the algorithms are the textbook in-place
// Cooley-Tukey ones: decimation in frequency for the forward transform
// (natural order in, bit-reversed order out) and decimation in time for the
// inverse (bit-reversed in, natural out), so a convolution never permutes.
//
// Every routine here is executed by one team: the kTeam threads (kTeam / 64
// wavefronts) of a workgroup, which own the buffers they touch.  Pointers
// carry their address space (global or LDS) so loads and stores compile to
// global_* and ds_* instructions rather than flat ones.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_internal.h"

#define FI_GLOBAL __attribute__((address_space(1)))
#define FI_SHARED __attribute__((address_space(3)))

namespace fi {

constexpr int kWave = 64;
// Threads of the team that runs one channel's FFT tiles: two wavefronts, so
// that each SIMD has a second wave to issue from while one waits on LDS or
// global memory.
constexpr int kTeamWaves = 2;
constexpr int kTeam = kTeamWaves * kWave;

template <typename T>
__device__ __forceinline__ FI_GLOBAL T* gmem(T* p) { return (FI_GLOBAL T*)p; }
template <typename T>
__device__ __forceinline__ const FI_GLOBAL T* gmem(const T* p) { return (const FI_GLOBAL T*)p; }
template <typename T>
__device__ __forceinline__ FI_SHARED T* smem_ptr(T* p) { return (FI_SHARED T*)p; }

// ------------------------------------------------------------------ complex
// A complex number as a two-lane clang vector (x = real, y = imaginary); the
// vector type can be loaded and stored through pointers of any address space.
template <typename R>
using Cx = R __attribute__((ext_vector_type(2)));
using V2 = float __attribute__((ext_vector_type(2)));
using V4 = float __attribute__((ext_vector_type(4)));

template <typename R>
__device__ __forceinline__ Cx<R> cadd(Cx<R> a, Cx<R> b) { return {a.x + b.x, a.y + b.y}; }
template <typename R>
__device__ __forceinline__ Cx<R> csub(Cx<R> a, Cx<R> b) { return {a.x - b.x, a.y - b.y}; }
template <typename R>
__device__ __forceinline__ Cx<R> cmul(Cx<R> a, Cx<R> b) {
    return {a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x};
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
template <typename R>
using TwPtr = const FI_GLOBAL Cx<R>*;

template <bool INV, typename R>
__device__ __forceinline__ Cx<R> twiddle(TwPtr<R> tw, int S, int m) {
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

// ------------------------------------------------------------ wave sync
// Workgroups are one wavefront wide.  A wavefront's LDS and global memory
// operations are performed in program order and see each other across lanes,
// so ordering between lanes only needs the compiler kept from moving memory
// operations across this point.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The thread's index in its team, recomputed where it is used: the empty asm
// keeps the compiler from hoisting lane-dependent indices and addresses of the
// many inlined FFT stages out of every loop (they would then all stay live,
// or be spilled, for the whole kernel).
__device__ __forceinline__ int team_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Team barriers.  team_sync orders LDS only (it waits for the team's own LDS
// operations, not for global loads in flight); team_sync_global also makes
// every global store before it visible to the whole team after it.
__device__ __forceinline__ void team_sync() {
    if constexpr (kTeam == kWave) {
        wave_sync();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
}
// The barrier of NT threads at the team's front: the whole team, or its first
// wavefront alone (whose LDS operations are ordered among themselves).
template <int NT>
__device__ __forceinline__ void group_sync() {
    if constexpr (NT == kWave) wave_sync();
    else team_sync();
}
__device__ __forceinline__ void team_sync_global() {
    if constexpr (kTeam == kWave) {
        wave_sync();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
}

// ------------------------------------------- in-place FFT stages in LDS
// LDS FFT buffers keep one spare slot per 8 points, which spreads the
// strided butterfly accesses over the banks.
__device__ __forceinline__ int lp(int p) { return p + (p >> 3); }

// Twiddle sources: powers(S, k, w) sets w[r] = exp(-2 pi i r k / S), r < R.
template <typename T>
struct GlobalTw {  // every power read from the global table tw[S + t]
    TwPtr<T> tw;
    template <int R>
    __device__ __forceinline__ void powers(int S, int k, Cx<T>* w) const {
#pragma unroll
        for (int r = 1; r < R; ++r) w[r] = tw[S + r * k];
    }
};
// One global lookup per butterfly, w_S^k; the other powers are products
// (depth <= 3, as the LDS table's).
template <typename T>
struct GlobalTwProd {
    TwPtr<T> tw;
    template <int R>
    __device__ __forceinline__ void powers(int S, int k, Cx<T>* w) const {
        w[1] = tw[S + k];
        if constexpr (R >= 4) {
            w[2] = cmul(w[1], w[1]);
            w[3] = cmul(w[2], w[1]);
        }
        if constexpr (R == 8) {
            w[4] = cmul(w[2], w[2]);
            w[5] = cmul(w[4], w[1]);
            w[6] = cmul(w[4], w[2]);
            w[7] = cmul(w[4], w[3]);
        }
    }
};
// Two-level LDS table for S <= 4096: with u = t * 4096 / S,
// exp(-2 pi i u / 4096) = A[u >> 6] * B[u & 63], A[a] = w_64^a, B[b] = w_4096^b.
// One lookup per butterfly; the other powers are products (depth <= 3).
struct LdsTw {
    const FI_SHARED Cx<float>* A;  // [64], B follows at A + 64
    template <int R>
    __device__ __forceinline__ void powers(int S, int k, Cx<float>* w) const {
        const int u = k * (kLdsFftMax / S);
        w[1] = cmul(A[u >> 6], A[64 + (u & 63)]);
        if constexpr (R >= 4) {
            w[2] = cmul(w[1], w[1]);
            w[3] = cmul(w[2], w[1]);
        }
        if constexpr (R == 8) {
            w[4] = cmul(w[2], w[2]);
            w[5] = cmul(w[4], w[1]);
            w[6] = cmul(w[4], w[2]);
            w[7] = cmul(w[4], w[3]);
        }
    }
};

// v_r *= w_S^{r k} for r = 1..R-1 (conjugated for the inverse).
template <int R, bool INV, typename T, typename Tw>
__device__ __forceinline__ void twiddle_apply(Cx<T>* v, const Tw& tw, int S, int k) {
    Cx<T> w[R];
    tw.template powers<R>(S, k, w);
#pragma unroll
    for (int r = 1; r < R; ++r) {
        if constexpr (INV) w[r].y = -w[r].y;
        v[r] = cmul(v[r], w[r]);
    }
}

// Radix of the stages of an M-point transform: 4 up to 512 points, where a
// stage has too few butterflies to fill a team and its latency is set by the
// work of one butterfly, else 8.
__host__ __device__ constexpr int ct_base(int M) { return M <= 512 ? 4 : 8; }
// Radix of the stage that splits a sub-problem of size S.
__host__ __device__ constexpr int ct_radix(int S, int M) { return S >= ct_base(M) ? ct_base(M) : S; }

// Size of the last (smallest) sub-problem stage of an M-point transform.
__host__ __device__ constexpr int ct_smallest(int M) {
    int S = M;
    while (S / ct_radix(S, M) > 1) S /= ct_radix(S, M);
    return S;
}

// Stage sources / sinks take a butterfly's first slot `off` and the distance
// `d` (a constant) of the slot wanted.  In the LDS buffer lp(off + d) =
// lp(off) + lp(d) for every slot a stage touches (off's low three bits stay
// below the butterfly stride when that stride is under 8), so only lp(off) is
// computed at run time.
template <typename T>
struct LdsIn {
    const FI_SHARED Cx<T>* b;
    __device__ __forceinline__ Cx<T> operator()(int off, int d) const { return (b + lp(off))[lp(d)]; }
};
template <typename T>
struct LdsOut {
    FI_SHARED Cx<T>* b;
    __device__ __forceinline__ void operator()(int off, int d, Cx<T> v) const { (b + lp(off))[lp(d)] = v; }
};

__host__ __device__ constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }

// Bit reversal of r over log2(R) bits, R in {2, 4, 8}.
template <int R>
__device__ __forceinline__ constexpr int rev_r(int r) {
    if constexpr (R == 8) return ((r & 1) << 2) | (r & 2) | ((r >> 2) & 1);
    else if constexpr (R == 4) return ((r & 1) << 1) | ((r >> 1) & 1);
    else return r;
}

// One in-place Cooley-Tukey stage on every sub-problem of size S of an
// M-point sequence (sub-problems contiguous), radix R = ct_radix(S, M), Q = S/R.
// Butterfly (base, j) owns the slots base + j + r*Q, r < R:
//   forward (decimation in frequency): v_r from slot r; u = DFT_R(v),
//     u_rho *= w_S^{j rho}, u_rho to slot rev(rho);
//   inverse (decimation in time): v_rho from slot rev(rho),
//     v_rho *= conj(w_S^{j rho}), u = IDFT_R(v), u_r to slot r.
// Storing each radix-R output in bit-reversed slot order makes the whole
// forward transform end in plain bit-reversed order.
// Each butterfly reads and writes the same slots, so no staging is needed;
// a thread processes its butterflies GRP at a time to overlap memory latency.
// The stage is run by the team's first NT threads (the whole team, or its
// first wavefront).
template <int M, int S, bool INV, typename T, int NT = kTeam, typename Src, typename Dst, typename Tw>
__device__ __forceinline__ void ct_stage(const Src& src, const Dst& dst, const Tw& tw) {
    constexpr int R = ct_radix(S, M);
    constexpr int Q = S / R;
    constexpr int NB = M / R;
    constexpr int PER = (NB + NT - 1) / NT;
    constexpr int GRP = PER < 2 ? PER : 2;
    const int lane = team_tid();
    // When Q divides NT, a thread's butterflies (n = lane + NT u) all
    // have j = lane mod Q: their twiddles are computed once.
    constexpr bool ONE_J = S > R && NT % Q == 0;
    Cx<T> wj[R];
    if constexpr (ONE_J) {
        tw.template powers<R>(S, lane % Q, wj);
#pragma unroll
        for (int r = 1; r < R; ++r)
            if constexpr (INV) wj[r].y = -wj[r].y;
    }
#pragma unroll 1
    for (int u0 = 0; u0 < PER; u0 += GRP) {
        Cx<T> v[GRP][R];
        int off[GRP], jj[GRP];
#pragma unroll
        for (int g = 0; g < GRP; ++g) {
            const int n = lane + NT * (u0 + g);
            jj[g] = n % Q;
            off[g] = (n / Q) * S + jj[g];
            if (NB % NT == 0 || n < NB) {
#pragma unroll
                for (int r = 0; r < R; ++r) v[g][r] = src(off[g], (INV ? rev_r<R>(r) : r) * Q);
            }
        }
#pragma unroll
        for (int g = 0; g < GRP; ++g) {
            const int n = lane + NT * (u0 + g);
            if (NB % NT == 0 || n < NB) {
                if constexpr (INV) {
                    if constexpr (ONE_J) {
#pragma unroll
                        for (int r = 1; r < R; ++r) v[g][r] = cmul(v[g][r], wj[r]);
                    } else if constexpr (S > R) {
                        twiddle_apply<R, true>(v[g], tw, S, jj[g]);
                    }
                    dft<R, true>(v[g]);
                } else {
                    dft<R, false>(v[g]);
                    if constexpr (ONE_J) {
#pragma unroll
                        for (int r = 1; r < R; ++r) v[g][r] = cmul(v[g][r], wj[r]);
                    } else if constexpr (S > R) {
                        twiddle_apply<R, false>(v[g], tw, S, jj[g]);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) dst(off[g], (INV ? r : rev_r<R>(r)) * Q, v[g][r]);
            }
        }
    }
    group_sync<NT>();
}

// Forward M-point FFT (unnormalised), natural order in, bit-reversed order
// out (position brev(k) holds frequency k): the first stage reads src,
// the others work in place on the LDS buffer.
template <int M, int S, typename T, int NT = kTeam, typename Src, typename Tw>
__device__ __forceinline__ void dif_lds(const Src& src, FI_SHARED Cx<T>* lds, const Tw& tw) {
    if constexpr (S > 1) {
        if constexpr (S == M) ct_stage<M, S, false, T, NT>(src, LdsOut<T>{lds}, tw);
        else ct_stage<M, S, false, T, NT>(LdsIn<T>{lds}, LdsOut<T>{lds}, tw);
        dif_lds<M, S / ct_radix(S, M), T, NT>(src, lds, tw);
    }
}

// The forward stages of dif_lds but the last (the smallest sub-problem
// size ct_smallest(M) is left to the caller).
template <int M, int S, typename T, typename Src, typename Tw>
__device__ __forceinline__ void dif_lds_head(const Src& src, FI_SHARED Cx<T>* lds, const Tw& tw) {
    if constexpr (S > ct_smallest(M)) {
        if constexpr (S == M) ct_stage<M, S, false, T>(src, LdsOut<T>{lds}, tw);
        else ct_stage<M, S, false, T>(LdsIn<T>{lds}, LdsOut<T>{lds}, tw);
        dif_lds_head<M, S / ct_radix(S, M), T>(src, lds, tw);
    }
}

// Inverse of dif_lds (unnormalised, times M): bit-reversed order in, natural
// order out, in place on the LDS buffer.  Every stage but the smallest has
// radix ct_base(M), so the sizes run ct_smallest(M), ct_base(M) times that,
// ..., M.
template <int M, int S, typename T, int NT = kTeam, typename Tw>
__device__ __forceinline__ void dit_lds(FI_SHARED Cx<T>* lds, const Tw& tw) {
    if constexpr (S <= M) {
        ct_stage<M, S, true, T, NT>(LdsIn<T>{lds}, LdsOut<T>{lds}, tw);
        if constexpr (S < M) dit_lds<M, S * ct_base(M), T, NT>(lds, tw);
    }
}

// Runtime-size dispatch (64 <= M <= kLdsFftMax), in place on the LDS buffer.
template <typename T, typename Tw>
__device__ __noinline__ void dif_lds_any(int M, FI_SHARED Cx<T>* lds, const Tw& tw) {
    const LdsIn<T> in{lds};
    switch (M) {
        case 64: dif_lds<64, 64, T>(in, lds, tw); break;
        case 128: dif_lds<128, 128, T>(in, lds, tw); break;
        case 256: dif_lds<256, 256, T>(in, lds, tw); break;
        case 512: dif_lds<512, 512, T>(in, lds, tw); break;
        case 1024: dif_lds<1024, 1024, T>(in, lds, tw); break;
        case 2048: dif_lds<2048, 2048, T>(in, lds, tw); break;
        case 4096: dif_lds<4096, 4096, T>(in, lds, tw); break;
        default: break;
    }
}
template <typename T, typename Tw>
__device__ __noinline__ void dit_lds_any(int M, FI_SHARED Cx<T>* lds, const Tw& tw) {
    switch (M) {
        case 64: dit_lds<64, ct_smallest(64), T>(lds, tw); break;
        case 128: dit_lds<128, ct_smallest(128), T>(lds, tw); break;
        case 256: dit_lds<256, ct_smallest(256), T>(lds, tw); break;
        case 512: dit_lds<512, ct_smallest(512), T>(lds, tw); break;
        case 1024: dit_lds<1024, ct_smallest(1024), T>(lds, tw); break;
        case 2048: dit_lds<2048, ct_smallest(2048), T>(lds, tw); break;
        case 4096: dit_lds<4096, ct_smallest(4096), T>(lds, tw); break;
        default: break;
    }
}
// ---------------------------------------------- passes over global scratch
// Radix-2 decimation in frequency on every sub-problem of size S of sc[0..M):
// (v0, v1) = (sc[b+j], sc[b+j+S/2]) -> (v0+v1, (v0-v1) w_S^j).  After the
// passes down to size F, the block of F points at p*F holds the transform of
// the frequencies k = brev(p) + (M/F)*kq (bit reversal over log2(M/F) bits);
// after the F-point transforms of the blocks, position q of every frequency k
// is brev(k) over log2(M) bits.
// Global-memory loops handle kBatch iterations per lane at a time, all loads
// of a batch issued before its first store, so one memory latency covers the
// batch.  Iterations of a batch touch disjoint elements.
constexpr int kBatch = 8;

template <typename T>
__device__ __forceinline__ void dif_pass(FI_GLOBAL Cx<T>* sc, int M, int S, TwPtr<T> tw) {
    const int lane = team_tid();
    const int half = S >> 1, nbf = M >> 1;
#pragma unroll 1
    for (int n0 = 0; n0 < nbf; n0 += kTeam * kBatch) {
        Cx<T> v0[kBatch], v1[kBatch], w[kBatch];
        int o[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int n = n0 + lane + kTeam * u;
            const int b = (n / half) * S, j = n % half;
            o[u] = b + j;
            if (n < nbf) {
                v0[u] = sc[o[u]];
                v1[u] = sc[o[u] + half];
                w[u] = tw[S + j];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (n0 + lane + kTeam * u < nbf) {
                sc[o[u]] = cadd(v0[u], v1[u]);
                sc[o[u] + half] = cmul(csub(v0[u], v1[u]), w[u]);
            }
        }
    }
    team_sync_global();
}

// Inverse of dif_pass (unnormalised): (v0, v1 w_S^-j) -> (v0+., v0-.).
template <typename T>
__device__ __forceinline__ void dit_pass(FI_GLOBAL Cx<T>* sc, int M, int S, TwPtr<T> tw) {
    const int lane = team_tid();
    const int half = S >> 1, nbf = M >> 1;
#pragma unroll 1
    for (int n0 = 0; n0 < nbf; n0 += kTeam * kBatch) {
        Cx<T> v0[kBatch], v1[kBatch], w[kBatch];
        int o[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int n = n0 + lane + kTeam * u;
            const int b = (n / half) * S, j = n % half;
            o[u] = b + j;
            if (n < nbf) {
                v0[u] = sc[o[u]];
                v1[u] = sc[o[u] + half];
                w[u] = tw[S + j];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (n0 + lane + kTeam * u < nbf) {
                const Cx<T> t = cmul(v1[u], cconj(w[u]));
                sc[o[u]] = cadd(v0[u], t);
                sc[o[u] + half] = csub(v0[u], t);
            }
        }
    }
    team_sync_global();
}

// One radix-R stage (R = 2, 4, 8) of span S over an M-point sequence held in
// global memory, the in-place Cooley-Tukey stage of ct_stage with run-time
// sizes: forward (decimation in frequency) stores radix outputs in
// bit-reversed slot order, the inverse (decimation in time) reads them so;
// twiddles from one global table load per butterfly and its products.  G butterflies per thread are in flight;
// M / R is a multiple of kTeam * G, so no load carries a condition (a load
// under a branch waits for every load issued before it).
template <int R, bool INV, typename T>
__device__ __forceinline__ void global_stage(FI_GLOBAL Cx<T>* sc, int M, int S, TwPtr<T> tw) {
    constexpr int G = 16 / R;
    const int lane = team_tid();
    const int Q = S / R, NB = M / R;
    const GlobalTwProd<T> gt{tw};   // one table load per butterfly
#pragma unroll 1
    for (int n0 = 0; n0 < NB; n0 += kTeam * G) {
        Cx<T> v[G][R];
        int off[G], jj[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int n = n0 + lane + kTeam * g;
            jj[g] = n % Q;
            off[g] = (n / Q) * S + jj[g];
#pragma unroll
            for (int r = 0; r < R; ++r) v[g][r] = sc[off[g] + (INV ? rev_r<R>(r) : r) * Q];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if constexpr (INV) {
                twiddle_apply<R, true>(v[g], gt, S, jj[g]);
                dft<R, true>(v[g]);
            } else {
                dft<R, false>(v[g]);
                twiddle_apply<R, false>(v[g], gt, S, jj[g]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) sc[off[g] + (INV ? r : rev_r<R>(r)) * Q] = v[g][r];
        }
    }
    team_sync_global();
}

// Forward stages of spans S0, S0/R, ... down to (not including) F, radix 8
// while it fits; inverse stages of spans F R, ..., up to S0 (the same
// sequence of sub-problem sizes, reversed).
template <typename T>
__device__ __forceinline__ void global_dif(FI_GLOBAL Cx<T>* sc, int M, int S0, int F, TwPtr<T> tw) {
    for (int S = S0; S > F;) {
        const int q = S / F;
        if (q >= 8) { global_stage<8, false>(sc, M, S, tw); S /= 8; }
        else if (q == 4) { global_stage<4, false>(sc, M, S, tw); S /= 4; }
        else { global_stage<2, false>(sc, M, S, tw); S /= 2; }
    }
}
template <typename T>
__device__ __forceinline__ void global_dit(FI_GLOBAL Cx<T>* sc, int M, int S0, int F, TwPtr<T> tw) {
    // the forward sequence's spans, walked back: radix 8 from the top, the
    // remainder (4 or 2) last in the forward order, so first here
    int q = S0 / F, r0 = 1;
    while (q >= 8) q /= 8;
    r0 = q;   // 1, 2 or 4
    int S = F;
    if (r0 == 4) { S *= 4; global_stage<4, true>(sc, M, S, tw); }
    else if (r0 == 2) { S *= 2; global_stage<2, true>(sc, M, S, tw); }
    while (S < S0) { S *= 8; global_stage<8, true>(sc, M, S, tw); }
}

// Copies n elements (a multiple of kTeam * 2 kBatch) between global and LDS
// (padded) buffers in batches of 2 kBatch per thread.  The loads carry no
// per-element condition: a load under a branch waits for every load issued
// before it.
template <typename T>
__device__ __forceinline__ void copy_to_lds(FI_SHARED Cx<T>* lds, const FI_GLOBAL Cx<T>* g, int n) {
    constexpr int B = 2 * kBatch;
    const int lane = team_tid();
#pragma unroll 1
    for (int q0 = 0; q0 < n; q0 += kTeam * B) {
        Cx<T> v[B];
#pragma unroll
        for (int u = 0; u < B; ++u) v[u] = g[q0 + lane + kTeam * u];
#pragma unroll
        for (int u = 0; u < B; ++u) lds[lp(q0 + lane + kTeam * u)] = v[u];
    }
    team_sync();
}
template <typename T>
__device__ __forceinline__ void copy_from_lds(FI_GLOBAL Cx<T>* g, const FI_SHARED Cx<T>* lds, int n) {
#pragma unroll 4
    for (int q = team_tid(); q < n; q += kTeam) g[q] = lds[lp(q)];
    team_sync_global();
}

__device__ __forceinline__ int brev_bits(int v, int nb) {
    return nb == 0 ? 0 : (int)(__brev((unsigned)v) >> (32 - nb));
}

// Frequency pairs (k, M-k) in bit-reversed position order: position p holds
// k = brev(p); its partner sits at the mirror of p within its octave,
// p' = 3*2^j - 1 - p for 2^j <= p < 2^(j+1), and p' = p for p < 2.
__device__ __forceinline__ int mirror_pos(int p) {
    if (p < 2) return p;
    const int j = 31 - __builtin_clz(p);
    return 3 * (1 << j) - 1 - p;
}
// The n-th position of a pair's first member, n in [0, M/2]: 0, 1, then the
// lower halves [2^j, 2^j + 2^(j-1)) of the octaves j >= 1, in order.
__device__ __forceinline__ int pair_first(int n) {
    if (n < 2) return n;
    const int m = n - 1;
    const int j = 32 - __builtin_clz(m);  // bit length of m
    return (1 << j) + (m - (1 << (j - 1)));
}

// ------------------------------------------------------------- scalar math
// tanh(y) = 1 - 2 / (1 + e^{2y}) with the hardware exp2 and reciprocal
// (absolute error a few 1e-7; exact limits +-1 for large |y|).
__device__ __forceinline__ float tanh_fast(float y) {
    const float e = __builtin_amdgcn_exp2f(y * 2.8853900817779268f);  // 2*log2(e)
    return __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
}

// The same with the argument already multiplied by 2*log2(e):
// r = 1 / (1 + 2^a); tanh = 1 - 2r.
__device__ __forceinline__ float tanh_rcp_scaled(float a) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a)); }
constexpr float kTanhScale = 2.8853900817779268f;  // 2*log2(e)

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

// Empty asm that takes v in a VGPR and gives it back: the computation of v
// stays ahead of this point (no instruction is emitted).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float readlane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

}  // namespace fi
