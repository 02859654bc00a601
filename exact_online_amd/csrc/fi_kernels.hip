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
//   k_step_tile; k_step, k_tile_fft         one online step (fi_step).
//   k_run                                   all L steps in one persistent pass
//       (open loop, closed loop, or a prompt then the closed loop): a team of
//       two wavefronts per channel; no grid-wide synchronisation is ever
//       needed because channels are independent ([FI] "Definizione
//       Specifica di LCSM": the mixer is a per-channel Hadamard convolution).
#include <mutex>
#include <type_traits>

#include "fi_device.hpp"
#include "fi_internal.h"

namespace fi {

// ------------------------------------------------------------------ io
template <bool BF16>
__device__ __forceinline__ float load_io(const void* p, int64_t idx) {
    if constexpr (BF16) return bf16_to_f32(gmem(static_cast<const uint16_t*>(p))[idx]);
    else return gmem(static_cast<const float*>(p))[idx];
}
template <bool BF16>
__device__ __forceinline__ void store_io(void* p, int64_t idx, float v) {
    if constexpr (BF16) gmem(static_cast<uint16_t*>(p))[idx] = f32_to_bf16_bits(v);
    else gmem(static_cast<float*>(p))[idx] = v;
}

__device__ __forceinline__ int ilog2(int64_t v) { return 63 - __builtin_clzll((unsigned long long)v); }

// ================================================================ fi_create
// h[L][D] -> hT[D][LS] (fp32), zero padding in [L, LS).  64x64 tiles via LDS.
template <bool BF16>
__global__ __launch_bounds__(256) void k_transpose(const void* h, float* hT, int64_t L, int64_t D, int64_t LS) {
    __shared__ float tile[64][65];
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    for (int64_t j0 = (int64_t)blockIdx.y * 64; j0 < LS; j0 += (int64_t)gridDim.y * 64) {
        for (int r = ty; r < 64; r += 4) {
            const int64_t j = j0 + r, c = c0 + tx;
            tile[r][tx] = (j < L && c < D) ? load_io<BF16>(h, j * D + c) : 0.f;
        }
        __syncthreads();
        for (int r = ty; r < 64; r += 4) {
            const int64_t c = c0 + r, j = j0 + tx;
            if (c < D && j < LS) hT[c * LS + j] = tile[tx][r];
        }
        __syncthreads();
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

// Filter spectra of level q (U = 2^q = M complex points).  The tile's filter
// segment g[n] = h[n] for 1 <= n < 2M (g[0] = 0: lag 0 never reaches the
// outputs [U, 2U) that are kept, [FI] "Trucco di Convoluzione Circolare") has
// the 2M-point DFT G; it is computed in fp64 from Z = DFT_M(g[2n] + i g[2n+1])
// as G[k] = (Z[k] + conj Z[M-k]) / 2 + w_2M^k (Z[k] - conj Z[M-k]) / (2i).
// Stored per channel, M + 2 entries G[k] / (4M) (the 1/(4M) folds the
// packing's halves and the inverse transform's 1/M): entry p < M holds
// frequency brev(p) (the tile's own bit-reversed position order), entry M
// holds G[M] (the partner of frequency 0), entry M + 1 is padding.
__global__ __launch_bounds__(kTeam) void k_spectra(const float* hT, int64_t LS, int64_t L, int64_t D, int M,
                                                V2* spec, Cx<double>* scd, int64_t scd_stride,
                                                const Cx<double>* twd_) {
    extern __shared__ __align__(16) unsigned char smem[];
    FI_SHARED Cx<double>* lbuf = smem_ptr(reinterpret_cast<Cx<double>*>(smem));
    TwPtr<double> twd = gmem(twd_);
    const GlobalTw<double> gtw{twd};
    const int lane = team_tid();
    const int F = M < kLdsFftMax ? M : kLdsFftMax;
    const int P = M / F, lm = ilog2(M);
    for (int64_t c = blockIdx.x; c < D; c += gridDim.x) {
        const FI_GLOBAL float* hr = gmem(hT + c * LS);
        auto g = [&](int64_t n) -> double { return (n >= 1 && n < L) ? (double)hr[n] : 0.0; };
        FI_GLOBAL Cx<double>* sc = gmem(scd + (int64_t)blockIdx.x * scd_stride);
        if (P == 1) {
            for (int n = lane; n < M; n += kTeam) lbuf[lp(n)] = Cx<double>{g(2 * n), g(2 * n + 1)};
            team_sync();
            dif_lds_any<double>(M, lbuf, gtw);
        } else {
            for (int n = lane; n < M; n += kTeam) sc[n] = Cx<double>{g(2 * n), g(2 * n + 1)};
            team_sync_global();
            for (int S = M; S > F; S >>= 1) dif_pass(sc, M, S, twd);
            for (int p = 0; p < P; ++p) {
                copy_to_lds(lbuf, sc + p * F, F);
                dif_lds_any<double>(F, lbuf, gtw);
                copy_from_lds(sc + p * F, lbuf, F);
            }
        }
        auto zat = [&](int p) -> Cx<double> { return P == 1 ? lbuf[lp(p)] : sc[p]; };
        FI_GLOBAL V2* out = gmem(spec + c * (int64_t)(M + 2));
        const double scale = 1.0 / (4.0 * (double)M);
        for (int p = lane; p < M; p += kTeam) {
            const int k = brev_bits(p, lm);
            const Cx<double> z1 = zat(p), z2c = cconj(zat(mirror_pos(p)));
            const Cx<double> ge = {(z1.x + z2c.x) * 0.5, (z1.y + z2c.y) * 0.5};
            const Cx<double> dz = {(z1.x - z2c.x) * 0.5, (z1.y - z2c.y) * 0.5};
            const Cx<double> go = {dz.y, -dz.x};   // dz / i
            const Cx<double> gk = cadd(ge, cmul(twd[2 * M + k], go));
            out[p] = V2{(float)(gk.x * scale), (float)(gk.y * scale)};
        }
        if (lane == 0) {
            const Cx<double> z0 = zat(0);
            out[M] = V2{(float)((z0.x - z0.y) * scale), 0.f};
            out[M + 1] = V2{0.f, 0.f};
        }
        team_sync_global();
    }
}

// Per channel c, the prefix sums of the closed-loop chain's scaled taps,
// pre[c][j] = sum_{l <= j} fl(s h[l][c]) for j < kRunBlock (s = 2 log2(e), the
// scale of the chain's accumulators; fl the fp32 rounding the chain's taps
// get), summed in fp64 and rounded once.  The chain that pushes r = (1 - x)/2
// instead of x adds these to its accumulators at the start of every block.
__global__ void k_prefix(const float* hT, int64_t LS, int64_t L, int64_t D, float* pre) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= D) return;
    const float* hr = hT + c * LS;
    double acc = 0.0;
    for (int j = 0; j < kRunBlock; ++j) {
        if (j < L) acc += (double)(kTanhScale * hr[j]);
        pre[c * kRunBlock + j] = (float)acc;
    }
}

__global__ void k_zero(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// ============================================================== FFT tile
// Where the outputs of the tile at i go: positions below `wend` into the LDS
// ring `accw` (slot = position & wmask; no ring when wend <= i -- an LDS
// pointer is never tested against null, since an object may sit at LDS
// address 0); the others into the channel's global row, added to what
// earlier tiles left there, or stored when `first` says no earlier tile
// reached them.
struct TileSink {
    FI_GLOBAL float* row;
    FI_SHARED float* accw;
    int64_t wend;
    int wmask;
    int64_t L;
    bool first;
};

// Adds w[m] = (a, b) to positions (i + 2m, i + 2m + 1) for m in [0, n):
// the first (wend - i) / 2 pairs into the LDS ring, the rest into the row
// (stored when the sink is its level's first, else added), kBatch
// thread-strided pairs at a time.  Every load of a batch is issued before
// any is used, from a clamped in-range index where the pair is out of range
// (a load under a branch would wait for the ones before it).  Run by the
// team's first NT threads.
template <int NT = kTeam, typename Get>
__device__ __forceinline__ void tile_output(const TileSink& s, int64_t i, int n, const Get& get) {
    const int lane = team_tid();
    int m0 = 0;
    if (s.wend > i) {
        const int nl = (int)((s.wend - i) / 2) < n ? (int)((s.wend - i) / 2) : n;
#pragma unroll 1
        for (int m = lane; m < nl; m += NT) {
            const int64_t o = i + 2 * (int64_t)m;
            if (o < s.L) {
                const Cx<float> w = get(m);
                s.accw[o & s.wmask] += w.x;
                if (o + 1 < s.L) s.accw[(o + 1) & s.wmask] += w.y;
            }
        }
        m0 = nl;
    }
#pragma unroll 1
    for (; m0 < n; m0 += NT * kBatch) {
        V2 v[kBatch];
        Cx<float> w[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int m = m0 + lane + NT * u;
            const int64_t o = i + 2 * (int64_t)m;
            w[u] = get(m < n ? m : n - 1);
            if (!s.first) v[u] = *reinterpret_cast<const FI_GLOBAL V2*>(s.row + (m < n && o + 1 < s.L ? o : 0));
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int m = m0 + lane + NT * u;
            const int64_t o = i + 2 * (int64_t)m;
            const V2 r = s.first ? V2{w[u].x, w[u].y} : V2{v[u].x + w[u].x, v[u].y + w[u].y};
            if (m < n && o + 1 < s.L) {
                *reinterpret_cast<FI_GLOBAL V2*>(s.row + o) = r;
            } else if (m < n && o < s.L) {
                s.row[o] = s.first ? w[u].x : s.row[o] + w[u].x;
            }
        }
    }
}

// The row values that tile_output adds to, loaded ahead of the inverse
// transform: for a sink whose ring takes the first kRunBlock positions, NP
// per thread, the pairs m = kRunBlock/2 + tid + kTeam u (the order of
// tile_output_ahead).  The last position of an odd L is left to a scalar
// read-modify-write.
template <int NP>
struct RowAhead {
    V2 v[NP];
    __device__ __forceinline__ void load(const TileSink& s, int64_t i, int n) {
        const int lane = team_tid();
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int m = kRunBlock / 2 + lane + kTeam * u;
            const int64_t o = i + 2 * (int64_t)m;
            // unconditional (a load under a branch would wait for the ones
            // before it): out-of-range pairs read position 0 and are unused
            v[u] = *reinterpret_cast<const FI_GLOBAL V2*>(s.row + (m < n && o + 1 < s.L ? o : 0));
        }
    }
};

// tile_output for a sink that is not a level's first and whose ring takes
// the first kRunBlock positions, with the row values already loaded.
template <int NP, typename Get>
__device__ __forceinline__ void tile_output_ahead(const TileSink& s, int64_t i, int n, const Get& get,
                                                  const RowAhead<NP>& ra) {
    const int lane = team_tid();
    constexpr int nl = kRunBlock / 2;
#pragma unroll 1
    for (int m = lane; m < nl; m += kTeam) {
        const int64_t o = i + 2 * (int64_t)m;
        if (m < n && o < s.L) {
            const Cx<float> w = get(m);
            s.accw[o & s.wmask] += w.x;
            if (o + 1 < s.L) s.accw[(o + 1) & s.wmask] += w.y;
        }
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int m = nl + lane + kTeam * u;
        const int64_t o = i + 2 * (int64_t)m;
        if (m < n && o + 1 < s.L) {
            const Cx<float> w = get(m);
            *reinterpret_cast<FI_GLOBAL V2*>(s.row + o) = V2{ra.v[u].x + w.x, ra.v[u].y + w.y};
        } else if (m < n && o < s.L) {
            s.row[o] += get(m).x;
        }
    }
}

// Output spectrum of a partner pair of frequencies (k, M-k) whose packed
// input transform values (z[n] = x[2n] + i x[2n+1]) are A = Z_k, B = Z_{M-k},
// with the filter entries gk = G[k] / (4M), gm = G[M-k] / (4M), w = w_2M^k:
//   P = A + conj B,  Q = -i w (A - conj B)
//   (2 X[k], 2 X[k+M]) = (P + Q, P - Q)             (real 2M-point spectrum)
//   Ya = gk (P + Q),  Yb = conj(gm) (P - Q)         (G[k+M] = conj G[M-k])
//   S = Ya + Yb,  E = i conj(w) (Ya - Yb)
//   W_k = S + E,  W_{M-k} = conj(S - E)             (the packed output spectrum)
// For the self-paired k = 0 (gm = G[M]) and k = M/2 both results agree.
__device__ __forceinline__ void untangle_pair(Cx<float>& A, Cx<float>& B, Cx<float> gk, Cx<float> gm, Cx<float> w) {
    const Cx<float> Bc = cconj(B);
    const Cx<float> wm = {w.y, -w.x};   // -i w
    const Cx<float> Pp = cadd(A, Bc);
    const Cx<float> Qq = cmul(wm, csub(A, Bc));
    const Cx<float> Ya = cmul(gk, cadd(Pp, Qq));
    const Cx<float> Yb = cmul(cconj(gm), csub(Pp, Qq));
    const Cx<float> Ss = cadd(Ya, Yb);
    const Cx<float> Ee = cmul(cconj(wm), csub(Ya, Yb));
    A = cadd(Ss, Ee);
    B = cconj(csub(Ss, Ee));
}
// Forward-FFT input of the tile: z[n] = x[2n] + i x[2n+1] for n < HALF,
// zero beyond (the input block padded on the right).  d is a constant once
// the stage is unrolled, so a slot that is padding in every butterfly is a
// constant zero.
template <int HALF>
struct TileIn {
    const FI_GLOBAL V2* xs;
    __device__ __forceinline__ Cx<float> operator()(int off, int d) const {
        if (d >= HALF) return {0.f, 0.f};
        const int n = off + d;
        if (n < HALF) {
            const V2 v = xs[n];
            return {v.x, v.y};
        }
        return {0.f, 0.f};
    }
};


// Twiddles w_N^k for the untangle: from the LDS table (A[64] = w_64^a,
// B[64] = w_4096^b, C[4] = w_16384^r) for N <= 16384, else from the global
// table.
struct TwLdsN {
    const FI_SHARED Cx<float>* t;
    int N;
    __device__ __forceinline__ Cx<float> operator()(int k) const {
        if (N <= kLdsFftMax) {
            const int j = k * (kLdsFftMax / N);
            return cmul(t[j >> 6], t[64 + (j & 63)]);
        }
        const int s = N / kLdsFftMax;   // 2 or 4
        const int j = k / s, r = k % s;
        const Cx<float> w = cmul(t[j >> 6], t[64 + (j & 63)]);
        return r ? cmul(w, t[128 + r * (4 / s)]) : w;
    }
};
// w_{2 kLdsFftMax}^k from the same table with no branch (C[0] = 1, and a
// product with it is exact), so the table reads of neighbouring calls are not
// serialised behind one another.
__device__ __forceinline__ Cx<float> tw_lds_2f(const FI_SHARED Cx<float>* t, int k) {
    const int j = k >> 1;
    return cmul(cmul(t[j >> 6], t[64 + (j & 63)]), t[128 + 2 * (k & 1)]);
}
struct TwGlobalN {
    TwPtr<float> tw;
    int N;
    __device__ __forceinline__ Cx<float> operator()(int k) const { return twiddle<false>(tw, N, k); }
};

constexpr int kUntangleBatch = 4;   // pairs per thread per untangle batch

// Filter entries of one batch of NB pairs per thread (pairs n0 + tid + NT u).
template <int NB, int NT = kTeam>
struct SpecBatch {
    V2 ga[NB], gb[NB];
    template <typename SpecP, typename Pos>
    __device__ __forceinline__ void load(SpecP spec, int n0, int nitems, const Pos& pos) {
        const int lane = team_tid();
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int n = n0 + lane + NT * u;
            int a, b;
            pos(n < nitems ? n : 0, a, b);   // item 0 stands in past the end (unused)
            ga[u] = spec[a];
            gb[u] = spec[b];
        }
    }
};

// Untangle nitems partner pairs held in the LDS buffer: pos(n) gives the
// (buffer-relative) slots of pair n, spec[slot] their filter entries, and the
// frequency of slot a is brev(pos_off + a) over lbits bits; gM is G[M] / (4M),
// the partner entry of frequency 0.  `cur` holds the first batch's filter
// entries, loaded by the caller (ahead of the forward transform); each later
// batch is loaded while the one before it is processed.  Run by the team's
// first NT threads.
template <int NB, int NT = kTeam, typename SpecP, typename Pos, typename TwF>
__device__ __forceinline__ void untangle_lds(FI_SHARED Cx<float>* lds, SpecP spec, V2 gM, int nitems,
                                             const Pos& pos, int pos_off, int lbits, const TwF& twf,
                                             SpecBatch<NB, NT> cur) {
    const int lane = team_tid();
#pragma unroll 1
    for (int n0 = 0; n0 < nitems; n0 += NT * NB) {
        SpecBatch<NB, NT> nxt;
        if (n0 + NT * NB < nitems) nxt.load(spec, n0 + NT * NB, nitems, pos);
        // the pairs of a batch are disjoint: all reads first, then all writes
        Cx<float> za[NB], zb[NB], w[NB];
        int pa[NB], pb[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int n = n0 + lane + NT * u;
            pos(n < nitems ? n : 0, pa[u], pb[u]);
            za[u] = lds[lp(pa[u])];
            zb[u] = lds[lp(pb[u])];
            w[u] = twf(brev_bits(pos_off + pa[u], lbits));
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const bool first = brev_bits(pos_off + pa[u], lbits) == 0;
            const V2 gm = first ? gM : cur.gb[u];
            untangle_pair(za[u], zb[u], Cx<float>{cur.ga[u].x, cur.ga[u].y}, Cx<float>{gm.x, gm.y}, w[u]);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (n0 + lane + NT * u < nitems) {
                lds[lp(pa[u])] = za[u];
                lds[lp(pb[u])] = zb[u];
            }
        }
        cur = nxt;
    }
    group_sync<NT>();
}

// ---------------------------------------------------------------- middle
// The middle of a tile's transform pair in one LDS pass: the forward
// transform's last stage, the untangle of every partner pair and the inverse
// transform's first stage.  Both stages have radix R = ct_smallest(M) and no
// twiddles, and work on groups of R consecutive positions.  The partner of
// position gR + s is g'R + R-1-s with g' = mirror_pos(g) the mirror group
// (groups 0 and 1 hold their own partners), so one thread takes a group and
// its mirror group through all three steps in registers.
// Position gR + s holds frequency k = brev(gR + s) = kg + brev_R(s) M/R, kg the
// bit reversal of g over log2(M/R) bits, so w_2M^k = w_2M^kg w_2R^brev_R(s).
// Item n of the pass: n = 0 takes groups 0 and 1, n >= 1 the group
// pair_first(n + 1) and its mirror.
// ODD: the M points are the odd-frequency half of a 2M-point transform
// (position q holds frequency 1 + 2 brev(q)); partners are q and M-1-q, so
// item n takes groups n and M/R-1-n, and every twiddle carries a factor
// w_4M.
template <int R>
struct GroupSpec {
    V2 a[R], b[R];
    template <typename SpecP>
    __device__ __forceinline__ void load(SpecP spec, int ga, int gb) {
#pragma unroll
        for (int s = 0; s < R; ++s) {
            a[s] = spec[ga * R + s];
            b[s] = spec[gb * R + s];
        }
    }
};

template <bool ODD, int NG>
__device__ __forceinline__ void middle_groups(int n, int& ga, int& gb) {
    if constexpr (ODD) {
        ga = n;
        gb = NG - 1 - n;
    } else {
        ga = n == 0 ? 0 : pair_first(n + 1);
        gb = n == 0 ? 1 : mirror_pos(ga);
    }
}

// w_2R^e as a compile-time constant (forward sign).
template <int R>
__device__ __forceinline__ Cx<float> w2r(int e) {
    const double ang = -3.14159265358979323846 * (double)e / (double)R;
    return Cx<float>{(float)__builtin_cos(ang), (float)__builtin_sin(ang)};
}

// The tile input (x[2n] + i x[2n+1], n < N/2) times w_N^n, N = 2 kLdsFftMax:
// the second half of an N-point transform after one radix-2 pass.  In a
// stage the offset d of a butterfly's point is a constant, so w_N^(off+d) =
// w_N^off (LDS table, once per butterfly) times a folded constant.
struct TileInTw {
    const FI_GLOBAL V2* xs;
    const FI_SHARED Cx<float>* twl;
    __device__ __forceinline__ Cx<float> operator()(int off, int d) const {
        const V2 v = xs[off + d];
        const Cx<float> w = cmul(TwLdsN{twl, 2 * kLdsFftMax}(off), w2r<kLdsFftMax>(d));
        return cmul(Cx<float>{v.x, v.y}, w);
    }
};

template <int M, bool ODD, typename SpecP>
__device__ __forceinline__ void middle_lds(FI_SHARED Cx<float>* lds, SpecP spec, V2 gM, const LdsTw& tw,
                                           GroupSpec<ct_smallest(M)> cur) {
    constexpr int R = ct_smallest(M);
    constexpr int NG = M / R;
    constexpr int NI = M / R / 2;             // items
    constexpr int GB = ilog2c(M / R);         // bits of a group index
    const int tid = team_tid();
    const TwLdsN twn{tw.A, 2 * M};
#pragma unroll 1
    for (int n = tid; n < NI; n += kTeam) {
        GroupSpec<R> nxt;
        if (n + kTeam < NI) {
            int na, nb;
            middle_groups<ODD, NG>(n + kTeam, na, nb);
            nxt.load(spec, na, nb);
        }
        int ga, gb;
        middle_groups<ODD, NG>(n, ga, gb);
        Cx<float> a[R], b[R];
#pragma unroll
        for (int s = 0; s < R; ++s) {
            a[s] = lds[lp(ga * R + s)];
            b[s] = lds[lp(gb * R + s)];
        }
        // last forward stage: afterwards position gR + s holds a[rev(s)]
        dft<R, false>(a);
        dft<R, false>(b);
        if (!ODD && n == 0) {
            // group 0: positions 0 (k = 0, partner G[M]) and 1 (k = M/2) pair
            // with themselves, the others p with mirror_pos(p); group 1 (the
            // octave of R): R + s with 2R - 1 - s.  All twiddles are constants.
#pragma unroll
            for (int s = 0; s < R; ++s) {
                const int s2 = s < 2 ? s : 3 * (1 << ilog2c(s)) - 1 - s;
                if (s2 < s) continue;
                Cx<float>& A = a[rev_r<R>(s)];
                Cx<float>& B = a[rev_r<R>(s2)];
                const V2 gm = s == 0 ? gM : cur.a[s2];
                if (s2 == s) {
                    Cx<float> t = A;
                    untangle_pair(A, t, Cx<float>{cur.a[s].x, cur.a[s].y}, Cx<float>{gm.x, gm.y},
                                  w2r<R>(rev_r<R>(s)));
                } else {
                    untangle_pair(A, B, Cx<float>{cur.a[s].x, cur.a[s].y}, Cx<float>{gm.x, gm.y},
                                  w2r<R>(rev_r<R>(s)));
                }
            }
            // group 1: k = M/(2R) + brev_R(s) M/R, w_2M^k = w_4R w_2R^brev_R(s)
#pragma unroll
            for (int s = 0; s < R / 2; ++s) {
                const int s2 = R - 1 - s;
                const Cx<float> w = cmul(w2r<2 * R>(1), w2r<R>(rev_r<R>(s)));
                untangle_pair(b[rev_r<R>(s)], b[rev_r<R>(s2)], Cx<float>{cur.b[s].x, cur.b[s].y},
                              Cx<float>{cur.b[s2].x, cur.b[s2].y}, w);
            }
        } else {
            Cx<float> wg = twn(brev_bits(ga, GB));
            if constexpr (ODD) wg = cmul(wg, w2r<2 * M>(1));
#pragma unroll
            for (int s = 0; s < R; ++s) {
                const int s2 = R - 1 - s;
                const Cx<float> w = s == 0 ? wg : cmul(wg, w2r<R>(rev_r<R>(s)));
                untangle_pair(a[rev_r<R>(s)], b[rev_r<R>(s2)], Cx<float>{cur.a[s].x, cur.a[s].y},
                              Cx<float>{cur.b[s2].x, cur.b[s2].y}, w);
            }
        }
        // first inverse stage: it reads position gR + rev(rho) = a[rho]
        dft<R, true>(a);
        dft<R, true>(b);
#pragma unroll
        for (int s = 0; s < R; ++s) {
            lds[lp(ga * R + s)] = a[s];
            lds[lp(gb * R + s)] = b[s];
        }
        cur = nxt;
    }
    team_sync();
}

// pairs of a whole bit-reversed transform (or of a block holding its octaves)
struct PairsAll {
    __device__ __forceinline__ void operator()(int n, int& a, int& b) const {
        a = pair_first(n);
        b = mirror_pos(a);
    }
};
// pairs (q, F-1-q) of one octave-block of size F
struct PairsMirror {
    int F;
    __device__ __forceinline__ void operator()(int n, int& a, int& b) const {
        a = n;
        b = F - 1 - n;
    }
};

// The same input staged in LDS.
template <int HALF>
struct TileInLds {
    const FI_SHARED V2* xs;
    __device__ __forceinline__ Cx<float> operator()(int off, int d) const {
        if (d >= HALF) return {0.f, 0.f};
        const int n = off + d;
        if (n < HALF) {
            const V2 v = xs[n];
            return {v.x, v.y};
        }
        return {0.f, 0.f};
    }
};

template <int M, typename XIn, typename SpecP>
__device__ __forceinline__ void fft_tile_lds(int64_t i, const XIn& xin, SpecP spec, FI_SHARED Cx<float>* lds,
                                             const LdsTw& tw, const TileSink& out) {
    // spectrum entries staged in LDS are read after the forward transform;
    // from global memory, the first batch is in flight during it
    constexpr bool staged = std::is_same<SpecP, const FI_SHARED V2*>::value;
    constexpr int R = ct_smallest(M);
    const V2 gM = spec[M];
    if constexpr (M / R / 2 >= kTeam) {
        // the fused middle pass (one LDS pass instead of three)
        GroupSpec<R> first;
        const int tid = team_tid();
        if constexpr (!staged) {
            int ga, gb;
            middle_groups<false, M / R>(tid, ga, gb);
            first.load(spec, ga, gb);
        }
        dif_lds_head<M, M, float>(xin, lds, tw);
        if constexpr (staged) {
            int ga, gb;
            middle_groups<false, M / R>(tid, ga, gb);
            first.load(spec, ga, gb);
        }
        middle_lds<M, false>(lds, spec, gM, tw, first);
        // the row values the output adds to, in flight during the inverse
        // transform
        constexpr int NPA = (M / 2 - kRunBlock / 2 + kTeam - 1) / kTeam;
        RowAhead<NPA> ra;
        const bool ahead = !out.first && out.wend - i == kRunBlock;
        if (ahead) ra.load(out, i, M / 2);
        dit_lds<M, R * ct_base(M), float>(lds, tw);
        if (ahead) {
            tile_output_ahead(out, i, M / 2, [lds](int m) { return lds[lp(M / 2 + m)]; }, ra);
            return;
        }
    } else {
        // small transforms: too few groups to spread the fused pass over the
        // team, so the last and first stages stay separate from an untangle
        // pass over single pairs.  Up to 256 points a stage is at most one
        // butterfly per lane of one wavefront: the first wavefront runs the
        // whole tile alone, its LDS operations ordered among themselves, with
        // no team barrier between the stages (the others wait for it at the
        // caller's barrier).
        constexpr int NT = M <= 256 ? kWave : kTeam;
        if (NT == kTeam || __builtin_amdgcn_readfirstlane(team_tid()) < kWave) {
            constexpr int NALL = M / 2 / NT + 1;
            constexpr int NB = NALL < kUntangleBatch ? NALL : kUntangleBatch;
            SpecBatch<NB, NT> first;
            if constexpr (!staged) first.load(spec, 0, M / 2 + 1, PairsAll{});
            dif_lds<M, M, float, NT>(xin, lds, tw);
            if constexpr (staged) first.load(spec, 0, M / 2 + 1, PairsAll{});
            untangle_lds<NB, NT>(lds, spec, gM, M / 2 + 1, PairsAll{}, 0, ilog2(M), TwLdsN{tw.A, 2 * M}, first);
            dit_lds<M, R, float, NT>(lds, tw);
            // point M/2 + m carries outputs 2m, 2m + 1 of the tile
            tile_output<NT>(out, i, M / 2, [lds](int m) { return lds[lp(M / 2 + m)]; });
        }
        return;
    }
    tile_output(out, i, M / 2, [lds](int m) { return lds[lp(M / 2 + m)]; });
}

// The forward transform's first two stages of a tile of more than kLdsFftMax
// points (radix R1 at span M, then radix R2 at span M / R1; R2 = 1: none),
// fused with the load of its input: inputs r >= R1/2 of every first-stage
// butterfly are the zero padding (z[n] = 0 for n >= M/2).  Thread item j2 <
// Q2 = M / (R1 R2) runs the first-stage butterflies j2 + r2 Q2 (r2 < R2),
// which hold every input of the second-stage butterflies (b, j2), b < R1.
// Outputs go to the stages' bit-reversed slot order (as global_stage).
template <int R1, int R2>
__device__ __forceinline__ void first_pass_load(FI_GLOBAL Cx<float>* sc, const FI_GLOBAL V2* xs, int M,
                                                TwPtr<float> tw) {
    constexpr int G = R1 * R2 >= 16 ? 2 : 16 / (R1 * R2);
    const int lane = team_tid();
    const int Q1 = M / R1, Q2 = Q1 / R2;   // Q2 a multiple of kTeam * G
    const GlobalTwProd<float> gt{tw};   // one table load per butterfly
#pragma unroll 1
    for (int n0 = 0; n0 < Q2; n0 += kTeam * G) {
        Cx<float> v[G][R2][R1];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int j2 = n0 + lane + kTeam * g;
#pragma unroll
            for (int r2 = 0; r2 < R2; ++r2) {
#pragma unroll
                for (int r = 0; r < R1; ++r) {
                    if (r < R1 / 2) {
                        const V2 x = xs[j2 + r2 * Q2 + r * Q1];
                        v[g][r2][r] = Cx<float>{x.x, x.y};
                    } else {
                        v[g][r2][r] = Cx<float>{0.f, 0.f};
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int j2 = n0 + lane + kTeam * g;
#pragma unroll
            for (int r2 = 0; r2 < R2; ++r2) {
                dft<R1, false>(v[g][r2]);
                twiddle_apply<R1, false>(v[g][r2], gt, M, j2 + r2 * Q2);
            }
#pragma unroll
            for (int p = 0; p < R1; ++p) {   // first-stage output p: sub-problem rev(p)
                const int b = rev_r<R1>(p);
                if constexpr (R2 == 1) {
                    sc[b * Q1 + j2] = v[g][0][p];
                } else {
                    Cx<float> t[R2];
#pragma unroll
                    for (int r2 = 0; r2 < R2; ++r2) t[r2] = v[g][r2][p];
                    dft<R2, false>(t);
                    twiddle_apply<R2, false>(t, gt, Q1, j2);
#pragma unroll
                    for (int r2 = 0; r2 < R2; ++r2) sc[b * Q1 + j2 + rev_r<R2>(r2) * Q2] = t[r2];
                }
            }
        }
    }
    team_sync_global();
}

// The inverse transform's last two stages of such a tile (radix R2 at span
// M / R1, then radix R1 at span M), fused with the output.  First-stage
// butterfly j keeps its outputs r >= R1/2 only: complex points j + r Q1 =
// M/2 + m with m = j + (r - R1/2) Q1, the tile's outputs i + 2m and i + 2m + 1
// (the ring for m < (wend - i) / 2, else the row: stored when the sink is its
// level's first, else added).  Every load of a group is issued before any is
// used (the row values from clamped indices).
template <int R1, int R2>
__device__ __forceinline__ void last_pass_output(const TileSink& s, int64_t i, const FI_GLOBAL Cx<float>* sc,
                                                 int M, TwPtr<float> tw) {
    constexpr int G = R1 * R2 >= 16 ? 1 : 16 / (R1 * R2);
    constexpr int H = R1 / 2;
    const int lane = team_tid();
    const int Q1 = M / R1, Q2 = Q1 / R2;   // Q2 a multiple of kTeam * G
    const int nl = s.wend > i ? (int)((s.wend - i) / 2) : 0;
    const GlobalTwProd<float> gt{tw};   // one table load per butterfly
#pragma unroll 1
    for (int n0 = 0; n0 < Q2; n0 += kTeam * G) {
        Cx<float> a[G][R1][R2];
        V2 old[G][R2][H];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int j2 = n0 + lane + kTeam * g;
#pragma unroll
            for (int b = 0; b < R1; ++b) {
#pragma unroll
                for (int r2 = 0; r2 < R2; ++r2) a[g][b][r2] = sc[b * Q1 + j2 + rev_r<R2>(r2) * Q2];
            }
            if (!s.first) {
#pragma unroll
                for (int r2 = 0; r2 < R2; ++r2) {
#pragma unroll
                    for (int r = 0; r < H; ++r) {
                        const int m = j2 + r2 * Q2 + r * Q1;
                        const int64_t o = i + 2 * (int64_t)m;
                        old[g][r2][r] =
                            *reinterpret_cast<const FI_GLOBAL V2*>(s.row + (m >= nl && o + 1 < s.L ? o : 0));
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int j2 = n0 + lane + kTeam * g;
            Cx<float> v[R2][R1];
#pragma unroll
            for (int b = 0; b < R1; ++b) {   // sub-problem b feeds first-stage input rev(b)
                if constexpr (R2 > 1) {
                    twiddle_apply<R2, true>(a[g][b], gt, Q1, j2);
                    dft<R2, true>(a[g][b]);
                }
#pragma unroll
                for (int r2 = 0; r2 < R2; ++r2) v[r2][rev_r<R1>(b)] = a[g][b][r2];
            }
#pragma unroll
            for (int r2 = 0; r2 < R2; ++r2) {
                const int j = j2 + r2 * Q2;
                twiddle_apply<R1, true>(v[r2], gt, M, j);
                dft<R1, true>(v[r2]);
#pragma unroll
                for (int r = 0; r < H; ++r) {
                    const int m = j + r * Q1;
                    const int64_t o = i + 2 * (int64_t)m;
                    const Cx<float> w = v[r2][H + r];
                    if (m < nl) {
                        if (o < s.L) {
                            s.accw[o & s.wmask] += w.x;
                            if (o + 1 < s.L) s.accw[(o + 1) & s.wmask] += w.y;
                        }
                    } else if (o + 1 < s.L) {
                        *reinterpret_cast<FI_GLOBAL V2*>(s.row + o) =
                            s.first ? V2{w.x, w.y} : V2{old[g][r2][r].x + w.x, old[g][r2][r].y + w.y};
                    } else if (o < s.L) {
                        s.row[o] = s.first ? w.x : s.row[o] + w.x;
                    }
                }
            }
        }
    }
}

// Tiles of more than kLdsFftMax points (the tile of fft_tile below).  The
// caller synchronises the team afterwards.
__device__ __forceinline__ void fft_tile_big(int M, int64_t i, const FI_GLOBAL float* xblock, const FI_GLOBAL V2* spec,
                                          FI_SHARED Cx<float>* lbuf, FI_GLOBAL Cx<float>* sc, TwPtr<float> tw,
                                          const FI_SHARED Cx<float>* twl, FI_GLOBAL float* row, FI_SHARED float* accw,
                                          int64_t wend, int wmask, int64_t L, bool first) {
    const TileSink out{row, accw, wend, wmask, L, first};
    const LdsTw ltw{twl};
    if (M == 2 * kLdsFftMax) {
        // One radix-2 decimation-in-frequency pass splits the transform into
        // halves z[n] + z[n + M/2] and (z[n] - z[n + M/2]) w_M^n; the input's
        // upper half is the zero padding, so these are z[n] and z[n] w_M^n,
        // formed while loading.  Each half holds its own partner frequencies
        // (half 0: octaves 0 .. log2(F)-1, half 1: octave log2(F)), so each
        // is transformed, untangled and transformed back in LDS; half 0's
        // result waits in the scratch slot for the last inverse pass, fused
        // with the output (only outputs M/2 .. M-1 are kept).
        constexpr int F = kLdsFftMax;
        constexpr int R = ct_smallest(F);
        const FI_GLOBAL V2* xs = reinterpret_cast<const FI_GLOBAL V2*>(xblock);
        const V2 gM = spec[M];
        const int tid = team_tid();
        int ga, gb;
        // half 0: the even frequencies, a 4096-point tile of its own
        GroupSpec<R> g0;
        middle_groups<false, F / R>(tid, ga, gb);
        g0.load(spec, ga, gb);
        dif_lds_head<F, F, float>(TileIn<F>{xs}, lbuf, ltw);
        middle_lds<F, false>(lbuf, spec, gM, ltw, g0);
        dit_lds<F, R * ct_base(F), float>(lbuf, ltw);
        copy_from_lds(sc, lbuf, F);
        // half 1: the odd frequencies
        middle_groups<true, F / R>(tid, ga, gb);
        g0.load(spec + F, ga, gb);
        dif_lds_head<F, F, float>(TileInTw{xs, twl}, lbuf, ltw);
        middle_lds<F, true>(lbuf, spec + F, gM, ltw, g0);
        dit_lds<F, R * ct_base(F), float>(lbuf, ltw);
        tile_output(out, i, F, [sc, lbuf, twl](int j) {
            const Cx<float> v0 = sc[j];
            const Cx<float> v1 = cmul(lbuf[lp(j)], cconj(tw_lds_2f(twl, j)));
            return csub(v0, v1);
        });
        return;
    }
    // M > 8192: the first decimation-in-frequency stages (radix R1 =
    // min(M / F, 8), then R2) fused with the load, then radix-8 passes over
    // the scratch slot until F = 4096-point blocks remain; after the blocks'
    // own transforms,
    // position p (block p / F) holds frequency brev(p) over log2(M) bits.
    // Block 0 holds octaves 0 .. log2(F)-1 and block 1 octave log2(F): both
    // hold their own partner frequencies and are transformed, multiplied and
    // transformed back in one LDS visit.  Blocks b >= 2 pair with the mirror
    // block of their octave through the scratch slot.
    const int lane = team_tid();
    const FI_GLOBAL V2* xs = reinterpret_cast<const FI_GLOBAL V2*>(xblock);
    constexpr int F = kLdsFftMax;
    const int P = M / F;
    // R2 = 2 where M / (R1 F) is twice a power of 8, else 1 (a factor of 4
    // left over goes to a global stage: 32 values per thread would spill)
    const int R1 = P < 8 ? P : 8;
    int R2 = P / R1;
    while (R2 >= 8) R2 /= 8;
    if (R2 != 2) R2 = 1;
    if (R1 == 4) first_pass_load<4, 1>(sc, xs, M, tw);
    else if (R2 == 1) first_pass_load<8, 1>(sc, xs, M, tw);
    else first_pass_load<8, 2>(sc, xs, M, tw);
    global_dif(sc, M, M / (R1 * R2), F, tw);   // radix-8 (4) stages down to F-point blocks
    for (int p = 0; p < 2; ++p) {
        FI_GLOBAL Cx<float>* blk = sc + (int64_t)p * F;
        copy_to_lds(lbuf, blk, F);
        dif_lds<F, F, float>(LdsIn<float>{lbuf}, lbuf, ltw);
        const TwGlobalN twn{tw, 2 * M};
        SpecBatch<kUntangleBatch> sb0;
        if (p == 0) {
            sb0.load(spec, 0, F / 2 + 1, PairsAll{});
            untangle_lds<kUntangleBatch>(lbuf, spec, spec[M], F / 2 + 1, PairsAll{}, 0, ilog2(M), twn, sb0);
        } else {
            sb0.load(spec + F, 0, F / 2, PairsMirror{F});
            untangle_lds<kUntangleBatch>(lbuf, spec + F, spec[M], F / 2, PairsMirror{F}, F, ilog2(M), twn, sb0);
        }
        dit_lds<F, ct_smallest(F), float>(lbuf, ltw);
        copy_from_lds(blk, lbuf, F);
    }
    // Blocks p >= 2 pair with the mirror block pp of their octave.  Per pair:
    // pp's forward transform waits in the scratch, p's stays in LDS; the
    // pair pass untangles the two (p from LDS, pp's mirrored entries from the
    // scratch) and p goes back through its inverse transform from LDS; then
    // pp makes its inverse visit.  Four block reads and four block writes
    // per pair.
    const int lm = ilog2(M);
    for (int p = 2; p < P; ++p) {
        const int a = 31 - __builtin_clz(p);   // octave of block p: blocks [2^a, 2^(a+1))
        const int pp = 3 * (1 << a) - 1 - p;
        if (pp < p) continue;
        FI_GLOBAL Cx<float>* bp = sc + (int64_t)p * F;
        FI_GLOBAL Cx<float>* bq = sc + (int64_t)pp * F;
        copy_to_lds(lbuf, bq, F);
        dif_lds<F, F, float>(LdsIn<float>{lbuf}, lbuf, ltw);
        copy_from_lds(bq, lbuf, F);
        copy_to_lds(lbuf, bp, F);
        dif_lds<F, F, float>(LdsIn<float>{lbuf}, lbuf, ltw);
        // every load of a batch (spectrum, scratch, twiddle) is issued
        // before any is used; each thread's LDS entries are its own
#pragma unroll 1
        for (int k0 = 0; k0 < F; k0 += kTeam * kBatch) {
            V2 sa[kBatch], sb[kBatch];
            Cx<float> zb[kBatch], wf[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int k = k0 + lane + kTeam * u;
                sa[u] = spec[(int64_t)p * F + k];
                sb[u] = spec[(int64_t)pp * F + (F - 1 - k)];
                zb[u] = bq[F - 1 - k];
                wf[u] = tw[2 * M + brev_bits(p * F + k, lm)];   // frequency never 0 in blocks >= 2
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int k = k0 + lane + kTeam * u;
                Cx<float> za = lbuf[lp(k)];
                untangle_pair(za, zb[u], Cx<float>{sa[u].x, sa[u].y}, Cx<float>{sb[u].x, sb[u].y}, wf[u]);
                lbuf[lp(k)] = za;
                bq[F - 1 - k] = zb[u];
            }
        }
        team_sync_global();
        dit_lds<F, ct_smallest(F), float>(lbuf, ltw);
        copy_from_lds(bp, lbuf, F);
        copy_to_lds(lbuf, bq, F);
        dit_lds<F, ct_smallest(F), float>(lbuf, ltw);
        copy_from_lds(bq, lbuf, F);
    }
    global_dit(sc, M, M / (R1 * R2), F, tw);
    // the last two inverse stages fused with the output; only the upper half
    // (outputs U..2U-1 of the circular convolution) is needed
    if (R1 == 4) last_pass_output<4, 1>(out, i, sc, M, tw);
    else if (R2 == 1) last_pass_output<8, 1>(out, i, sc, M, tw);
    else last_pass_output<8, 2>(out, i, sc, M, tw);
}

// The tile tau(x, [i-U, i), h, [i, i+U)) as the circular convolution of
// length 2U of [x[i-U..i), 0_U] with the segment h[1..2U) ([FI] "Trucco di
// Convoluzione Circolare": outputs U..2U-1 are free of wrap-around; the input
// block is padded on the right, [FI] "Dettagli di Implementazione").  The real
// sequences are packed in pairs into M = U complex points; the per-level
// filter spectrum G (M + 2 entries) is untangled against the packing.
// `row` holds the channel's input history (row[s] = x[s] for s < i).
// When x_staged, xst holds the input block x[i-U, i) in LDS (staged by the
// caller); when spec_staged, spec_lds holds the tile's spectrum entries.
// The sink's fields come as separate arguments (registers, not a stack copy).
// The team synchronises after the call (no barrier at its end).
__device__ __forceinline__ void fft_tile(int U, int64_t i, FI_GLOBAL float* row, const FI_GLOBAL V2* spec,
                                      FI_SHARED Cx<float>* lbuf, FI_GLOBAL Cx<float>* sc, TwPtr<float> tw,
                                      const FI_SHARED Cx<float>* twl, FI_SHARED float* accw, int64_t wend,
                                      int wmask, int64_t L, bool first, bool x_staged, const FI_SHARED float* xst,
                                      bool spec_staged, const FI_SHARED V2* spec_lds) {
    const TileSink out{row, accw, wend, wmask, L, first};
    const LdsTw ltw{twl};
    const int M = U;
    const FI_GLOBAL float* xblock = row + (i - U);
    if (x_staged) {
        const FI_SHARED V2* xsl = reinterpret_cast<const FI_SHARED V2*>(xst);
        if (spec_staged) {
            switch (M) {
                case 128: fft_tile_lds<128>(i, TileInLds<64>{xsl}, spec_lds, lbuf, ltw, out); return;
                case 256: fft_tile_lds<256>(i, TileInLds<128>{xsl}, spec_lds, lbuf, ltw, out); return;
                case 512: fft_tile_lds<512>(i, TileInLds<256>{xsl}, spec_lds, lbuf, ltw, out); return;
                case 1024: fft_tile_lds<1024>(i, TileInLds<512>{xsl}, spec_lds, lbuf, ltw, out); return;
                default: break;
            }
        } else if (M == 2048) {
            fft_tile_lds<2048>(i, TileInLds<1024>{xsl}, spec, lbuf, ltw, out);
            return;
        }
    }
    const FI_GLOBAL V2* xg = reinterpret_cast<const FI_GLOBAL V2*>(xblock);
    switch (M) {
        case 64: fft_tile_lds<64>(i, TileIn<32>{xg}, spec, lbuf, ltw, out); return;
        case 128: fft_tile_lds<128>(i, TileIn<64>{xg}, spec, lbuf, ltw, out); return;
        case 256: fft_tile_lds<256>(i, TileIn<128>{xg}, spec, lbuf, ltw, out); return;
        case 512: fft_tile_lds<512>(i, TileIn<256>{xg}, spec, lbuf, ltw, out); return;
        case 1024: fft_tile_lds<1024>(i, TileIn<512>{xg}, spec, lbuf, ltw, out); return;
        case 2048: fft_tile_lds<2048>(i, TileIn<1024>{xg}, spec, lbuf, ltw, out); return;
        case 4096: fft_tile_lds<4096>(i, TileIn<2048>{xg}, spec, lbuf, ltw, out); return;
        default: break;
    }
    fft_tile_big(M, i, xblock, spec, lbuf, sc, tw, twl, row, accw, wend, wmask, L, first);
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

// The red cell of position t and, in the same launch, the direct tile of
// side U <= T that position t+1 completes.  Thread (channel, r) computes
// output r of the tile; it takes x[t] (the tile's last input) from x_t
// rather than from the row, so it does not wait for the red cell's store,
// and thread r = 0 also does the red cell.  Each output is the direct
// Toeplitz sum acc[i+r] += sum_{j<U} x[i-U+j] h[U+r-j], j ascending.
template <bool BF16>
__global__ void k_step_tile(float* state, const float* hT, int64_t LS, int64_t L, int64_t D, int64_t C,
                            int64_t t, const void* x_t, float* y_t, int U) {
    const int64_t n = C * (int64_t)U;
    const int64_t i = t + 1;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ch = idx / U;
        const int r = (int)(idx % U);
        const float* hr = hT + (ch % D) * LS;
        float* row = state + ch * LS;
        const float xv = load_io<BF16>(x_t, ch);
        if (r == 0) {
            y_t[ch] = __builtin_fmaf(hr[0], xv, row[t]);   // accumulated tiles + red cell
            row[t] = xv;                                   // the slot now holds x[t]
        }
        if (i + r >= L) continue;
        const float* xr = row + (i - U);
        const float* hu = hr + U + r;
        float acc = 0.f;
        for (int j = 0; j < U - 1; ++j) acc = __builtin_fmaf(xr[j], hu[-j], acc);
        acc = __builtin_fmaf(xv, hu[-(U - 1)], acc);
        row[i + r] += acc;
    }
}

// Fills the twiddle table A[64] = w_64^a, B[64] = w_4096^b, C[4] = w_16384^r (fp64
// sincospi of exact dyadic arguments, rounded to fp32).
__device__ __forceinline__ void fill_lds_twiddles(FI_SHARED Cx<float>* t) {
    const int lane = threadIdx.x;
    if (lane >= 64) return;
    double sn, cs;
    sincospi(2.0 * lane / 64.0, &sn, &cs);
    t[lane] = Cx<float>{(float)cs, (float)-sn};
    sincospi(2.0 * lane / 4096.0, &sn, &cs);
    t[64 + lane] = Cx<float>{(float)cs, (float)-sn};
    if (lane < 4) {
        sincospi(2.0 * lane / 16384.0, &sn, &cs);
        t[128 + lane] = Cx<float>{(float)cs, (float)-sn};
    }
}

__global__ __launch_bounds__(kTeam) void k_tile_fft(DevState d, int64_t i, int U) {
    extern __shared__ __align__(16) unsigned char smem[];
    FI_SHARED Cx<float>* twl = smem_ptr(reinterpret_cast<Cx<float>*>(smem));
    FI_SHARED Cx<float>* lbuf = twl + kTwLds;
    fill_lds_twiddles(twl);
    team_sync();
    const int q = ilog2(U);  // level
    const FI_GLOBAL V2* spec = gmem(static_cast<const V2*>(d.spec)) + d.spec_off[q];
    for (int64_t ch = blockIdx.x; ch < d.C; ch += gridDim.x) {
        FI_GLOBAL float* row = gmem(d.state + ch * d.LS);
        FI_GLOBAL Cx<float>* sc = gmem(static_cast<Cx<float>*>(d.scratch)) + (int64_t)blockIdx.x * d.sc_stride;
        const int64_t frow = (ch / (d.fset * d.D)) * d.D + ch % d.D;   // the channel's filter row
        fft_tile(U, i, row, spec + frow * (int64_t)(U + 2), lbuf, sc, gmem(static_cast<const Cx<float>*>(d.twf)), twl,
                 reinterpret_cast<FI_SHARED float*>(lbuf), i, 0, d.L, false, false, nullptr, false, nullptr);
        team_sync_global();
    }
}

// ============================================================ persistent run
// One team per channel runs all L positions, in blocks of kBlk = 256
// positions.  Its first wavefront runs the serial part (lane r holds
// positions t0 + 64k + r, k < kRegs, in registers); the whole team runs the
// tiles.
//  * Within a block, the red cells and every tile of side < 256 -- these lie
//    inside one 256-position block and together cover its lower triangle --
//    run in registers: once x[t] is known it is pushed, times the filter tap
//    of each lag, into the accumulators of t and of every later position of
//    the block (lag 0 is the red cell), so the register of position t holds
//    y[t] when it is read.  The same products reach the same outputs as those
//    tiles.  Taps come from an LDS table of 16-byte entries, the taps of
//    four consecutive steps each (zero for negative lags).
//  * At each block boundary i = t0 + kBlk the tile of side U = lowbit(i) >=
//    kBlk runs: a direct Toeplitz product from LDS when U <= T, else the FFT
//    tile.
// Accumulators of positions [t0, t0+W) (W = kBlk) live in an LDS ring.  A
// tile's outputs beyond it go to the channel's global row, which holds the
// input history x below the current position (the FFT tiles read their input
// blocks there) and the accumulated tile outputs above it: the first tile of
// each level (i = U) stores, later ones add.  A block loads its successor's
// accumulators from the row while its chain runs.
constexpr int kRegs = kRunBlock / kWave;   // accumulator registers per lane
constexpr int kBlk = kRunBlock;
constexpr int kLog2Blk = ilog2c(kBlk);
static_assert((1 << kLog2Blk) == kBlk && kRegs <= 8, "block size");

// f(integral_constant<int, K>) for K = K0 .. kRegs-1, in order.
template <int K0, typename F>
__device__ __forceinline__ void for_segments(F&& f) {
    if constexpr (K0 < kRegs) {
        f(std::integral_constant<int, K0>{});
        for_segments<K0 + 1>(f);
    }
}
// f(integral_constant<int, N>) for N = N0 .. N1-1, in order.
template <int N0, int N1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N0 < N1) {
        f(std::integral_constant<int, N0>{});
        static_for<N0 + 1, N1>(f);
    }
}

// ------------------------------------------------ tile of side kBlk, MFMA
// The tile at a block boundary i with U = lowbit(i) = kBlk = 256 (the pages'
// relaxed tiling: inputs [i-256, i), outputs [i, i+256), filter lags
// 1 .. 511), as a direct Toeplitz product on the matrix cores.
// Outputs q = a + 16 alpha (a, alpha < 16) and inputs p = a - d + 16 bt, with
// d = (a - p) mod 16 in [0, 16) and bt in [0, 17): the lag is
//   256 + q - p = 256 + d + 16 (alpha - bt),
// which does not depend on a.  So with K = (d, bt) and
//   A_d[alpha][bt] = h[256 + d + 16 (alpha - bt)],  B_d[bt][a] = x[a - d + 16 bt]
// (x = 0 outside [0, 256)), y[a + 16 alpha] = sum_d (A_d B_d)[alpha][a]: per
// d five 16x16x4 fp32 MFMA steps over bt = 4c + kk (bt = 17 .. 19 meet zero
// inputs), 80 steps in all.  The 16x16 result is added into the LDS ring
// (the next block's accumulators).
//   xz[15 + p] = x[p], zero for p in [-15, 0) and [256, 321);
//   hsk[s(g)] = h[g] for g in [-64, 512) (zero for g < 0 and g >= L), at
//     slot s(g) = (g + 64) + (g + 64) / 16: consecutive alpha - kk = j read
//     slots 17 apart (distinct banks).
// MFMA lane layout (16x16x4): A[i][k] in lane i + 16k, B[k][j] in lane
// j + 16k, D[i][j] in lane j + 16 (i / 4), register i % 4.
typedef float v4f __attribute__((ext_vector_type(4)));

// The accumulation shared by the matrix-core products of one block: init
// plus the 16 NC steps (d = n / NC, c = n % NC) of A_d B_d in the decimated
// order above, where step (d, c), lane (alpha, kk) of A reads the skewed
// filter copy at G + G / 16 + 17 (alpha - kk) with G = GBASE + d - 64 c, and B
// reads the padded input at a + 16 kk + 64 c - d + 15.  Run by the calling
// wavefront; D[alpha][a] in lane a + 16 (alpha / 4), register alpha % 4.
// The operands of a group of kG steps are loaded while the group before it
// is multiplied; four accumulators keep four products in flight.
template <int NC, int GBASE, int D0 = 0, int ND = 16>
__device__ __forceinline__ v4f mm_toeplitz(const FI_SHARED float* ab, const FI_SHARED float* bb, v4f init) {
    constexpr int kSteps = ND * NC, kG = 8, kGroups = kSteps / kG;
    static_assert(kSteps % kG == 0, "whole groups");
    v4f acc[4];
    acc[0] = init;
#pragma unroll
    for (int u = 1; u < 4; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
    float av[2][kG], bv[2][kG];
    auto load = [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        static_for<0, kG>([&](auto uc) {
            constexpr int n = g * kG + decltype(uc)::value;
            constexpr int d = D0 + n / NC, c = n % NC;
            constexpr int G = GBASE + d - 64 * c;
            static_assert(G >= 64, "slots of the filter copy stay in range");
            av[g & 1][n % kG] = ab[G + G / 16];
            bv[g & 1][n % kG] = bb[64 * c - d + 15];
        });
    };
    load(std::integral_constant<int, 0>{});
    static_for<0, kGroups>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        // the scheduler keeps the next group's loads ahead of this group's
        // products
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g + 1 < kGroups) load(std::integral_constant<int, g + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, kG>([&](auto uc) {
            constexpr int u = decltype(uc)::value, n = g * kG + u;
            acc[n & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[g & 1][u], bv[g & 1][u], acc[n & 3], 0, 0, 0);
        });
    });
    __builtin_amdgcn_sched_barrier(0);
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// ------------------------------- tiles of side 256 and 512, fp16 halves
// The tiles at the block boundaries i with lowbit(i) = 256 or 512 (the
// relaxed tiling of [FI] "Strategia di Tiling (Algoritmo 1)") as direct
// Toeplitz products on the matrix cores.  Every product here takes one input
// block of 256 positions and adds into the next block's accumulators (the
// LDS ring), with filter lags G + q - p (q, p the output and input offsets in
// their blocks):
//   i = 256 mod 512: the tile of side 256, G = 256 (lags 1 .. 511);
//   i = 512 mod 1024: the tile of side 512 into its first output block --
//     inputs [i-256, i) with G = 256 and [i-512, i-256) with G = 512;
//   i = 768 mod 1024: also the second output block of the tile of side 512
//     formed at i - 256 -- inputs [i-512, i-256) with G = 512 and
//     [i-768, i-512) with G = 768 -- since those outputs are the block that
//     now comes next.
// Outputs q = a + 16 alpha and inputs p = a - d + 16 bt (a, alpha, d < 16):
// the lag G + d + 16 (alpha - bt) does not depend on a, so with K = (bt, d)
//   A[alpha][(bt, d)] = h[G + d + 16 (alpha - bt)],  B[(bt, d)][a] = x[a - d + 16 bt]
// (x = 0 outside the block) the tile is the 16 x 16 product A B, K = 18 x 16
// (bt < 17 suffices): nine 16x16x32 steps, one per pair of bt values, a lane
// holding eight consecutive d for one bt.  Each operand is the sum of two
// fp16 parts, hi = fp16(v) and lo = fp16(v - hi), after an exact power-of-two
// scaling that puts the largest |v| in [2^13, 2^14): a step is the three
// products hi hi + hi lo + lo hi, accumulated in fp32, and the result is
// scaled back exactly.  The part left out, lo lo, and the parts' rounding are
// below 2^-21 of the largest product.
// Operands in LDS: A from the filter table (H[lag - lo], eight
// consecutive lags, 16-byte aligned); B from the slot's reversed input copies
// (copy c holds x[287 + c - m] at m, so the eight values x[s], x[s-1], ...,
// x[s-7] sit at m = 287 - s + c, .. + 7, with c the parity that makes m
// even: four aligned dwords).
// MFMA lane layout (16x16x32 f16): A[i][k] in lane i + 16 (k / 8), half k % 8;
// B[k][j] in lane j + 16 (k / 8); D[i][j] in lane j + 16 (i / 4), register i % 4.
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// The largest |v| over a wavefront (every lane gets it).
__device__ __forceinline__ float wave_max_abs(float v) {
    int m = __float_as_int(fabsf(v));   // non-negative floats order as integers
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x124, 0xF, 0xF, false));   // row_ror 4
    m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x128, 0xF, 0xF, false));   // row_ror 8
    const int r = max(max(__builtin_amdgcn_readlane(m, 0), __builtin_amdgcn_readlane(m, 16)),
                      max(__builtin_amdgcn_readlane(m, 32), __builtin_amdgcn_readlane(m, 48)));
    return __int_as_float(r);
}
// The scale exponent e with m 2^e < 2^14 (m = the largest magnitude; 14 when m = 0).
__device__ __forceinline__ int scale16(float m) { return 14 - __builtin_amdgcn_frexp_expf(m); }
// The fp16 parts of v 2^e.
__device__ __forceinline__ void split16(float v, int e, _Float16& hi, _Float16& lo) {
    const float s = __builtin_amdgcn_ldexpf(v, e);
    hi = (_Float16)s;
    lo = (_Float16)(s - (float)hi);
}

// One wavefront's steps n in [N0, N1) of the product of an input slot X with
// filter offset G, added to acc (D layout above, still scaled).
template <int N0, int N1, bool TRI>
__device__ __forceinline__ v4f mm16_steps(const FI_SHARED _Float16* H, const FI_SHARED _Float16* X, int G, v4f acc) {
    const int l = team_tid() & (kWave - 1);
    const int r = l & 15, g = l >> 4;
    const int d0 = 8 * (g & 1), bh = g >> 1;   // step n: bt = 2 n + bh, d = d0 .. d0 + 7
    using A16 = F16Area<TRI>;
    const FI_SHARED _Float16* ah = H + (G - A16::kLo + 16 * (r - bh) + d0);   // step n: - 32 n
    const int e0 = 287 - (r + 16 * bh - d0);                                 // step n: - 32 n
    const int cp = e0 & 1;
    const FI_SHARED _Float16* xh = X + cp * kX16N + e0 + cp;
    h8v a_hi[2], a_lo[2], b_hi[2], b_lo[2];
    auto load = [&](int n, int u) {
        a_hi[u] = *reinterpret_cast<const FI_SHARED h8v*>(ah - 32 * n);
        a_lo[u] = *reinterpret_cast<const FI_SHARED h8v*>(ah - 32 * n + A16::kN);
        const FI_SHARED unsigned* ph = reinterpret_cast<const FI_SHARED unsigned*>(xh - 32 * n);
        const FI_SHARED unsigned* pl = reinterpret_cast<const FI_SHARED unsigned*>(xh - 32 * n + 2 * kX16N);
        b_hi[u] = __builtin_bit_cast(h8v, u4v{ph[0], ph[1], ph[2], ph[3]});
        b_lo[u] = __builtin_bit_cast(h8v, u4v{pl[0], pl[1], pl[2], pl[3]});
    };
    load(N0, 0);
#pragma unroll
    for (int n = N0; n < N1; ++n) {
        const int u = (n - N0) & 1;
        if (n + 1 < N1) load(n + 1, u ^ 1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[u], b_hi[u], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[u], b_lo[u], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[u], b_hi[u], acc, 0, 0, 0);
    }
    return acc;
}

// The number of products at boundary i (lowbit(i) = U in {256, 512}).
__device__ __forceinline__ int mm16_count(int64_t i, int U) {
    return U == kBlk ? (((i & (4 * kBlk - 1)) == 3 * kBlk) ? 3 : 1) : 2;
}

// Products 1 .. np-1 of boundary i, whose inputs are older than the block
// before i: formed by one wavefront alone (all nine steps), so that the team's
// second wavefront can form them during the chain of that block, on the
// matrix cores the chain leaves idle.
template <bool TRI>
__device__ __forceinline__ v4f mm16_pre(int64_t i, int np, const FI_SHARED _Float16* H, const FI_SHARED _Float16* X16,
                                        const FI_SHARED int* ex, int eh) {
    v4f y = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1   // one code path, cached between boundaries (faster than unrolled)
    for (int pr = 1; pr < 3; ++pr) {
        if (pr < np) {
            const int64_t tin = i - (int64_t)kBlk * (pr + 1);
            const int slot = (int)(tin >> kLog2Blk) & 3;
            const v4f a = mm16_steps<0, 9, TRI>(H, X16 + F16Area<TRI>::slot_off(slot), kBlk * (pr + 1),
                                                v4f{0.f, 0.f, 0.f, 0.f});
            const int e = -(ex[slot] + eh);
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] += __builtin_amdgcn_ldexpf(a[k], e);
        }
    }
    return y;
}

// The products 0 .. np-1 of boundary i (see above), added into the LDS ring,
// plus `pre` (the second wavefront's sum of products formed earlier; zero
// elsewhere).  The first wavefront takes steps 0 .. 4 of every product, the
// second 5 .. 8 and hands its sums over through `part` (256 floats); the first
// adds both to the ring in a fixed order.  ex[slot] and eh are the scale
// exponents of the input slots and of the filter table.  EARLY (np = 1): the
// second wavefront formed steps 0 .. 3 of product 0 during the chain, from
// the first half of the block's inputs (they only reach inputs below 128),
// and `pre` holds them; the rest is split 4 .. 6 / 7 .. 8.
template <bool TRI, bool EARLY = false>
__device__ __forceinline__ void mm16_tiles(int64_t i, int np, const FI_SHARED _Float16* H,
                                           const FI_SHARED _Float16* X16, const FI_SHARED int* ex, int eh,
                                           FI_SHARED float* ring, FI_SHARED float* part, v4f pre) {
    const int tid = team_tid();
    const int l = tid & (kWave - 1);
    const bool first = __builtin_amdgcn_readfirstlane(tid) < kWave;
    v4f y = pre;
    if constexpr (EARLY) {
        const int slot = (int)((i - kBlk) >> kLog2Blk) & 3;
        const FI_SHARED _Float16* X = X16 + F16Area<TRI>::slot_off(slot);
        v4f a = v4f{0.f, 0.f, 0.f, 0.f};
        if (first) a = mm16_steps<4, 7, TRI>(H, X, kBlk, a);
        else a = mm16_steps<7, 9, TRI>(H, X, kBlk, a);
        const int e = -(ex[slot] + eh);
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] += __builtin_amdgcn_ldexpf(a[k], e);
    }
#pragma unroll 1   // one code path, cached between boundaries (faster than unrolled)
    for (int pr = 0; pr < 3; ++pr) {
        if (!EARLY && pr < np) {
            const int64_t tin = i - (int64_t)kBlk * (pr + 1);   // the input block
            const int G = kBlk * (pr + 1);
            const int slot = (int)(tin >> kLog2Blk) & 3;
            const FI_SHARED _Float16* X = X16 + F16Area<TRI>::slot_off(slot);
            v4f a = v4f{0.f, 0.f, 0.f, 0.f};
            if (first) a = mm16_steps<0, 5, TRI>(H, X, G, a);
            else a = mm16_steps<5, 9, TRI>(H, X, G, a);
            const int e = -(ex[slot] + eh);
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] += __builtin_amdgcn_ldexpf(a[k], e);
        }
    }
    if (!first) {
#pragma unroll
        for (int k = 0; k < 4; ++k) part[4 * l + k] = y[k];
    }
    team_sync();
    if (first) {
        const int al = l & 15, kk = l >> 4;
        // position q = al + 16 alpha, alpha = 4 kk + k
#pragma unroll
        for (int k = 0; k < 4; ++k) ring[al + 16 * (4 * kk + k)] += y[k] + part[4 * l + k];
    }
}

// The block's inputs x[p] (lane l holds p = 64 k + l in v[k]), for k in
// [K0, K1), into input slot X as fp16 parts scaled by 2^e, in both reversed
// copies.
template <int K0 = 0, int K1 = kRegs>
__device__ __forceinline__ void put_x16(FI_SHARED _Float16* X, const float* v, int e) {
    const int l = team_tid() & (kWave - 1);
#pragma unroll
    for (int k = K0; k < K1; ++k) {
        const int p = kWave * k + l;
        _Float16 hi, lo;
        split16(v[k], e, hi, lo);
        X[287 - p] = hi;
        X[kX16N + 288 - p] = hi;
        X[2 * kX16N + 287 - p] = lo;
        X[3 * kX16N + 288 - p] = lo;
    }
}

// The zero padding of the input slots: in each copy the positions no input
// reaches (x[p] for p outside [0, 256); copy 0 holds inputs at [32, 288),
// copy 1 at [33, 289)).  Without TRI, as whole dwords [0, 17) and [144, 152)
// (a dword there that also holds an input is written before the block's
// inputs are); with TRI, no dword an input reaches, so the chain wavefront
// may write a block's inputs at any time.  Run by NT threads from tid.
template <int NT, bool TRI>
__device__ __forceinline__ void zero_x16_pad(FI_SHARED _Float16* X16, int tid) {
    FI_SHARED unsigned* w = reinterpret_cast<FI_SHARED unsigned*>(X16);
    if constexpr (!TRI) {
        constexpr int kPerCopy = 17 + 8, kCopies = 3 * 4;
        for (int q = tid; q < kPerCopy * kCopies; q += NT) {
            const int cpy = q / kPerCopy, o = q % kPerCopy;
            w[cpy * (kX16N / 2) + (o < 17 ? o : 144 + (o - 17))] = 0u;
        }
    } else {
        constexpr int kPerCopy = 16 + 8, kCopies = F16Area<TRI>::kSlots * 4;
        for (int q = tid; q < kPerCopy * kCopies; q += NT) {
            const int cpy = q / kPerCopy, o = q % kPerCopy;
            const bool c1 = cpy & 1;   // copy 1 of its part
            if (o < 16) w[cpy * (kX16N / 2) + o] = 0u;   // halfs [0, 32)
            else if (!c1 || o > 16) w[cpy * (kX16N / 2) + 144 + (o - 16)] = 0u;   // [288 (c1: 290), 304)
            else {   // copy 1: the halfs 32 and 289
                X16[cpy * kX16N + 32] = (_Float16)0.f;
                X16[cpy * kX16N + 289] = (_Float16)0.f;
            }
        }
    }
}

// The filter table from the channel's filter row (lags below kFirst, >= 1024
// and >= L are zero), scaled by 2^eh: load (every load issued before any is
// used), then store.  Run by NT threads from tid.
template <int NT, bool TRI>
struct H16Rows {
    using A16 = F16Area<TRI>;
    static constexpr int NPER = (A16::kN + NT - 1) / NT;
    float v[NPER];
    __device__ __forceinline__ void load(const FI_GLOBAL float* hrow, int64_t L, int tid) {
#pragma unroll
        for (int u = 0; u < NPER; ++u) {
            const int64_t g = (int64_t)(tid + NT * u) + A16::kLo;
            v[u] = hrow[g < A16::kFirst ? 0 : (g < L ? g : L - 1)];
        }
#pragma unroll
        for (int u = 0; u < NPER; ++u) {
            const int g = tid + NT * u + A16::kLo;
            if (!(g >= A16::kFirst && g < L && g < 1024)) v[u] = 0.f;
        }
    }
    __device__ __forceinline__ float max_abs() const {
        float m = 0.f;
#pragma unroll
        for (int u = 0; u < NPER; ++u) m = fmaxf(m, fabsf(v[u]));
        return m;
    }
    __device__ __forceinline__ void store(FI_SHARED _Float16* H, int eh, int tid) const {
#pragma unroll
        for (int u = 0; u < NPER; ++u) {
            const int q = tid + NT * u;
            if (q < A16::kN) {
                _Float16 hi, lo;
                split16(v[u], eh, hi, lo);
                H[q] = hi;
                H[A16::kN + q] = lo;
            }
        }
    }
};

// Open loop: a block's own lower triangle (lags 0 .. 255; the inputs are all
// known, so nothing is serial) as one matrix-core product in the same
// decimated order, lag d + 16 (alpha - bt): with the filter copy hz holding
// h[g] for g in [-256, 256) at slot s(g) = (g + 256) + (g + 256) / 16 (zero
// at negative lags), G = 256 + d - 64 c.  bt = 4c + kk <= 15 suffices (larger
// bt only meets negative lags): 64 steps, split by d between the team's two
// wavefronts (mm_triangle_half<0> from init, mm_triangle_half<8> from zero),
// each result in MFMA layout.
template <int D0>
__device__ __forceinline__ v4f mm_triangle_half(const FI_SHARED float* xz, const FI_SHARED float* hz, v4f init) {
    const int l = team_tid() & (kWave - 1);
    const int al = l & 15, kk = l >> 4;
    return mm_toeplitz<4, 256, D0, 8>(hz + 17 * (al - kk), xz + al + 16 * kk, init);
}

constexpr int kTapBatch = 4;         // chain: taps loaded per batch, one batch ahead
constexpr int kStageSpecMax = 1024;  // tiles up to this side get spectrum and input staged in LDS
// (FFT buffer 9M bytes + input 4U + spectrum 8 (U + 2) fits the 36 KiB region
// for U <= 1024; U = 2048 stages the input only)

struct RunArgs {
    DevState d;
    const void* x_in;
    float* y;
    void* x_out;
    int64_t prompt;   // prompted runs: the number of given inputs
};

__device__ __forceinline__ void direct_tile_lds(int64_t i, int U, const FI_SHARED float* xring, int xmask,
                                                const FI_SHARED float* htap, FI_SHARED float* accw, int wmask,
                                                int64_t L) {
    for (int r = team_tid(); r < U; r += kTeam) {
        float acc = 0.f;
        const FI_SHARED float* hp = htap + U + r;
#pragma unroll 8
        for (int j = 0; j < U; ++j) acc = __builtin_fmaf(xring[(i - U + j) & xmask], hp[-j], acc);
        if (i + r < L) accw[(i + r) & wmask] += acc;
    }
}

// LDS of k_run: static arrays for the tap table, the twiddle table and the
// accumulator ring (separate objects, so the compiler sees that the direct-to-
// LDS staging loads into the dynamic region never touch them), and a dynamic
// region: FFT / staging area [fftreg bytes] | (T >= kBlk only) xring[XR] | htap[2T].
inline int run_lds_floats(const DevState& d) { return kRunFftReg / 4 + (d.T >= kBlk ? d.XR + 2 * d.T : 0); }

template <bool CLOSED, bool BF16, bool PROMPT = false>
__global__ __launch_bounds__(kTeam) __attribute__((amdgpu_waves_per_eu(kTeamWaves))) void k_run(RunArgs a) {
    static_assert(CLOSED || !PROMPT, "a prompted run feeds back after its prompt");
    // The fp32 closed loop's chain pushes r = 1 / (1 + 2^(c y)) = (1 - x) / 2
    // rather than x = tanh(y) = 1 - 2 r: with the taps -2 c h and, added to
    // every position's accumulator at the start of its block, the prefix sums
    // of the taps c h (the "1" of every input of the block that reaches it),
    // the accumulators hold the same sums, and x = 1 - 2 r is no longer on
    // the serial path.  (bf16 storage rounds x itself, and a prompted run
    // pushes given inputs: both keep pushing x.)
    constexpr bool RPUSH = CLOSED && !BF16 && !PROMPT;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ Cx<float> s_tw[kTwLds];  // twiddles A[64] = w_64^a, B[64] = w_4096^b, C[4] = w_16384^r
    __shared__ float s_ring[kBlk];      // accumulators of positions [t0, t0+W)
    __shared__ float s_pre[RPUSH ? kBlk : 1];   // the chain's tap prefix sums (RPUSH)
    const DevState& d = a.d;
    FI_SHARED Cx<float>* lbuf = smem_ptr(reinterpret_cast<Cx<float>*>(smem));
    FI_SHARED Cx<float>* twl = smem_ptr(s_tw);
    FI_SHARED float* accw = smem_ptr(s_ring);
    FI_SHARED float* xring = reinterpret_cast<FI_SHARED float*>(smem_ptr(smem) + kRunFftReg);  // direct tiles only
    FI_SHARED float* htap = xring + d.XR;    // h[0 .. 2T), direct tiles only
    const bool direct = d.T >= kBlk;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // The team's first wavefront runs the chain; the others wait at the
    // barrier before each tile and share the tile's work (the test is uniform
    // per wavefront, so it is a branch, not a mask).
    const bool chain_wave = __builtin_amdgcn_readfirstlane(tid) < kWave;
    const int wmask = kBlk - 1, xmask = d.XR - 1;
    const int64_t L = d.L, D = d.D;
    // Positions [0, P) take their input from x_in (x_in[B][P][D]), later ones
    // the fed-back tanh(y): P = L in open loop, 1 in closed loop, the
    // prompt's length in a prompted run.  A block whose inputs are all given
    // has no serial chain and runs as in open loop.
    const int64_t P = PROMPT ? a.prompt : (CLOSED ? 1 : L);
    auto open_block = [&](int64_t t) { return !CLOSED || (PROMPT && t + kBlk <= P); };
    const int G = gridDim.x, bid = blockIdx.x;
    // consecutive channels on the same XCD (workgroups go round-robin over
    // the 8 XCDs), so their strided y / x_out rows meet in one L2
    const int64_t ch0 = (G % 8 == 0) ? (int64_t)(bid % 8) * (G / 8) + bid / 8 : bid;
    TwPtr<float> tw = gmem(static_cast<const Cx<float>*>(d.twf));
    FI_GLOBAL Cx<float>* sc = gmem(static_cast<Cx<float>*>(d.scratch)) + (int64_t)bid * d.sc_stride;
    FI_GLOBAL float* yout = gmem(a.y);
    // The chain's taps: with hz[q] = s h[q - 64] for 64 <= q < 64 + kBlk, else
    // 0 (s = c in closed loop, see below, else 1), tz[q + 3] = (hz[q],
    // hz[q-1], hz[q-2], hz[q-3]) holds the taps of four consecutive chain
    // steps in one 16-byte read.
    constexpr int t4_off = kRunFftReg - kTapTableBytes;
    FI_SHARED V4* tz = reinterpret_cast<FI_SHARED V4*>(smem_ptr(smem) + t4_off);
    const float tap_scale = CLOSED ? kTanhScale : 1.0f;
    const float chain_scale = RPUSH ? -2.0f * kTanhScale : tap_scale;   // the chain's taps
    // A block with every input given has no chain: the same region then
    // holds the filter copy of the block triangle on the matrix cores,
    // hz[s(g)] = h[g] for g in [-256, 256), s(g) = (g + 256) + (g + 256) / 16,
    // zero at negative lags and from L on (open_form).
    FI_SHARED float* hz = reinterpret_cast<FI_SHARED float*>(tz);
    static_assert((2 * kBlk + 2 * kBlk / 16) * 4 <= kTapTableBytes, "the triangle's filter copy fits");
    auto build_taps4 = [&](const FI_GLOBAL float* hrow, bool open_form) {
        if (CLOSED && !open_form) {
            for (int e = tid; e < kTapTableBytes / 16; e += kTeam) {
                const int q = e - 3 - kWave;   // lag of the first component
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (q - j >= 0 && q - j < kBlk && q - j < L) ? chain_scale * hrow[q - j] : 0.f;
                tz[e] = V4{v[0], v[1], v[2], v[3]};
            }
        } else {
            for (int e = tid; e < 2 * kBlk; e += kTeam) {
                const int g = e - kBlk;
                hz[e + e / 16] = (g >= 0 && g < L) ? hrow[g] : 0.f;
            }
        }
    };
    // the block's zero-padded inputs (cleared when a channel starts and
    // after a tile whose transform reaches them)
    FI_SHARED float* mxz = reinterpret_cast<FI_SHARED float*>(smem_ptr(smem) + kRunMmOff);
    FI_SHARED float* myb = mxz + kMmXFloats;   // the block's y, for the other wavefronts' stores
    auto build_mm = [&](const FI_GLOBAL float* hrow) {
        for (int q = tid; q < kMmXFloats; q += kTeam) mxz[q] = 0.f;
    };
    // The tiles of side kBlk and 2 kBlk on the matrix cores in fp16 halves
    // (mm16_tiles) wherever the direct tiles stop below kBlk: the filter
    // table, the input slots and their scale exponents.
    const bool f16 = d.T < kBlk;
    FI_SHARED _Float16* H16 = reinterpret_cast<FI_SHARED _Float16*>(smem_ptr(smem) + kH16Off);
    // runs with blocks whose inputs are all given form those blocks'
    // triangles in fp16 halves too (a wider table and a fourth input slot)
    constexpr bool TRI = !CLOSED || PROMPT;
    using A16 = F16Area<TRI>;
    FI_SHARED _Float16* X16 = reinterpret_cast<FI_SHARED _Float16*>(smem_ptr(smem) + A16::kXOff);
    __shared__ int s_ex16[A16::kSlots];
    __shared__ float s_hmax[kTeamWaves];
    int eh = 0;   // the filter table's scale exponent (per channel)
    // RPUSH chain blocks before a boundary of side kBlk or 2 kBlk: after the
    // chain's second segment the chain wavefront hands over its registers of
    // the block's first 128 positions and then stores the count of such
    // blocks so far here; the other wavefront, waiting for that count, forms
    // those positions' inputs in fp16 parts and the steps of the block's
    // product that reach only them, during the rest of the chain (mm16_tiles,
    // EARLY)
    __shared__ int s_early;
    int n_early = 0;
    if (tid == 0) *smem_ptr(&s_early) = 0;   // ordered by the first channel's barrier
    fill_lds_twiddles(twl);
    // Phase timing (profile build only; kProfile is false in the product
    // build and all of this folds away): the chain wavefront's cycle sums,
    // per-level tile sums and counts in LDS.
    __shared__ unsigned long long s_pf[kProfile ? 2 * 24 : 1];
    __shared__ unsigned long long s_hw[kProfile ? 2 : 1];   // each wavefront's XCC id and HW_ID
    [[maybe_unused]] unsigned long long pf_t0 = 0, pf_tb = 0, pf_tc = 0, pf_td = 0, pf_te = 0;
    [[maybe_unused]] unsigned long long pf_setup = 0, pf_chain = 0, pf_wait = 0, pf_store = 0;
    [[maybe_unused]] unsigned long long pf_blocks = 0, pf_chans = 0;
    [[maybe_unused]] unsigned long long pf_s0 = 0, pf_s1 = 0, pf_pro = 0, pf_epi = 0, pf_vm = 0;
    [[maybe_unused]] unsigned long long pf_seg[kRegs] = {};
    if constexpr (kProfile) {
        pf_t0 = clock64();
        for (int q = tid; q < 2 * 24; q += kTeam) s_pf[q] = 0;
        if (lane == 0) {
            // s_getreg operands: (size - 1) << 11 | offset << 6 | register (HW_ID = 4, XCC_ID = 20)
            const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
            const unsigned xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);
            s_hw[chain_wave ? 0 : 1] = ((unsigned long long)xcc << 32) | hw;
        }
    }

    for (int64_t ch = ch0; ch < d.C; ch += G) {
        const int64_t b = ch / D, c = ch % D;
        FI_GLOBAL float* row = gmem(d.state + ch * d.LS);
        const FI_GLOBAL float* hrow = gmem(d.hT + c * d.LS);
        if constexpr (kProfile) {
            pf_tb = clock64();
            pf_chans += 1;
        }
        team_sync();   // the previous channel's last chain is done with the taps and the ring
        for (int q = tid; q < kBlk; q += kTeam) accw[q] = 0.f;
        if (direct)
            for (int q = tid; q < 2 * d.T; q += kTeam) htap[q] = q < L ? hrow[q] : 0.f;
        build_taps4(hrow, open_block(0));
        build_mm(hrow);
        if (f16) {
            // the filter table and its scale (the largest |h| over the lags
            // it holds), and zeroed input slots
            H16Rows<kTeam, TRI> hr;
            hr.load(hrow, L, tid);
            const float hm = wave_max_abs(hr.max_abs());
            if (lane == 0) smem_ptr(s_hmax)[tid / kWave] = hm;
            for (int q = tid; q < A16::kSlots * kX16Slot / 2; q += kTeam) reinterpret_cast<FI_SHARED unsigned*>(X16)[q] = 0u;
            team_sync();
            eh = scale16(fmaxf(smem_ptr(s_hmax)[0], smem_ptr(s_hmax)[1]));
            hr.store(H16, eh, tid);
        }
        if constexpr (RPUSH) {
            const FI_GLOBAL float* pr = gmem(d.pre + c * kBlk);
            for (int q = tid; q < kBlk; q += kTeam) s_pre[q] = pr[q];
        }
        team_sync();
        const float ch0v = chain_scale * hrow[0];   // closed loop: c h[0] (RPUSH: -2 c h[0])

        float xcur = 0.f;        // closed loop: x at the next position (uniform)
        float rcur = 0.f;        // RPUSH: (1 - x) / 2 at the next position (uniform)
        float xbn[kRegs];        // open loop: inputs of the next block
#pragma unroll
        for (int k = 0; k < kRegs; ++k) xbn[k] = 0.f;
        if (chain_wave) {
            if constexpr (CLOSED) xcur = load_io<BF16>(a.x_in, b * P * D + c);   // x[0]
            if constexpr (RPUSH) rcur = (1.0f - xcur) * 0.5f;
            if constexpr (!CLOSED || PROMPT) {
#pragma unroll
                for (int k = 0; k < kRegs; ++k) {
                    const int64_t n = kWave * k + lane;
                    if (n < P) xbn[k] = load_io<BF16>(a.x_in, (b * P + n) * D + c);
                }
            }
            // nothing in flight when the block loop starts, so the waits inside it
            // only cover what each block issues
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        if constexpr (kProfile) pf_setup += clock64() - pf_tb;
        // y and x_out of a block go out during the next block (their
        // addresses are D floats apart per position, so each store touches 64
        // lines and holds up the wavefront that issues it for about as many
        // cycles): the chain wavefront leaves them in LDS (myb, mxz).  Before
        // a chain block the other wavefront stores them; before a block with
        // known inputs the chain wavefront does, at the block's start.  Lane l
        // writes position t0 + 64 k + l of column c.
        const uint32_t ylane = (uint32_t)lane * (uint32_t)D;
        bool defer_prev = false;   // the previous block's y / x_out wait in LDS
        auto store_deferred = [&](int64_t tp) {
            const bool full = tp + kBlk <= L;
#pragma unroll
            for (int k = 0; k < kRegs; ++k) {
                const float yv = myb[kWave * k + lane];
                const float xv = mxz[15 + kWave * k + lane];
                const int64_t ob = (b * L + tp + kWave * k) * D + c;   // uniform
                if (full || tp + kWave * k + lane < L) {
                    (yout + ob)[ylane] = yv;
                    if (a.x_out) store_io<BF16>(a.x_out, ob + ylane, xv);
                }
            }
        };
        for (int64_t t0 = 0; t0 < L; t0 += kBlk) {
            float p[kRegs], xk[kRegs];
            [[maybe_unused]] unsigned long long pf_tw = 0;
            if constexpr (kProfile) {
                pf_tb = clock64();
                pf_s0 = pf_s1 = pf_tw = 0;
                pf_blocks += 1;
            }
            // the next tile's spectrum and older input block go straight to the
            // idle LDS FFT region while the chain runs
            const int64_t inext = t0 + kBlk;
            const int Un = inext < L ? (int)(inext & -inext) : 0;
            // next tile of side kBlk: on the matrix cores (mm_tile256)
            const bool mm_next = Un > d.T && (Un == kBlk || (f16 && Un == 2 * kBlk));
            const bool stage_x = Un > d.T && Un <= 2 * kStageSpecMax && !mm_next;
            const bool stage_spec = Un > d.T && Un <= kStageSpecMax && !mm_next;
            FI_SHARED float* xst = reinterpret_cast<FI_SHARED float*>(lbuf + lds_fft_elems(Un));
            FI_SHARED V2* sst = reinterpret_cast<FI_SHARED V2*>(xst + Un);
            const bool row_input = Un > d.T && !stage_x && !mm_next;   // next tile: FFT reading the row
            // y, x_out and the input history: before a tile that reads its
            // input block from the row, after one that has it staged in LDS;
            // before the matrix-core tile the chain wavefront leaves y in LDS
            // (x is the tile's input there) and the other wavefronts, idle
            // during that tile, store the block
            auto store_block = [&]() {
                const bool full = t0 + kBlk <= L;
#pragma unroll
                for (int k = 0; k < kRegs; ++k) {
                    if (full || t0 + kWave * k + lane < L) {
                        const int64_t ob = (b * L + t0 + kWave * k) * D + c;   // uniform
                        (yout + ob)[ylane] = p[k];
                        if (a.x_out) store_io<BF16>(a.x_out, ob + ylane, xk[k]);
                        row[t0 + kWave * k + lane] = xk[k];  // the slot of a consumed accumulator now holds x
                    }
                }
            };
            // The next block's accumulators beyond the LDS ring: some earlier
            // tile left them in the row exactly when a bit of base other than
            // its lowest is set at or above 2 kBlk (the tile of that bit's
            // level covered them, its ring did not).
            const int64_t base = t0 + kBlk;
            // (with the tiles of side 2 kBlk on the matrix cores, no tile
            // below 4 kBlk writes the row)
            const bool nx_in_row = ((base & (base - 1)) >> (kLog2Blk + (f16 ? 2 : 1))) != 0;
            // A closed-loop block that runs the serial chain: the other
            // wavefront, idle during the chain, issues the previous block's
            // deferred y / x_out stores from LDS and moves the next block's
            // accumulators from the row into the ring, work that would
            // otherwise sit on the chain wavefront's critical path.  It meets
            // the chain wavefront at the start of the chain's second segment:
            // by then the chain wavefront has read the ring, and it rewrites
            // the LDS copies of y / x only after its chain.
            const bool chain_block = CLOSED && !open_block(t0);
            const bool early16 = RPUSH && f16 && inext < L && Un > d.T && Un <= 2 * kBlk;
            if (early16) ++n_early;
            float hnx[kRegs];
            v4f pre16 = v4f{0.f, 0.f, 0.f, 0.f};   // the other wavefront's early products (mm16_pre)
            // after a tile that overwrote the fp16 area (every FFT tile, at
            // multiples of 4 kBlk), the other wavefront restores it: the slots'
            // zero padding before its first barrier (before the chain
            // wavefront writes this block's inputs there), the filter table
            // before the block ends
            const bool redo16 = f16 && t0 > 0 && (t0 & (4 * kBlk - 1)) == 0;
            if (!chain_wave && redo16) zero_x16_pad<kWave, TRI>(X16, lane);
            if (!chain_wave && chain_block) {
                if (defer_prev) store_deferred(t0 - kBlk);
                team_sync();
#pragma unroll
                for (int k = 0; k < kRegs; ++k) {
                    // loaded from a clamped index, kept where in range: a
                    // load under a per-lane branch would wait for the stores
                    const int64_t pn = base + kWave * k + lane;
                    const float v = row[pn < L ? pn : L - 1];
                    hnx[k] = (nx_in_row && pn < L) ? v : 0.f;
                }
            }
            if (!chain_wave) {
                // The other wavefront, idle during the chain, stages the next
                // tile's spectrum and the older part of its input block
                // straight into the idle LDS FFT region, and waits for them
                // before the barrier that ends the chain.
                if (stage_spec) {   // Un + 2 entries of 8 bytes, 16 bytes per lane
                    const FI_GLOBAL V4* sp = reinterpret_cast<const FI_GLOBAL V4*>(
                        gmem(static_cast<const V2*>(d.spec)) + d.spec_off[ilog2(Un)] + c * (int64_t)(Un + 2));
                    FI_SHARED V4* sd = reinterpret_cast<FI_SHARED V4*>(sst);
                    const int n16 = (Un + 2) / 2;
                    for (int k = 0; k < n16; k += kWave)
                        if (k + lane < n16)
                            __builtin_amdgcn_global_load_lds((const FI_GLOBAL void*)(sp + k + lane), (FI_SHARED void*)(sd + k), 16, 0, 0);
                }
                if (stage_x) {
                    for (int k = 0; k < Un - kBlk; k += kWave)
                        __builtin_amdgcn_global_load_lds((const FI_GLOBAL void*)(row + (inext - Un) + k + lane),
                                                         (FI_SHARED void*)(xst + k), 4, 0, 0);
                }
                if (redo16) {
                    H16Rows<kWave, TRI> hr;
                    hr.load(hrow, L, lane);
                    hr.store(H16, eh, lane);
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                if (chain_block) {
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) accw[kWave * k + lane] = hnx[k];   // the ring now holds the next block
                    // the next boundary's products of inputs older than this
                    // block, on the matrix cores the chain leaves idle
                    if (f16 && inext < L && Un > d.T && Un <= 2 * kBlk) pre16 = mm16_pre<TRI>(inext, mm16_count(inext, Un), H16, X16, smem_ptr(s_ex16), eh);
                    if (early16) {
                        // wait (bounded) for the chain wavefront's registers of
                        // the block's first 128 positions; from them, with the
                        // same operations as its epilogue, the inputs x of those
                        // positions into the block's slot as fp16 parts (tanh
                        // values: scale 2^14); then the steps of the block's
                        // product that reach only those inputs
                        for (int it = 0; it < (1 << 22); ++it) {
                            if (__hip_atomic_load(smem_ptr(&s_early), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == n_early) break;
                            __builtin_amdgcn_s_sleep(1);
                        }
                        const int s0 = (int)(t0 >> kLog2Blk) & 3;
                        {
                            const FI_SHARED float* hv = reinterpret_cast<const FI_SHARED float*>(lbuf);
                            const float f0 = __builtin_fmaf(-2.0f, tanh_rcp_scaled(hv[lane]), 1.0f);
                            const float f1 = __builtin_fmaf(-2.0f, tanh_rcp_scaled(hv[kWave + lane]), 1.0f);
                            const float xs = hv[2 * kWave];
                            float xh[2];
                            const float sh0 = wave_shr1(f0), sh1 = wave_shr1(f1);
                            xh[0] = lane == 0 ? xs : sh0;
                            xh[1] = lane == 0 ? readlane(f0, kWave - 1) : sh1;
                            put_x16<0, 2>(X16 + A16::slot_off(s0), xh, 14);
                            if (lane == 0) smem_ptr(s_ex16)[s0] = 14;
                        }
                        const v4f a = mm16_steps<0, 4, TRI>(H16, X16 + A16::slot_off(s0), kBlk, v4f{0.f, 0.f, 0.f, 0.f});
                        const int e = -(smem_ptr(s_ex16)[s0] + eh);
#pragma unroll
                        for (int r = 0; r < 4; ++r) pre16[r] += __builtin_amdgcn_ldexpf(a[r], e);
                    }
                }
                // an open block's own triangle: this wavefront forms the
                // products d >= 8 and hands them over through LDS (the first
                // 256 floats of the FFT region, which no staging reaches)
                if (open_block(t0)) {
                    team_sync();   // the chain wavefront has written the block's inputs
                    v4f yh;
                    if (f16) {
                        const int bslot = (int)(t0 >> kLog2Blk) & 3;
                        const v4f a = mm16_steps<5, 9, TRI>(H16, X16 + A16::slot_off(bslot), 0, v4f{0.f, 0.f, 0.f, 0.f});
                        const int e = -(smem_ptr(s_ex16)[bslot] + eh);
#pragma unroll
                        for (int r = 0; r < 4; ++r) yh[r] = __builtin_amdgcn_ldexpf(a[r], e);
                    } else {
                        yh = mm_triangle_half<8>(mxz, hz, v4f{0.f, 0.f, 0.f, 0.f});
                    }
                    FI_SHARED float* part = reinterpret_cast<FI_SHARED float*>(lbuf);
#pragma unroll
                    for (int r = 0; r < 4; ++r) part[4 * lane + r] = yh[r];
                    team_sync();
                }
            }
            if (chain_wave) {
                // the serial chain goes first wherever it shares a SIMD with
                // another team's tile work
                __builtin_amdgcn_s_setprio(2);
                if (defer_prev && !chain_block) store_deferred(t0 - kBlk);
                float xb[kRegs];
#pragma unroll
                for (int k = 0; k < kRegs; ++k) {
                    xb[k] = xbn[k];
                    p[k] = accw[(kWave * k + lane) & wmask];   // t0 is a multiple of the ring size
                }
                if constexpr (!CLOSED || PROMPT) {
                    if (!CLOSED || t0 + kBlk < P) {   // the next block has given inputs
#pragma unroll
                        for (int k = 0; k < kRegs; ++k) {
                            const int64_t n = t0 + kBlk + kWave * k + lane;
                            xbn[k] = n < P ? load_io<BF16>(a.x_in, (b * P + n) * D + c) : 0.f;
                        }
                    }
                }
                // the accumulators of the next block's positions that wait in
                // the row (the other wavefront moves them in chain blocks)
                float nx[kRegs];
#pragma unroll
                for (int k = 0; k < kRegs; ++k) nx[k] = 0.f;
                if (!chain_block) {
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) {
                        const int64_t pn = base + kWave * k + lane;
                        nx[k] = (nx_in_row && pn < L) ? row[pn] : 0.f;
                    }
                }
                float xstart = 0.f;
                const bool openb = open_block(t0);
                // a prompted run's block that holds the prompt's end: inputs
                // below P are given, the rest fed back
                const bool bnd = PROMPT && t0 < P && P < t0 + kBlk;
                const int pl = (int)(P - t0);   // given inputs of a boundary block
                if (openb) {
                    // every input of the block is known, so its own
                    // triangle is one matrix-core product (mm_triangle_half on
                    // each wavefront) on
                    // top of the ring's accumulators; the inputs go to the
                    // padded block the product (and the tile of side kBlk at
                    // the block's end) reads, and y comes back to the lane
                    // layout through the LDS y buffer
                    static_assert(kRegs * kWave == kBlk && kBlk == 256, "matrix-core triangle layout");
                    const int al = lane & 15, kk = lane >> 4;
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) mxz[15 + kWave * k + lane] = xb[k];
                    v4f init;
#pragma unroll
                    for (int r = 0; r < 4; ++r) init[r] = accw[al + 16 * (4 * kk + r)];
                    const int bslot = (int)(t0 >> kLog2Blk) & 3;
                    if (f16) {
                        // the block's inputs as fp16 halves: its triangle here
                        // (a block product with lag offset 0: the table is
                        // zero at negative lags) and the block products of the
                        // boundaries after it
                        float m = fabsf(xb[0]);
#pragma unroll
                        for (int k = 1; k < kRegs; ++k) m = fmaxf(m, fabsf(xb[k]));
                        const int e = scale16(wave_max_abs(m));
                        put_x16(X16 + A16::slot_off(bslot), xb, e);
                        if (lane == 0) smem_ptr(s_ex16)[bslot] = e;
                    }
                    // the products d < 8 here, d >= 8 on the other wavefront
                    // (fp16 halves: steps 0 .. 4 here, 5 .. 8 there)
                    team_sync();
                    v4f yq;
                    if (f16) {
                        const v4f a = mm16_steps<0, 5, TRI>(H16, X16 + A16::slot_off(bslot), 0, v4f{0.f, 0.f, 0.f, 0.f});
                        const int e = -(smem_ptr(s_ex16)[bslot] + eh);
#pragma unroll
                        for (int r = 0; r < 4; ++r) yq[r] = init[r] + __builtin_amdgcn_ldexpf(a[r], e);
                    } else {
                        yq = mm_triangle_half<0>(mxz, hz, init);
                    }
                    team_sync();
                    const FI_SHARED float* part = reinterpret_cast<const FI_SHARED float*>(lbuf);
#pragma unroll
                    for (int r = 0; r < 4; ++r) yq[r] += part[4 * lane + r];
#pragma unroll
                    for (int r = 0; r < 4; ++r) myb[al + 16 * (4 * kk + r)] = yq[r];
                    wave_sync();
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) p[k] = myb[kWave * k + lane];
                    if constexpr (PROMPT) {
                        // the prompt ends with this block: the next input is
                        // the first fed back, as the chain forms it
                        if (t0 + kBlk == P) {
                            xcur = __builtin_fmaf(-2.0f, tanh_rcp_scaled(kTanhScale * readlane(p[kRegs - 1], kWave - 1)), 1.0f);
                            if constexpr (BF16) xcur = round_bf16(xcur);
                        }
                    }
                } else if constexpr (CLOSED) {
                    // tz0[64k - n]: the taps of position 64k + lane for inputs
                    // n .. n+3 (n a multiple of kTapBatch), in two batches
                    static_assert(kTapBatch == 4, "a tap batch is one 16-byte entry");
                    const FI_SHARED V4* tz0 = tz + 3 + kWave + lane;
                    V4 ta[kRegs][2];
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) ta[k][0] = tz0[kWave * k];
                    float v = 0.f;
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) {
                        if constexpr (RPUSH) p[k] = __builtin_fmaf(p[k], kTanhScale, s_pre[kWave * k + lane]);
                        else p[k] *= kTanhScale;
                    }
                    v = readlane(p[0], 0);
                    if (bnd) xcur = readlane(xb[0], 0);   // x[t0] is given
                    // the block's first input as recorded: the given x[0], or
                    // 1 - 2 r as the previous block's recomputation forms it
                    if constexpr (RPUSH) xstart = t0 == 0 ? xcur : __builtin_fmaf(-2.0f, rcur, 1.0f);
                    else xstart = xcur;
                    // one 64-step segment of the chain (steps 64K .. 64K+63);
                    // BND: inputs below P come from xb instead of the feedback
                    auto segment = [&](auto kc, auto bndc) {
                        constexpr int K = decltype(kc)::value;
                        constexpr bool BND = decltype(bndc)::value;
#pragma unroll
                        for (int m2 = 0; m2 < kWave; ++m2) {
                            const int m = kWave * K + m2;
                            float tv[kRegs];
#pragma unroll
                            for (int k = 0; k < kRegs; ++k) {
                                const V4 t4 = ta[k][(m / kTapBatch) % 2];
                                tv[k] = m % 4 == 0 ? t4.x : m % 4 == 1 ? t4.y : m % 4 == 2 ? t4.z : t4.w;
                            }
                            // closed loop: the accumulators run in units of c = 2 log2(e)
                            // (the taps are c h), so tanh(y) = 1 - 2 r with
                            // r = 1 / (1 + 2^(c y)); v holds position t0+m's accumulator
                            // with every input but its own pushed (read one step ahead,
                            // off the serial path), and the serial path of a position is
                            // c y = v + c h[0] x, exp2, add, rcp, x = 1 - 2 r.  Position
                            // m's own lag-0 push is the same fma as c y, so its register
                            // ends equal to it.
                            // RPUSH: the pushed value is r of the previous position
                            // (x = 1 - 2 r), the taps are -2 c h, and the serial path
                            // is c y = v + (-2 c h[0]) r, exp2, add, rcp
                            const float xm = RPUSH ? rcur : CLOSED ? xcur : readlane(xb[K], m2);
                            const float cy = __builtin_fmaf(ch0v, xm, v);
                            // the exponential goes first; the read of the next
                            // accumulator (a scalar register) then sits two
                            // instructions before its use, clear of the wait
                            // states a scalar written by the vector unit needs
                            [[maybe_unused]] const float ey = CLOSED ? __builtin_amdgcn_exp2f(cy) : 0.f;
#pragma unroll
                            for (int k = K; k < kRegs; ++k) {
                                p[k] = __builtin_fmaf(tv[k], xm, p[k]);
                                pin(p[k]);   // push now: x[t] is then dead after this step
                            }
                            if (m % kTapBatch == 0 && m + kTapBatch < kBlk) {
                                __builtin_amdgcn_sched_barrier(0);
                                const int n = m + kTapBatch;
#pragma unroll
                                for (int k = 0; k < kRegs; ++k)
                                    if (n < kWave * (k + 1)) ta[k][(n / kTapBatch) % 2] = tz0[kWave * k - n];
                            }
                            if constexpr (CLOSED) {
                                if (m + 1 < kBlk) v = readlane(p[(m + 1) / kWave], (m + 1) % kWave);
                                __builtin_amdgcn_sched_barrier(0);
                                // r = 1 / (1 + 2^(c y)), tanh(y) = 1 - 2 r
                                const float rr = __builtin_amdgcn_rcpf(1.0f + ey);
                                if constexpr (RPUSH) {
                                    rcur = rr;
                                } else {
                                    xcur = __builtin_fmaf(-2.0f, rr, 1.0f);
                                    if constexpr (BF16) xcur = round_bf16(xcur);
                                }
                                if constexpr (BND) {
                                    if (m + 1 < kBlk && m + 1 < pl)
                                        xcur = readlane(xb[(m + 1) / kWave], (m + 1) % kWave);
                                }
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    };
                    auto timed = [&](auto kc, auto bndc) {
                        // the other wavefront has taken what it stores and
                        // moves (see chain_block): meet it here
                        if constexpr (decltype(kc)::value == 1) team_sync();
                        if constexpr (RPUSH && decltype(kc)::value == 2) {
                            if (early16) {
                                // the registers of positions below 128 no longer
                                // change: hand them over (with x of the block's
                                // first position) through the hand-over area, idle
                                // during the chain, then the count
                                FI_SHARED float* hv = reinterpret_cast<FI_SHARED float*>(lbuf);
                                hv[lane] = p[0];
                                hv[kWave + lane] = p[1];
                                if (lane == 0) hv[2 * kWave] = xstart;
                                __hip_atomic_store(smem_ptr(&s_early), n_early, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
                            }
                        }
                        [[maybe_unused]] unsigned long long ts = 0;
                        if constexpr (kProfile) {
                            ts = clock64();
                            if (decltype(kc)::value == 0) pf_s0 = ts;
                        }
                        segment(kc, bndc);
                        if constexpr (kProfile) {
                            pf_s1 = clock64();
                            pf_seg[decltype(kc)::value] += pf_s1 - ts;
                        }
                    };
                    if constexpr (PROMPT) {
                        if (bnd) for_segments<0>([&](auto kc) { timed(kc, std::true_type{}); });
                        else for_segments<0>([&](auto kc) { timed(kc, std::false_type{}); });
                    } else {
                        for_segments<0>([&](auto kc) { timed(kc, std::false_type{}); });
                    }
                }
                if (openb) {
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) xk[k] = xb[k];
                } else if constexpr (CLOSED) {
                    // The inputs of the block, one per lane: the register of
                    // position t ended as the same fma as the chain's c y[t], so
                    // the same exp2 / rcp / fma on it gives back x[t+1] exactly.
                    float f[kRegs];
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) {
                        f[k] = __builtin_fmaf(-2.0f, tanh_rcp_scaled(p[k]), 1.0f);
                        if constexpr (BF16) f[k] = round_bf16(f[k]);
                    }
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) {
                        const float prev = k == 0 ? xstart : readlane(f[k - 1], kWave - 1);
                        const float sh = wave_shr1(f[k]);
                        xk[k] = lane == 0 ? prev : sh;
                        if (bnd && t0 + kWave * k + lane < P) xk[k] = xb[k];   // given
                        p[k] *= 1.0f / kTanhScale;
                    }
                }
                // Everything this block loaded (staging, next accumulators) was
                // issued a whole chain ago: wait for it here, before the stores
                // below (stores count in the same counter, and their
                // acknowledgement is not needed before the tile).
                [[maybe_unused]] unsigned long long pf_w0 = 0;
                if constexpr (kProfile) pf_w0 = clock64();
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                if constexpr (kProfile) {
                    pf_tw = clock64();
                    pf_vm += pf_tw - pf_w0;
                }
                // the block's inputs for the fp16 tiles of the next three
                // boundaries (the block before a multiple of 4 kBlk feeds an
                // FFT tile instead); fed-back inputs are tanh values in [-1, 1]
                if (f16 && !openb && t0 + kBlk < L && (t0 & (4 * kBlk - 1)) != 3 * kBlk) {
                    const int slot = (int)(t0 >> kLog2Blk) & 3;
                    int e = 14;
                    if (!chain_block || bnd) {
                        float m = fabsf(xk[0]);
#pragma unroll
                        for (int k = 1; k < kRegs; ++k) m = fmaxf(m, fabsf(xk[k]));
                        e = scale16(wave_max_abs(m));
                    }
                    if (early16) {
                        put_x16<2, kRegs>(X16 + A16::slot_off(slot), xk, e);   // the first half went during the chain
                    } else {
                        put_x16(X16 + A16::slot_off(slot), xk, e);
                        if (lane == 0) smem_ptr(s_ex16)[slot] = e;
                    }
                }
                // p now holds y of the block (lane m's accumulator stopped
                // changing at step m: later pushes carry a zero tap there)
                if (!chain_block) {
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) accw[kWave * k + lane] = nx[k];   // the ring now holds the next block
                }
                if (direct) {
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) xring[(t0 + kWave * k + lane) & xmask] = xk[k];
                }
                if (stage_x) {   // completes the staged input block
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) xst[Un - kBlk + kWave * k + lane] = xk[k];
                }
                if (row_input) {
                    // the next tile reads its input block from the row, and
                    // its transform reaches the LDS copies: store it all now
                    store_block();
                } else {
                    // the matrix-core tile's input and what the next block
                    // stores; the input history (the slot of a consumed
                    // accumulator now holds x), read by later tiles
#pragma unroll
                    for (int k = 0; k < kRegs; ++k) {
                        mxz[15 + kWave * k + lane] = xk[k];
                        myb[kWave * k + lane] = p[k];
                    }
                    FI_GLOBAL float* rb = row + t0;
                    if (t0 + kBlk <= L) {
#pragma unroll
                        for (int k = 0; k < kRegs; ++k) rb[kWave * k + lane] = xk[k];
                    } else {
#pragma unroll
                        for (int k = 0; k < kRegs; ++k)
                            if (t0 + kWave * k + lane < L) rb[kWave * k + lane] = xk[k];
                    }
                }
                __builtin_amdgcn_s_setprio(0);
            }
            // the whole team sees the block's LDS writes and its stores
            if constexpr (kProfile) pf_tc = clock64();
            team_sync_global();
            if constexpr (kProfile) {
                pf_td = clock64();
                pf_chain += pf_tc - pf_tb;
                pf_wait += pf_td - pf_tc;
                if (pf_s0 > pf_tb) {   // the block ran a chain
                    pf_pro += pf_s0 - pf_tb;
                    pf_epi += pf_tc - pf_s1;
                }
            }
            const int64_t i = t0 + kBlk;
            if (i < L) {
                const int U = (int)(i & -i);
                if (U <= d.T) {
                    direct_tile_lds(i, U, xring, xmask, htap, accw, wmask, L);
                } else if (f16 && U <= 2 * kBlk) {
                    // after a chain block the second wavefront has formed
                    // the products of the older inputs during the chain
                    const int np = mm16_count(i, U);
                    if constexpr (RPUSH) {   // every block a chain block, early16 here
                        mm16_tiles<TRI, true>(i, 1, H16, X16, smem_ptr(s_ex16), eh, accw,
                                              reinterpret_cast<FI_SHARED float*>(lbuf), pre16);
                    } else {
                        mm16_tiles<TRI>(i, CLOSED && !open_block(t0) ? 1 : np, H16, X16, smem_ptr(s_ex16), eh, accw,
                                        reinterpret_cast<FI_SHARED float*>(lbuf), pre16);
                    }
                } else {
                    const int q = ilog2(U);
                    const FI_GLOBAL V2* spec =
                        gmem(static_cast<const V2*>(d.spec)) + d.spec_off[q] + c * (int64_t)(U + 2);
                    fft_tile(U, i, row, spec, lbuf, sc, tw, twl, accw, i + kBlk, wmask, L, i == U,
                             stage_x, xst, stage_spec, sst);
                    // the transform buffer reached the matrix-core tile's data
                    // and the tap table: rebuild them
                    if (lds_fft_elems(U < kLdsFftMax ? U : kLdsFftMax) * 8 > kRunMmOff) {
                        team_sync();
                        if (lds_fft_elems(U < kLdsFftMax ? U : kLdsFftMax) * 8 > t4_off) build_taps4(hrow, open_block(i));
                        build_mm(hrow);
                    }
                }
                // The chain wavefront reads the ring and (a block later) the row
                // positions this tile wrote: the other wavefronts' stores must
                // be complete; the chain wavefront's own stores stay in flight
                // (its later loads of the same addresses come after them).
                if (!chain_wave) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                team_sync();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                if constexpr (PROMPT) {
                    // the last block with every input given is done: the
                    // chain's taps replace the triangle's filter copy
                    if (open_block(t0) && !open_block(i)) {
                        build_taps4(hrow, false);
                        team_sync();
                    }
                }
            }
            if constexpr (kProfile) {
                pf_te = clock64();
                if (i < L && chain_wave && lane == 0) {
                    const int q = ilog2(i & -i);
                    s_pf[q] += pf_te - pf_td;
                    s_pf[24 + q] += 1;
                }
            }
            defer_prev = !row_input;
            if constexpr (kProfile) {
                const unsigned long long tf = clock64();
                pf_store += tf - pf_te;
                // the first team's first channel: the block's timeline
                if (bid == 0 && ch == ch0 && chain_wave && lane == 0 && d.prof) {
                    unsigned long long* o =
                        d.prof + kProfHeader + (int64_t)G * kProfSlots + (t0 / kBlk) * kProfSeriesW;
                    o[0] = pf_tb;
                    o[1] = pf_s0;
                    o[2] = pf_s1;
                    o[3] = pf_tw;
                    o[4] = pf_tc;
                    o[5] = pf_td;
                    o[6] = pf_te;
                    o[7] = tf;
                }
            }
        }
        // the last block's outputs (no block follows it)
        if (chain_wave && defer_prev) store_deferred((L - 1) / kBlk * kBlk);
    }
    if constexpr (kProfile) {
        const unsigned long long total = clock64() - pf_t0;
        team_sync();
        if (chain_wave && lane == 0 && d.prof) {
            unsigned long long* o = d.prof + kProfHeader + (int64_t)bid * kProfSlots;
            for (int k = 0; k < kProfSlots; ++k) o[k] = 0;
            unsigned long long segs = 0;
#pragma unroll
            for (int k = 0; k < kRegs; ++k) {
                o[kPfSeg + k] = pf_seg[k];
                segs += pf_seg[k];
            }
            o[kPfTotal] = total;
            o[kPfSetup] = pf_setup;
            o[kPfChainRest] = pf_chain - segs;
            o[kPfWait] = pf_wait;
            o[kPfStore] = pf_store;
            o[kPfBlocks] = pf_blocks;
            o[kPfChannels] = pf_chans;
            o[kPfPrologue] = pf_pro;
            o[kPfEpilogue] = pf_epi;
            o[kPfLoadWait] = pf_vm;
            o[kPfHwChain] = s_hw[0];
            o[kPfHwHelper] = s_hw[1];
            for (int q = 0; q < 24; ++q) {
                o[kPfTile + q] = s_pf[q];
                o[kPfTileCount + q] = s_pf[24 + q];
            }
            if (bid == 0) {
                d.prof[0] = (unsigned long long)G;
                d.prof[1] = kProfSlots;
                d.prof[2] = (unsigned long long)((L + kBlk - 1) / kBlk);
                d.prof[3] = 0;
            }
        }
    }
}

// ======================================================== the layer stack
// The multi-layer model of [FI] "Algoritmo di Inferenza LCSM (Algoritmo 2)":
// layer l mixes its input sequence a^l (a^0 = x) with its filter rho^l, and
// its block maps the mixer output to the next layer's input,
// a^{l+1} = W2^l act(W1^l z^l) (the synthetic MLP + GELU blocks of [FI]
// "Configurazione Sperimentale"); the sampler feeds x[t+1] = a^M[t] +
// sigma noise[t] back.  Channels are (layer, b, c), each a row of the state
// like a single mixer's, with layer l's filter rows.
//
// One position of every layer runs in one launch (k_stack_chain) over P
// workgroups.  Workgroup p owns the slice S_p = [D p / P, D (p+1) / P) of
// each block's hidden units: it forms h_j = act(W1[j] . z) for j in S_p and
// the partial product W2[:, S_p] h_{S_p}, a full D-vector.  The next layer's
// input is the sum of the P partials in slice order, which every workgroup
// forms for itself; every weight is read by exactly one workgroup.  Each
// workgroup also forms the whole mixer output z itself (D fused
// multiply-adds), and parks the inputs of its own slice of channels.
//
// There is no grid barrier: a partial value travels in one 64-bit word with
// a tag naming (run, position, layer) in its high half, stored and loaded as
// relaxed device-scope atomics, and a reader waits until every word it needs
// carries the tag it expects.  Only the parked inputs need ordering: the
// last layer's words are stored after a release fence and read before an
// acquire fence.  Two buffers of words alternate by layer: a workgroup
// overwrites layer l's words (at layer l + 2) only after it has read every
// workgroup's layer l + 1 words, which each wrote after reading layer l.
//
// After the last layer the tile that position t+1 completes runs in the same
// launch when it is small (side <= kChainFuseMax; [FI] "Parallelizzazione
// Cross-Layer (Algoritmo 3)": the tiles of all layers at once), otherwise in
// its own launch.
struct ChainArgs {
    DevState d;
    int64_t B, M;
    const float* w1;     // [M][D][D]: W1^l[j][k], row j = output j
    const float* w2t;    // [M][D][D]: w2t[(l D + j) D + i] = W2^l[i][j]
    const float* x0;     // [B][D]
    const float* noise;  // [B][L][D] or NULL
    float sigma;
    int act;             // 0 GELU, 1 tanh, 2 identity
    float* xnext;        // [B][D]: the next position's input
    float* y;            // [B][L][D]: a^M
    float* x_out;        // [B][L][D] or NULL: x
    unsigned long long* part;   // [2][P][B][D] tagged partial products
    float* hist;         // [M][B][D]: every layer's input at t, until the rows take it
    int* fail;           // set when a wait passes its limit
    int64_t t;
    unsigned tag0;       // the run's tag base: the word of (t, l) carries tag0 + t M + l + 1
    int P;               // workgroups
    int fuse_u;          // side of the fused tile, 0 for none
    int pre;             // 1: stage every layer's accumulator at t in LDS first; 0 on the register
                         // path with B <= kChainPreB: each layer prefetches its own
};

constexpr int kChainThreads = 256;
constexpr long kChainSpinLimit = 1L << 20;   // about a second of polling
constexpr int kChainRegs = 16;               // weights per thread and matrix held in registers
constexpr int kChainPreB = 4;                // batch rows whose accumulators a thread prefetches per layer

__device__ __forceinline__ float stack_act(float v, int act) {
    if (act == 0) return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
    if (act == 1) return tanhf(v);
    return v;
}

__device__ __forceinline__ unsigned long long tagged(unsigned tag, float v) {
    return ((unsigned long long)tag << 32) | __float_as_uint(v);
}

__device__ __forceinline__ void put_word(unsigned long long* w, unsigned long long v) {
    __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long get_word(const unsigned long long* w) {
    return __hip_atomic_load(const_cast<unsigned long long*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// sum_{q < P} value(w[q stride]) in q order, once every word carries `tag`;
// all loads in flight together, stale ones reloaded.  A wait past the limit
// marks the run failed and returns what it has (every wave exits).
__device__ __forceinline__ float gather_sum(const unsigned long long* w, int64_t stride, int P, unsigned tag,
                                            int* fail) {
    // every load unconditional (slots past P read the last workgroup's word
    // and are replaced by a zero that carries the tag): a load under a
    // per-lane branch would wait for the ones before it
    unsigned long long x[kChainMaxWorkgroups];
    const unsigned long long zero = tagged(tag, 0.f);
#pragma unroll
    for (int q = 0; q < kChainMaxWorkgroups; ++q) {
        const unsigned long long v = get_word(w + (q < P ? q : P - 1) * stride);
        x[q] = q < P ? v : zero;
    }
    for (long spins = 0;; ++spins) {
        bool ready = true;
#pragma unroll
        for (int q = 0; q < kChainMaxWorkgroups; ++q) ready &= (unsigned)(x[q] >> 32) == tag;
        if (ready) break;
        if (spins > kChainSpinLimit) {
            __hip_atomic_store(fail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int q = 0; q < kChainMaxWorkgroups; ++q) {
            const unsigned long long v = get_word(w + (q < P ? q : P - 1) * stride);
            x[q] = ((unsigned)(x[q] >> 32) == tag) ? x[q] : (q < P ? v : zero);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kChainMaxWorkgroups; ++q) s += __uint_as_float((unsigned)x[q]);
    return s;
}

// A direct tile of side U over channels [idx0, ...) with stride `step`:
// acc[i + r] += sum_{j<U} x[i-U+j] h[U+r-j], j ascending, the inputs read
// from the channel's row history.  With `last` given, the input at position
// i-1 of channel ch is last[ch] instead of the row's.
__device__ __forceinline__ void tile_direct_range(const DevState& d, int64_t i, int U, int64_t idx0, int64_t step,
                                                  const float* last = nullptr) {
    const int64_t n = d.C * (int64_t)U;
    for (int64_t idx = idx0; idx < n; idx += step) {
        const int64_t ch = idx / U;
        const int r = (int)(idx % U);
        if (i + r >= d.L) continue;
        const int64_t frow = (ch / (d.fset * d.D)) * d.D + ch % d.D;
        const float* hu = d.hT + frow * d.LS + U + r;
        float* row = d.state + ch * d.LS;
        const float* xr = row + (i - U);
        float acc = 0.f;
        for (int j = 0; j < U - 1; ++j) acc = __builtin_fmaf(xr[j], hu[-j], acc);
        acc = __builtin_fmaf(last ? last[ch] : xr[U - 1], hu[1 - U], acc);
        row[i + r] += acc;
    }
}

// tile_direct_range at a side known at compile time, every load in flight
// before the sum (the same products in the same order).
template <int U>
__device__ __forceinline__ void tile_small(const DevState& d, int64_t i, int64_t idx0, int64_t step, const float* last) {
    const int64_t n = d.C * (int64_t)U;
    for (int64_t idx = idx0; idx < n; idx += step) {
        const int64_t ch = idx / U;
        const int r = (int)(idx % U);
        if (i + r >= d.L) continue;
        const int64_t frow = (ch / (d.fset * d.D)) * d.D + ch % d.D;
        const float* hu = d.hT + frow * d.LS + U + r;
        float* row = d.state + ch * d.LS;
        const float* xr = row + (i - U);
        float xv[U], hv[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            xv[j] = j == U - 1 ? last[ch] : xr[j];
            hv[j] = hu[-j];
        }
        const float old = row[i + r];
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < U; ++j) acc = __builtin_fmaf(xv[j], hv[j], acc);
        row[i + r] = old + acc;
    }
}

// The register plan of a slice (REGW): W1's rows of the slice, TPR threads
// per row (a power of two <= 64), KC weights each; W2's columns of the
// slice, one output per thread (IC = 1: D <= kChainThreads), ns weights.
struct ChainRegPlan {
    int tpr, kc, ic;
};

__host__ __device__ inline ChainRegPlan chain_reg_plan(int64_t D, int64_t ns) {
    ChainRegPlan r{0, 0, 0};
    if (ns < 1 || ns > kChainThreads) return r;
    int tpr = 64;
    while (tpr > 1 && (int64_t)tpr * ns > kChainThreads) tpr >>= 1;
    r.tpr = tpr;
    r.kc = (int)((D + tpr - 1) / tpr);
    r.ic = (int)((D + kChainThreads - 1) / kChainThreads);
    return r;
}

__host__ __device__ inline bool chain_regs_fit(int64_t D, int64_t ns) {
    const ChainRegPlan r = chain_reg_plan(D, ns);
    return r.tpr > 0 && r.kc <= kChainRegs && r.ic == 1 && ns <= kChainRegs;
}

// A workgroup barrier that orders LDS only: a thread passes it without
// waiting for its global stores (the tagged words and parked inputs need no
// order among the workgroup's threads; the parked inputs are released by
// every thread's own fence before the last layer's words).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <bool REGW>
__global__ __launch_bounds__(kChainThreads) void k_stack_chain(ChainArgs a) {
    extern __shared__ float sm[];
    const DevState& d = a.d;
    const int p = (int)blockIdx.x, P = a.P, tid = threadIdx.x;
    const int64_t D = d.D, L = d.L, LS = d.LS, t = a.t, B = a.B, M = a.M;
    const int64_t j0 = D * p / P, j1 = D * (p + 1) / P, ns = j1 - j0;
    float* zv = sm;                           // the mixer output of one batch row
    float* hv = sm + D;                       // act(W1 z) on this slice
    float* accp = sm + D + ((ns + 63) & ~63LL);   // [M][B][D] accumulators at t
    if (a.pre) {
        // eight independent loads in flight per thread
        const int64_t n = M * B * D;
        for (int64_t k0 = tid; k0 < n; k0 += 8 * kChainThreads) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t k = k0 + (int64_t)u * kChainThreads;
                v[u] = k < n ? d.state[k * LS + t] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t k = k0 + (int64_t)u * kChainThreads;
                if (k < n) accp[k] = v[u];
            }
        }
    }
    lds_barrier();   // the staged accumulators, for every thread
    // per-layer prefetch of the red cell's operands instead of the staging
    const bool pf = REGW && a.pre == 0 && B <= kChainPreB;
    static_assert(kChainPreB == 4, "the red cell selects among four prefetched rows");
    const ChainRegPlan rp = chain_reg_plan(D, ns);
    const int row = REGW ? tid / rp.tpr : 0, li = REGW ? tid % rp.tpr : 0;
    const unsigned tag_t = a.tag0 + (unsigned)(t * M);
    for (int64_t l = 0; l < M; ++l) {
        const unsigned tag_prev = tag_t + (unsigned)l, tag_mine = tag_prev + 1u;
        const unsigned long long* prev = a.part + ((l - 1) & 1) * P * B * D;
        unsigned long long* mine = a.part + ((l & 1) * P + p) * B * D;
        // this layer's weights of the slice, in flight while the inputs arrive
        // (loaded unconditionally from a clamped in-range index, then zeroed
        // where unused: the zero weights cancel the clamped operands below)
        float w1r[REGW ? kChainRegs : 1], w2r[REGW ? kChainRegs : 1];
        if (REGW) {
            const int64_t rr = row < ns ? row : ns - 1;
#pragma unroll
            for (int m = 0; m < kChainRegs; ++m) {
                const int64_t k = li + (int64_t)m * rp.tpr;
                const bool ok = m < rp.kc && row < ns && k < D;
                const float v = a.w1[(l * D + j0 + rr) * D + (k < D ? k : D - 1)];
                w1r[m] = ok ? v : 0.f;
            }
            const int64_t ic = tid < D ? tid : D - 1;
#pragma unroll
            for (int m = 0; m < kChainRegs; ++m) {
                const bool ok = m < ns && tid < D;
                const float v = a.w2t[(l * D + j0 + (m < ns ? m : ns - 1)) * D + ic];
                w2r[m] = ok ? v : 0.f;
            }
        }
        // the red cell's lag-0 tap and accumulators at t of this thread's
        // channel (c = tid on the register path), in flight with the weights
        float h0r = 0.f, accr[kChainPreB];
        if (pf) {
            const int64_t c = tid < D ? tid : D - 1;
            h0r = d.hT[(l * D + c) * LS];
#pragma unroll
            for (int bb = 0; bb < kChainPreB; ++bb)
                accr[bb] = d.state[((l * B + (bb < B ? bb : B - 1)) * D + c) * LS + t];
        }
        for (int64_t b = 0; b < B; ++b) {
            // the red cell: the tiles' accumulation plus the lag-0 term; the
            // slice owner parks the input (other workgroups may still read
            // the accumulator at t until they have formed their last partial)
            for (int64_t c = tid; c < D; c += kChainThreads) {
                const float v = l == 0 ? (t == 0 ? a.x0[b * D + c] : a.xnext[b * D + c])
                                       : gather_sum(prev + b * D + c, B * D, P, tag_prev, a.fail);
                const int64_t ch = (l * B + b) * D + c;
                float acc, h0;
                if (pf) {
                    acc = b == 0 ? accr[0] : b == 1 ? accr[1] : b == 2 ? accr[2] : accr[3];
                    h0 = h0r;
                } else {
                    acc = a.pre ? accp[ch] : d.state[ch * LS + t];
                    h0 = d.hT[(l * D + c) * LS];
                }
                zv[c] = __builtin_fmaf(h0, v, acc);
                if (c >= j0 && c < j1) {
                    a.hist[ch] = v;
                    if (l == 0 && t == 0 && a.x_out) a.x_out[(b * L) * D + c] = v;
                }
            }
            lds_barrier();
            // the parked inputs of every layer (this row's of the last layer
            // included) before the last layer's words
            if (l == M - 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            if (REGW) {
                // h_j = act(W1[j] . z) for j in the slice
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < kChainRegs; ++m) {
                    const int64_t k = li + (int64_t)m * rp.tpr;
                    s = __builtin_fmaf(w1r[m], zv[k < D ? k : D - 1], s);
                }
                for (int o = rp.tpr >> 1; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
                if (li == 0 && row < ns) hv[row] = stack_act(s, a.act);
                lds_barrier();
                // this slice's share of W2 h, every output (one per thread)
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < kChainRegs; ++m) acc = __builtin_fmaf(w2r[m], hv[m < ns ? m : 0], acc);
                if (tid < D) put_word(mine + b * D + tid, tagged(tag_mine, acc));
            } else {
                const int wave = tid >> 6, lane = tid & 63;
                for (int64_t j = j0 + wave; j < j1; j += kChainThreads / 64) {
                    const float* wr = a.w1 + (l * D + j) * D;
                    float s = 0.f;
#pragma unroll 8
                    for (int64_t k = lane; k < D; k += 64) s = __builtin_fmaf(wr[k], zv[k], s);
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
                    if (lane == 0) hv[j - j0] = stack_act(s, a.act);
                }
                lds_barrier();
                for (int64_t i = tid; i < D; i += kChainThreads) {
                    const float* wc = a.w2t + (l * D + j0) * D + i;
                    float acc = 0.f;
#pragma unroll 8
                    for (int64_t jj = 0; jj < ns; ++jj) acc = __builtin_fmaf(wc[jj * D], hv[jj], acc);
                    put_word(mine + b * D + i, tagged(tag_mine, acc));
                }
            }
            lds_barrier();
        }
    }
    // a^M on this workgroup's slice: the output, and the sampler's next input
    const unsigned long long* last = a.part + ((M - 1) & 1) * P * B * D;
    const unsigned tag_last = tag_t + (unsigned)M;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t c = j0 + tid; c < j1; c += kChainThreads) {
            const float v = gather_sum(last + b * D + c, B * D, P, tag_last, a.fail);
            a.y[(b * L + t) * D + c] = v;
            if (t + 1 < L) {
                const float xn = a.noise ? __builtin_fmaf(a.sigma, a.noise[(b * L + t) * D + c], v) : v;
                a.xnext[b * D + c] = xn;
                if (a.x_out) a.x_out[(b * L + t + 1) * D + c] = xn;
            }
        }
    }
    // every workgroup has formed its last partial, so every accumulator at t
    // has been read: the parked inputs become the rows' histories, and the
    // small tile position t+1 completes reads them on every layer's channels
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    for (int64_t k = tid; k < M * B * ns; k += kChainThreads) {
        const int64_t ch = (k / ns) * D + j0 + k % ns;
        d.state[ch * LS + t] = a.hist[ch];
    }
    const int64_t i0 = (int64_t)p * kChainThreads + tid, st = (int64_t)P * kChainThreads;
    switch (a.fuse_u) {
        case 1: tile_small<1>(d, t + 1, i0, st, a.hist); break;
        case 2: tile_small<2>(d, t + 1, i0, st, a.hist); break;
        case 4: tile_small<4>(d, t + 1, i0, st, a.hist); break;
        case 8: tile_small<8>(d, t + 1, i0, st, a.hist); break;
        case 16: tile_small<16>(d, t + 1, i0, st, a.hist); break;
        case 32: tile_small<32>(d, t + 1, i0, st, a.hist); break;
        default: if (a.fuse_u) tile_direct_range(d, t + 1, a.fuse_u, i0, st, a.hist); break;
    }
}

// A direct tile of side U on every channel, over the whole grid.
__global__ void k_tile_direct(DevState d, int64_t i, int U) {
    tile_direct_range(d, i, U, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
}

// ======================================================= static workspace
// The device memory of fi_conv_static, the entry point for callers that
// cannot allocate: one fixed array per device, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol): it looks up the device address once per device
// and hands that out.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    *bytes = kStaticScratchBytes;
    return hipSuccess;
}

// ================================================================ launchers
static int grid_for(int64_t n, int block, int cap = 65536) {
    int64_t g = (n + block - 1) / block;
    if (g < 1) g = 1;
    return (int)(g < cap ? g : cap);
}

hipError_t launch_transpose(const DevState& d, const void* h, hipStream_t st) {
    const int64_t gy = (d.LS + 63) / 64;
    dim3 grid((unsigned)((d.D + 63) / 64), (unsigned)(gy < 32768 ? gy : 32768));
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
    const size_t lds = (size_t)lds_fft_elems(F) * sizeof(Cx<double>);
    if (lds > 65536) (void)hipFuncSetAttribute((const void*)k_spectra, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int grid = (int)(d.DF < slots ? d.DF : slots);
    V2* spec = static_cast<V2*>(d.spec) + d.spec_off[q];
    hipLaunchKernelGGL(k_spectra, dim3(grid), dim3(kTeam), lds, st, d.hT, d.LS, d.L, d.DF, M, spec,
                       static_cast<Cx<double>*>(scd), scd_stride, static_cast<const Cx<double>*>(twd));
    return hipGetLastError();
}

hipError_t launch_prefix(const DevState& d, hipStream_t st) {
    hipLaunchKernelGGL(k_prefix, dim3(grid_for(d.D, 256, 1 << 30)), dim3(256), 0, st, d.hT, d.LS, d.L, d.D, d.pre);
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

hipError_t launch_step_tile(const DevState& d, int64_t t, const void* x_t, float* y_t, int U, hipStream_t st) {
    const int grid = grid_for(d.C * (int64_t)U, 256);
    if (d.io_bf16)
        hipLaunchKernelGGL((k_step_tile<true>), dim3(grid), dim3(256), 0, st, d.state, d.hT, d.LS, d.L, d.D, d.C, t,
                           x_t, y_t, U);
    else
        hipLaunchKernelGGL((k_step_tile<false>), dim3(grid), dim3(256), 0, st, d.state, d.hT, d.LS, d.L, d.D, d.C, t,
                           x_t, y_t, U);
    return hipGetLastError();
}

int stack_chain_lds_bytes(int64_t B, int64_t D, int64_t M, int P, int* pre) {
    const int64_t ns = (D + P - 1) / P;
    const int64_t base = D + ((ns + 63) & ~63LL);
    const int64_t staged = M * B * D;
    *pre = (base + staged) * 4 <= kChainStageBytes ? 1 : 0;
    return (int)((base + (*pre ? staged : 0)) * 4);
}

hipError_t launch_stack_chain(const DevState& d, const StackChain& sc, const float* x0, const float* noise,
                              float sigma, float* y, float* x_out, int64_t t, unsigned tag0, int fuse_u,
                              hipStream_t st) {
    ChainArgs a{d, sc.B, sc.M, sc.w1, sc.w2t, x0, noise, sigma, sc.act, sc.xnext, y, x_out, sc.part, sc.hist,
                sc.fail, t, tag0, sc.P, fuse_u, 0};
    const bool regw = chain_regs_fit(d.D, (d.D + sc.P - 1) / sc.P);
    size_t lds = (size_t)stack_chain_lds_bytes(sc.B, d.D, sc.M, sc.P, &a.pre);
    if (regw && sc.B <= kChainPreB) {   // each layer prefetches its own accumulators: no staging
        a.pre = 0;
        lds = (size_t)(d.D + ((d.D + sc.P - 1) / sc.P + 63) / 64 * 64) * sizeof(float);
    }
    const void* fn = regw ? (const void*)k_stack_chain<true> : (const void*)k_stack_chain<false>;
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (regw) hipLaunchKernelGGL(k_stack_chain<true>, dim3((unsigned)sc.P), dim3(kChainThreads), lds, st, a);
    else hipLaunchKernelGGL(k_stack_chain<false>, dim3((unsigned)sc.P), dim3(kChainThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_tile_direct(const DevState& d, int64_t i, int U, hipStream_t st) {
    hipLaunchKernelGGL(k_tile_direct, dim3(grid_for(d.C * (int64_t)U, 256)), dim3(256), 0, st, d, i, U);
    return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* src, float* dst, int64_t rows, int64_t cols, int64_t ld, hipStream_t st) {
    const int64_t gy = (ld + 63) / 64;
    dim3 grid((unsigned)((cols + 63) / 64), (unsigned)(gy < 32768 ? gy : 32768));
    hipLaunchKernelGGL((k_transpose<false>), grid, dim3(256), 0, st, static_cast<const void*>(src), dst, rows, cols, ld);
    return hipGetLastError();
}

int tile_fft_lds_bytes() { return (lds_fft_elems(kLdsFftMax) + kTwLds) * (int)sizeof(Cx<float>); }

hipError_t launch_tile(const DevState& d, int64_t i, hipStream_t st) {
    const int U = (int)(i & -i);   // > T: the direct tiles go with the red cell (k_step_tile)
    const int F = U < kLdsFftMax ? U : kLdsFftMax;
    const int grid = (int)(d.C < d.sc_slots ? d.C : d.sc_slots);
    hipLaunchKernelGGL(k_tile_fft, dim3(grid), dim3(kTeam), (size_t)(lds_fft_elems(F) + kTwLds) * sizeof(Cx<float>), st,
                       d, i, U);
    return hipGetLastError();
}

int run_lds_bytes(const DevState& d) { return run_lds_floats(d) * (int)sizeof(float); }

// The persistent pass of a mode (kRunOpen, kRunClosed, kRunPrompted) and
// storage type.
static const void* run_kernel(const DevState& d, int mode) {
    if (mode == kRunClosed) return d.io_bf16 ? (const void*)k_run<true, true> : (const void*)k_run<true, false>;
    if (mode == kRunPrompted)
        return d.io_bf16 ? (const void*)k_run<true, true, true> : (const void*)k_run<true, false, true>;
    return d.io_bf16 ? (const void*)k_run<false, true> : (const void*)k_run<false, false>;
}

int run_max_blocks_per_cu(const DevState& d, int mode) {
    int nb = 0;
    const void* fn = run_kernel(d, mode);
    const int lds = run_lds_bytes(d);
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kTeam, lds) != hipSuccess) return 0;
    return nb;
}

hipError_t launch_run(const DevState& d, const void* x_in, int mode, int64_t prompt, float* y, void* x_out,
                      int grid, hipStream_t st) {
    RunArgs a{d, x_in, y, x_out, prompt};
    const size_t lds = (size_t)run_lds_bytes(d);
    hipLaunchKernelGGL(reinterpret_cast<void (*)(RunArgs)>(const_cast<void*>(run_kernel(d, mode))), dim3(grid),
                       dim3(kTeam), lds, st, a);
    return hipGetLastError();
}

}  // namespace fi
