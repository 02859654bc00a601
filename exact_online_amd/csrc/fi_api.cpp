// fi_api.cpp -- host side of the C ABI declared in include/fi.h: argument
// validation, device allocation, the one-time precompute in fi_create, and the
// dispatch of the online step / the persistent pass.
//
// [FI] = the page "Flash Inference: Inferenza in Tempo Quasi-Lineare per
// Modelli di Sequenza a Convoluzione Lunga e Oltre" (lowest.today summary of
// arXiv 2410.12982).
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstring>
#include <new>

#include "fi.h"
#include "fi_internal.h"

using fi::DevState;

struct fi_handle {
    DevState d;
    hipStream_t stream;
    int64_t pos;
    int dirty;         // accumulators need zeroing before the next fi_step
    int run_grid[fi::kRunModes];   // persistent-pass grid per mode (open, closed, prompted)
};

namespace {

thread_local char g_errbuf[256];
thread_local hipError_t g_last_hip = hipSuccess;

int hip_fail(hipError_t e) {
    g_last_hip = e;
    return e == hipErrorOutOfMemory ? FI_ERR_NOMEM : FI_ERR_HIP;
}

#define FI_HIP(expr)                                 \
    do {                                             \
        hipError_t e_ = (expr);                      \
        if (e_ != hipSuccess) return hip_fail(e_);   \
    } while (0)

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) { return 63 - __builtin_clzll((unsigned long long)v); }

// Largest tile side for positions i in [1, L): the largest power of two < L.
int64_t max_tile(int64_t L) { return L <= 1 ? 0 : ((int64_t)1 << ilog2(L - 1)); }

void free_state(DevState &d) {
    if (d.hT) (void)hipFree(d.hT);
    if (d.state) (void)hipFree(d.state);
    if (d.spec) (void)hipFree(d.spec);
    if (d.twf) (void)hipFree(d.twf);
    if (d.scratch) (void)hipFree(d.scratch);
    d.hT = nullptr;
    d.state = nullptr;
    d.spec = nullptr;
    d.twf = nullptr;
    d.scratch = nullptr;
}

template <typename T>
hipError_t dalloc(T **p, size_t bytes) {
    void *v = nullptr;
    hipError_t e = hipMalloc(&v, bytes < 256 ? 256 : bytes);
    *p = static_cast<T *>(v);
    return e;
}

int build(fi_handle *s, const void *h) {
    DevState &d = s->d;
    hipStream_t st = s->stream;
    const int64_t umax = max_tile(d.L);
    // FFT levels: T < U <= umax
    int64_t spec_total = 0;
    int smax = 1;
    for (int q = 0; q < fi::kMaxLevels; ++q) d.spec_off[q] = -1;
    d.umax_fft = 0;
    for (int q = 0; ((int64_t)1 << q) <= umax; ++q) {
        const int64_t U = (int64_t)1 << q;
        if (U <= d.T) continue;
        d.spec_off[q] = spec_total;
        spec_total += d.D * (U + 2);
        d.umax_fft = (int)U;
        smax = q;
    }
    d.F = d.umax_fft > 0 ? (d.umax_fft < fi::kLdsFftMax ? d.umax_fft : fi::kLdsFftMax) : 1;
    // FFT region of the persistent pass: the largest LDS transform, or the
    // staging of a tile's input (4U bytes) and, for U <= 1024, its spectrum
    // (8 (U + 2) bytes) behind that tile's own transform buffer.  Above every
    // staging area: the data of the tile of side kRunBlock (done on the
    // matrix cores), then the chain's tap table at the top of the region
    // (both rebuilt after a tile whose transform reaches them).
    int staged = 0;
    for (int q = 0; q < fi::kMaxLevels; ++q) {
        if (d.spec_off[q] < 0) continue;
        const int U = 1 << q;
        int need = 0;
        if (U == fi::kRunBlock) need = 0;   // the matrix-core tile: its own area
        else if (U <= 1024) need = fi::lds_fft_elems(U) * 8 + 4 * U + 8 * (U + 2);
        else if (U <= 2048) need = fi::lds_fft_elems(U) * 8 + 4 * U;
        if (need > staged) staged = need;
    }
    d.mm_off = (staged + 15) / 16 * 16;
    d.fftreg = fi::lds_fft_elems(d.F) * 8;
    if (d.mm_off + fi::kMmBytes + fi::kTapTableBytes > d.fftreg)
        d.fftreg = d.mm_off + fi::kMmBytes + fi::kTapTableBytes;

    FI_HIP(dalloc(&d.hT, (size_t)(d.D * d.LS) * sizeof(float)));
    FI_HIP(dalloc(&d.state, (size_t)(d.C * d.LS) * sizeof(float)));
    FI_HIP(dalloc(&d.spec, (size_t)(spec_total > 0 ? spec_total : 1) * 8));
    // twiddles up to 2 umax points (the untangle of the largest tiles uses
    // w_2U^k)
    smax += 1;
    FI_HIP(dalloc(&d.twf, (size_t)((int64_t)2 << smax) * 8));

    // persistent-pass grid: every resident wavefront slot, at most one per channel
    int dev = 0, ncu = 0;
    FI_HIP(hipGetDevice(&dev));
    FI_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    int64_t slots = 0;
    for (int mode = 0; mode < fi::kRunModes; ++mode) {
        int nb = fi::run_max_blocks_per_cu(d, mode);
        if (nb < 1) nb = 1;
        int64_t g = (int64_t)nb * ncu;
        if (g > d.C) g = d.C;
        s->run_grid[mode] = (int)g;
        if (g > slots) slots = g;
    }
    // scratch for FFT tiles larger than LDS: one slot per resident wavefront
    // of the persistent pass (its largest grid), and as many for the per-step
    // tile kernel
    d.sc_slots = slots;
    d.sc_stride = d.umax_fft > fi::kLdsFftMax ? d.umax_fft : 0;
    if (d.sc_stride > 0) FI_HIP(dalloc(&d.scratch, (size_t)(slots * d.sc_stride) * 8));

    FI_HIP(fi::launch_transpose(d, h, st));
    void *twd = nullptr;
    FI_HIP(dalloc(&twd, (size_t)((int64_t)2 << smax) * 16));
    hipError_t e = fi::launch_twiddles(twd, d.twf, smax, st);
    void *scd = nullptr;
    int64_t scd_slots = d.D < 1024 ? d.D : 1024;
    if (e == hipSuccess && d.umax_fft > fi::kLdsFftMax)
        e = dalloc(&scd, (size_t)(scd_slots * d.umax_fft) * 16);
    for (int q = 0; e == hipSuccess && q < fi::kMaxLevels; ++q)
        if (d.spec_off[q] >= 0) e = fi::launch_spectra(d, q, scd, d.umax_fft, scd_slots, twd, st);
    if (e == hipSuccess) e = fi::launch_zero(d.state, d.C * d.LS, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (scd) (void)hipFree(scd);
    (void)hipFree(twd);
    if (e != hipSuccess) return hip_fail(e);
    return FI_OK;
}

}  // namespace

extern "C" {

int fi_create(const fi_config *cfg, const void *h, fi_handle **out) {
    if (out) *out = nullptr;
    if (!cfg || !h || !out) return FI_ERR_INVALID;
    if (cfg->B < 1 || cfg->D < 1 || cfg->L < 1) return FI_ERR_INVALID;
    if (cfg->io_dtype != FI_F32 && cfg->io_dtype != FI_BF16) return FI_ERR_INVALID;
    int T = cfg->small_tile_max == 0 ? FI_DEFAULT_SMALL_TILE_MAX : cfg->small_tile_max;
    if (!is_pow2(T) || T < 64 || T > 256) return FI_ERR_INVALID;
    // sizes: every element count must fit comfortably in int64 and the
    // per-channel position index in int32 kernels' loop bounds
    const int64_t lim = (int64_t)1 << 31;
    if (cfg->B >= lim || cfg->D >= lim || cfg->L >= lim) return FI_ERR_INVALID;
    if (cfg->L > FI_MAX_L) return FI_ERR_UNSUPPORTED;
    const int64_t LS = (cfg->L + 63) / 64 * 64;
    const int64_t C = cfg->B * cfg->D;
    if (C >= lim || (C > 0 && LS > ((int64_t)1 << 46) / C)) return FI_ERR_INVALID;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        g_last_hip = hipErrorNoDevice;
        return FI_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return FI_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return FI_ERR_UNSUPPORTED;

    fi_handle *s = new (std::nothrow) fi_handle();
    if (!s) return FI_ERR_NOMEM;
    std::memset(&s->d, 0, sizeof(s->d));
    DevState &d = s->d;
    d.B = cfg->B;
    d.D = cfg->D;
    d.L = cfg->L;
    d.C = C;
    d.LS = LS;
    d.T = T;
    d.W = fi::kRunBlock;        // LDS accumulator ring of the persistent pass: one block
    d.XR = T >= fi::kRunBlock ? T : 0;   // LDS ring of recent inputs, only for its direct tiles
    d.io_bf16 = cfg->io_dtype == FI_BF16;
    s->stream = static_cast<hipStream_t>(cfg->stream);
    s->pos = 0;
    s->dirty = 0;
    int rc = build(s, h);
    if (rc != FI_OK) {
        (void)hipStreamSynchronize(s->stream);
        free_state(d);
        delete s;
        return rc;
    }
    *out = s;
    return FI_OK;
}

int fi_step(fi_handle *s, const void *x_t, float *y_t) {
    if (!s || !x_t || !y_t) return FI_ERR_INVALID;
    if (s->pos >= s->d.L) return FI_ERR_STATE;
    const int64_t t = s->pos;
    if (s->dirty) {
        FI_HIP(fi::launch_zero(s->d.state, s->d.C * s->d.LS, s->stream));
        s->dirty = 0;
    }
    const int64_t i = t + 1;
    const int64_t U = i & -i;
    if (i < s->d.L && U <= s->d.T) {
        // one launch: the red cell and the direct tile
        FI_HIP(fi::launch_step_tile(s->d, t, x_t, y_t, (int)U, s->stream));
    } else {
        FI_HIP(fi::launch_step(s->d, t, x_t, y_t, s->stream));
        if (i < s->d.L) FI_HIP(fi::launch_tile(s->d, i, s->stream));
    }
    s->pos = t + 1;
    return FI_OK;
}

int fi_run_closed_loop(fi_handle *s, const void *x_in, int32_t fb, float *y, void *x_out) {
    if (!s || !x_in || !y) return FI_ERR_INVALID;
    if (fb != FI_FEEDBACK_NONE && fb != FI_FEEDBACK_TANH) return FI_ERR_INVALID;
    if (s->pos != 0) return FI_ERR_STATE;
    const int mode = fb == FI_FEEDBACK_TANH ? fi::kRunClosed : fi::kRunOpen;
    // the persistent pass zeroes the accumulator rows it owns itself
    FI_HIP(fi::launch_run(s->d, x_in, mode, 0, y, x_out, s->run_grid[mode], s->stream));
    s->pos = s->d.L;
    s->dirty = 1;
    return FI_OK;
}

int fi_run_prompted(fi_handle *s, const void *x_prompt, int64_t p, float *y, void *x_out) {
    if (!s || !x_prompt || !y) return FI_ERR_INVALID;
    if (p < 1 || p > s->d.L) return FI_ERR_INVALID;
    if (s->pos != 0) return FI_ERR_STATE;
    // p = L is the open loop and p = 1 the closed loop (same layouts)
    const int mode = p == s->d.L ? fi::kRunOpen : p == 1 ? fi::kRunClosed : fi::kRunPrompted;
    FI_HIP(fi::launch_run(s->d, x_prompt, mode, p, y, x_out, s->run_grid[mode], s->stream));
    s->pos = s->d.L;
    s->dirty = 1;
    return FI_OK;
}

int fi_reset(fi_handle *s) {
    if (!s) return FI_ERR_INVALID;
    s->pos = 0;
    s->dirty = 1;  // zeroed by the next fi_step (fi_run_closed_loop zeroes its own rows)
    return FI_OK;
}

void fi_destroy(fi_handle *s) {
    if (!s) return;
    (void)hipStreamSynchronize(s->stream);
    free_state(s->d);
    delete s;
}

int64_t fi_position(const fi_handle *s) { return s ? s->pos : -1; }

const char *fi_strerror(int status) {
    switch (status) {
        case FI_OK: return "ok";
        case FI_ERR_INVALID: return "invalid argument";
        case FI_ERR_NOMEM: return "device out of memory";
        case FI_ERR_STATE: return "call not allowed at the handle's position";
        case FI_ERR_UNSUPPORTED: return "unsupported (needs a gfx950 device)";
        case FI_ERR_HIP:
            std::snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(g_last_hip));
            return g_errbuf;
        default: return "unknown status";
    }
}

int fi_tile_at(int64_t L, int64_t i, fi_tile *out) {
    if (!out || L < 2 || i < 1 || i >= L) return FI_ERR_INVALID;
    const int64_t U = i & -i;
    out->U = U;
    out->in_lo = i - U;
    out->in_hi = i;
    out->out_lo = i;
    out->out_hi = i + U < L ? i + U : L;
    return FI_OK;
}

}  // extern "C"
