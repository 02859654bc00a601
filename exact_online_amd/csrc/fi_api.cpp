// fi_api.cpp -- host side of the C ABI declared in include/fi.h: argument
// validation, device allocation, the one-time precompute in fi_create, and the
// dispatch of the online step / the persistent pass.
//
// [FI] = the page "Flash Inference: Inferenza in Tempo Quasi-Lineare per
// Modelli di Sequenza a Convoluzione Lunga e Oltre" (lowest.today summary of
// arXiv 2410.12982).
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "fi.h"
#include "fi_internal.h"
#if FI_PROFILE
#include "fi_profile.h"
#endif

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
    if (d.pre) (void)hipFree(d.pre);
    d.pre = nullptr;
    if (d.state) (void)hipFree(d.state);
    if (d.spec) (void)hipFree(d.spec);
    if (d.twf) (void)hipFree(d.twf);
    if (d.scratch) (void)hipFree(d.scratch);
    if (d.prof) (void)hipFree(d.prof);
    d.prof = nullptr;
    d.hT = nullptr;
    d.state = nullptr;
    d.spec = nullptr;
    d.twf = nullptr;
    d.scratch = nullptr;
}

// A failed hipMalloc also leaves its error as the thread's "last error",
// which the next launch check (hipGetLastError) would then report as its own:
// take it back here, so a rejected fi_create leaves no trace for later calls.
template <typename T>
hipError_t dalloc(T **p, size_t bytes) {
    void *v = nullptr;
    hipError_t e = hipMalloc(&v, bytes < 256 ? 256 : bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        v = nullptr;
    }
    *p = static_cast<T *>(v);
    return e;
}

// Sizes of a handle's device buffers (bytes) and its persistent-pass grid.
struct Plan {
    size_t hT, pre, state, spec, twf, scratch, twd, scd, prof;
    int smax;            // twiddle tables up to 2^smax points
    int64_t scd_slots;   // fp64 spectrum scratch slots (levels above LDS only)
};

// Fills the layout fields of s->d (levels, spectra offsets, grid, scratch
// slots) and the buffer sizes; no device memory is touched.
int plan(fi_handle *s, Plan &pl) {
    DevState &d = s->d;
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
        spec_total += d.DF * (U + 2);
        d.umax_fft = (int)U;
        smax = q;
    }
    d.F = d.umax_fft > 0 ? (d.umax_fft < fi::kLdsFftMax ? d.umax_fft : fi::kLdsFftMax) : 1;
    // the persistent pass's LDS FFT / staging region has a fixed layout
    d.mm_off = fi::kRunMmOff;
    d.fftreg = fi::kRunFftReg;
    // twiddles up to 2 umax points (the untangle of the largest tiles uses
    // w_2U^k)
    smax += 1;
    pl.smax = smax;
    pl.hT = (size_t)(d.DF * d.LS) * sizeof(float);
    pl.pre = (size_t)(d.D * fi::kRunBlock) * sizeof(float);
    pl.state = (size_t)(d.C * d.LS) * sizeof(float);
    pl.spec = (size_t)(spec_total > 0 ? spec_total : 1) * 8;
    pl.twf = (size_t)((int64_t)2 << smax) * 8;
    pl.twd = (size_t)((int64_t)2 << smax) * 16;

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
    pl.scratch = (size_t)(slots * d.sc_stride) * 8;
    pl.scd_slots = d.DF < 1024 ? d.DF : 1024;
    pl.scd = d.umax_fft > fi::kLdsFftMax ? (size_t)(pl.scd_slots * d.umax_fft) * 16 : 0;
    pl.prof = 0;
    if (fi::kProfile) {
        // header, one slot row per team of the largest grid, one entry per block
        d.prof_n = fi::kProfHeader + slots * fi::kProfSlots +
                   ((d.L + fi::kRunBlock - 1) / fi::kRunBlock) * fi::kProfSeriesW;
        pl.prof = (size_t)d.prof_n * 8;
    }
    return FI_OK;
}

// The one-time precompute on the stream: filter rows, tap prefix sums,
// twiddles, per-level spectra, and zeroed accumulator rows.
hipError_t init_state(const DevState &d, const Plan &pl, const void *h, void *twd, void *scd, hipStream_t st) {
    hipError_t e = fi::launch_transpose(d, h, st);
    if (e == hipSuccess) e = fi::launch_prefix(d, st);
    if (e == hipSuccess) e = fi::launch_twiddles(twd, d.twf, pl.smax, st);
    for (int q = 0; e == hipSuccess && q < fi::kMaxLevels; ++q)
        if (d.spec_off[q] >= 0) e = fi::launch_spectra(d, q, scd, d.umax_fft, pl.scd_slots, twd, st);
    if (e == hipSuccess) e = fi::launch_zero(d.state, d.C * d.LS, st);
    return e;
}

int build(fi_handle *s, const void *h) {
    DevState &d = s->d;
    hipStream_t st = s->stream;
    Plan pl;
    const int rc = plan(s, pl);
    if (rc != FI_OK) return rc;
    FI_HIP(dalloc(&d.hT, pl.hT));
    FI_HIP(dalloc(&d.pre, pl.pre));
    FI_HIP(dalloc(&d.state, pl.state));
    FI_HIP(dalloc(&d.spec, pl.spec));
    FI_HIP(dalloc(&d.twf, pl.twf));
    if (pl.scratch > 0) FI_HIP(dalloc(&d.scratch, pl.scratch));
    if (pl.prof > 0) {
        FI_HIP(dalloc(&d.prof, pl.prof));
        FI_HIP(hipMemsetAsync(d.prof, 0, pl.prof, st));
    }
    void *twd = nullptr, *scd = nullptr;
    FI_HIP(dalloc(&twd, pl.twd));
    hipError_t e = hipSuccess;
    if (pl.scd > 0) e = dalloc(&scd, pl.scd);
    if (e == hipSuccess) e = init_state(d, pl, h, twd, scd, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (scd) (void)hipFree(scd);
    (void)hipFree(twd);
    if (e != hipSuccess) return hip_fail(e);
    return FI_OK;
}

// The int a caller put in an enum-typed field or argument, read as its
// bytes: a value outside the enumeration is not one the enum type may hold,
// so it is never loaded as that type.
template <typename E>
int raw_int(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "an int-sized enum");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

// Validation shared by fi_create and fi_conv_static; fills the handle's
// configuration fields.
int configure(const fi_config *cfg, fi_handle *s) {
    if (cfg->B < 1 || cfg->D < 1 || cfg->L < 1) return FI_ERR_INVALID;
    const int dt = raw_int(cfg->io_dtype);   // the caller may store any int there
    if (dt != FI_F32 && dt != FI_BF16) return FI_ERR_INVALID;
    int T = cfg->small_tile_max;
    if (T == 0) {
        // left to the library: the environment's FI_SMALL_TILE_MAX (an
        // ablation override) or the default
        const char *env = std::getenv("FI_SMALL_TILE_MAX");
        T = env && *env ? std::atoi(env) : FI_DEFAULT_SMALL_TILE_MAX;
    }
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

    std::memset(&s->d, 0, sizeof(s->d));
    DevState &d = s->d;
    d.B = cfg->B;
    d.D = cfg->D;
    d.L = cfg->L;
    d.C = C;
    d.LS = LS;
    d.fset = cfg->B;   // one filter set, shared by every batch row
    d.DF = cfg->D;
    d.T = T;
    d.W = fi::kRunBlock;        // LDS accumulator ring of the persistent pass: one block
    d.XR = T >= fi::kRunBlock ? T : 0;   // LDS ring of recent inputs, only for its direct tiles
    d.io_bf16 = dt == FI_BF16;
    s->stream = static_cast<hipStream_t>(cfg->stream);
    s->pos = 0;
    s->dirty = 0;
    return FI_OK;
}

}  // namespace

extern "C" {

int fi_create(const fi_config *cfg, const void *h, fi_handle **out) {
    if (out) *out = nullptr;
    if (!cfg || !h || !out) return FI_ERR_INVALID;
    fi_handle *s = new (std::nothrow) fi_handle();
    if (!s) return FI_ERR_NOMEM;
    int rc = configure(cfg, s);
    if (rc != FI_OK) {
        delete s;
        return rc;
    }
    rc = build(s, h);
    if (rc != FI_OK) {
        (void)hipStreamSynchronize(s->stream);
        free_state(s->d);
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

int fi_run_closed_loop(fi_handle *s, const void *x_in, fi_feedback fb, float *y, void *x_out) {
    if (!s || !x_in || !y) return FI_ERR_INVALID;
    const int fbv = raw_int(fb);   // the caller may pass any int
    if (fbv != FI_FEEDBACK_NONE && fbv != FI_FEEDBACK_TANH) return FI_ERR_INVALID;
    if (s->pos != 0) return FI_ERR_STATE;
    const int mode = fbv == FI_FEEDBACK_TANH ? fi::kRunClosed : fi::kRunOpen;
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

int fi_conv_static(const fi_config *cfg, const void *h, const void *x_in, fi_feedback fb, float *y,
                   void *x_out) {
    if (!cfg || !h || !x_in || !y) return FI_ERR_INVALID;
    const int fbv = raw_int(fb);   // the caller may pass any int
    if (fbv != FI_FEEDBACK_NONE && fbv != FI_FEEDBACK_TANH) return FI_ERR_INVALID;
    fi_handle s;   // host-side only: its device buffers are carved from the workspace
    int rc = configure(cfg, &s);
    if (rc != FI_OK) return rc;
    Plan pl;
    rc = plan(&s, pl);
    if (rc != FI_OK) return rc;
    DevState &d = s.d;
    // carve every buffer, 256-byte aligned, out of the device's workspace
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    const size_t o_hT = take(pl.hT), o_pre = take(pl.pre), o_state = take(pl.state), o_spec = take(pl.spec),
                 o_twf = take(pl.twf), o_sc = take(pl.scratch), o_twd = take(pl.twd), o_scd = take(pl.scd);
    void *base = nullptr;
    size_t cap = 0;
    FI_HIP(fi::static_scratch(&base, &cap));
    if (off > cap) return FI_ERR_UNSUPPORTED;   // beyond FI_STATIC_WORKSPACE_BYTES
    char *b = static_cast<char *>(base);
    d.hT = reinterpret_cast<float *>(b + o_hT);
    d.pre = reinterpret_cast<float *>(b + o_pre);
    d.state = reinterpret_cast<float *>(b + o_state);
    d.spec = b + o_spec;
    d.twf = b + o_twf;
    d.scratch = pl.scratch > 0 ? b + o_sc : nullptr;
    d.prof = nullptr;
    FI_HIP(init_state(d, pl, h, b + o_twd, pl.scd > 0 ? b + o_scd : nullptr, s.stream));
    const int mode = fbv == FI_FEEDBACK_TANH ? fi::kRunClosed : fi::kRunOpen;
    FI_HIP(fi::launch_run(d, x_in, mode, 0, y, x_out, s.run_grid[mode], s.stream));
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
        case FI_ERR_UNSUPPORTED:
            return "unsupported (needs a gfx950 device; L <= FI_MAX_L; for fi_conv_static, buffers within "
                   "FI_STATIC_WORKSPACE_BYTES)";
        case FI_ERR_HIP:
            std::snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(g_last_hip));
            return g_errbuf;
        default: return "unknown status";
    }
}

// ------------------------------------------------------------------ stack
}  // extern "C"

struct fi_stack {
    fi_handle h;   // the M B D channels (layer, b, c); filter rows per layer
    fi::StackChain sc;
    float *w1, *w2t, *xnext, *hist;
    void *part;    // tagged partial products
    void *sync;    // the failure mark
    uint32_t tag0; // the next run's tag base
};

namespace {
void free_stack(fi_stack *s) {
    free_state(s->h.d);
    for (void *p : {(void *)s->w1, (void *)s->w2t, (void *)s->xnext, s->part, (void *)s->hist, s->sync})
        if (p) (void)hipFree(p);
    s->w1 = s->w2t = s->xnext = s->hist = nullptr;
    s->part = s->sync = nullptr;
}

int build_stack(fi_stack *s, const float *rho, const float *w1, const float *w2) {
    DevState &d = s->h.d;
    hipStream_t st = s->h.stream;
    Plan pl;
    int rc = plan(&s->h, pl);
    if (rc != FI_OK) return rc;
    FI_HIP(dalloc(&d.hT, pl.hT));
    FI_HIP(dalloc(&d.pre, pl.pre));
    FI_HIP(dalloc(&d.state, pl.state));
    FI_HIP(dalloc(&d.spec, pl.spec));
    FI_HIP(dalloc(&d.twf, pl.twf));
    if (pl.scratch > 0) FI_HIP(dalloc(&d.scratch, pl.scratch));
    fi::StackChain &sc = s->sc;
    const int64_t D = d.D, L = d.L, M = sc.M;
    FI_HIP(dalloc(&s->w1, (size_t)(M * D * D) * sizeof(float)));
    FI_HIP(dalloc(&s->w2t, (size_t)(M * D * D) * sizeof(float)));
    FI_HIP(dalloc(&s->xnext, (size_t)(sc.B * D) * sizeof(float)));
    const size_t part_bytes = (size_t)(2 * sc.P * sc.B * D) * sizeof(unsigned long long);
    FI_HIP(dalloc(&s->part, part_bytes));
    FI_HIP(dalloc(&s->hist, (size_t)(M * sc.B * D) * sizeof(float)));
    FI_HIP(dalloc(&s->sync, 256));
    FI_HIP(hipMemcpyAsync(s->w1, w1, (size_t)(M * D * D) * sizeof(float), hipMemcpyDeviceToDevice, st));
    for (int64_t l = 0; l < M; ++l) {
        // layer l's filter rows, and W2 with its output index innermost
        FI_HIP(fi::launch_transpose_f32(rho + l * L * D, d.hT + l * D * d.LS, L, D, d.LS, st));
        FI_HIP(fi::launch_transpose_f32(w2 + l * D * D, s->w2t + l * D * D, D, D, D, st));
    }
    // tag 0 is never awaited: cleared words are never taken for a partial
    FI_HIP(fi::launch_zero(static_cast<float *>(s->part), (int64_t)(part_bytes / sizeof(float)), st));
    FI_HIP(fi::launch_zero(static_cast<float *>(s->sync), 64, st));
    sc.w1 = s->w1;
    sc.w2t = s->w2t;
    sc.xnext = s->xnext;
    sc.part = static_cast<unsigned long long *>(s->part);
    sc.hist = s->hist;
    sc.fail = static_cast<int *>(s->sync);
    void *twd = nullptr, *scd = nullptr;
    FI_HIP(dalloc(&twd, pl.twd));
    hipError_t e = hipSuccess;
    if (pl.scd > 0) e = dalloc(&scd, pl.scd);
    if (e == hipSuccess) e = fi::launch_twiddles(twd, d.twf, pl.smax, st);
    for (int q = 0; e == hipSuccess && q < fi::kMaxLevels; ++q)
        if (d.spec_off[q] >= 0) e = fi::launch_spectra(d, q, scd, d.umax_fft, pl.scd_slots, twd, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (scd) (void)hipFree(scd);
    (void)hipFree(twd);
    if (e != hipSuccess) return hip_fail(e);
    return FI_OK;
}
}  // namespace

extern "C" {

int fi_stack_create(const fi_stack_config *cfg, const float *rho, const float *w1, const float *w2,
                    fi_stack **out) {
    if (out) *out = nullptr;
    if (!cfg || !rho || !w1 || !w2 || !out) return FI_ERR_INVALID;
    const int act = raw_int(cfg->act);
    if (act != FI_ACT_GELU && act != FI_ACT_TANH && act != FI_ACT_IDENTITY) return FI_ERR_INVALID;
    const int64_t lim = (int64_t)1 << 31;
    if (cfg->M < 1 || cfg->B < 1 || cfg->M >= lim || cfg->B >= lim || cfg->M > lim / cfg->B) return FI_ERR_INVALID;
    if (cfg->D > fi::kChainMaxD) return FI_ERR_UNSUPPORTED;   // a D-vector of a block in LDS
    if (cfg->L > 0 && cfg->M > fi::kChainMaxTags / cfg->L) return FI_ERR_UNSUPPORTED;   // L M tags per run
    fi_config c;
    std::memset(&c, 0, sizeof(c));
    c.B = cfg->M * cfg->B;   // rows (layer, b)
    c.D = cfg->D;
    c.L = cfg->L;
    c.io_dtype = FI_F32;
    c.stream = cfg->stream;
    c.small_tile_max = cfg->small_tile_max;
    fi_stack *s = new (std::nothrow) fi_stack();
    if (!s) return FI_ERR_NOMEM;
    int rc = configure(&c, &s->h);
    if (rc != FI_OK) {
        delete s;
        return rc;
    }
    s->sc.B = cfg->B;
    s->sc.M = cfg->M;
    s->sc.act = act;
    s->sc.P = (int)(cfg->D < fi::kChainMaxWorkgroups ? cfg->D : fi::kChainMaxWorkgroups);
    s->tag0 = 0;
    s->h.d.fset = cfg->B;            // B rows per layer share its filter rows
    s->h.d.DF = cfg->M * cfg->D;     // filter rows: (layer, c)
    rc = build_stack(s, rho, w1, w2);
    if (rc != FI_OK) {
        (void)hipStreamSynchronize(s->h.stream);
        free_stack(s);
        delete s;
        return rc;
    }
    *out = s;
    return FI_OK;
}

int fi_stack_run(fi_stack *s, const float *x0, const float *noise, float sigma, float *y, float *x_out) {
    if (!s || !x0 || !y) return FI_ERR_INVALID;
    const DevState &d = s->h.d;
    hipStream_t st = s->h.stream;
    // a barrier of an earlier run that waited past its limit fails the handle
    int failed = 0;
    FI_HIP(hipMemcpyAsync(&failed, s->sc.fail, sizeof(int), hipMemcpyDeviceToHost, st));
    FI_HIP(hipStreamSynchronize(st));
    if (failed) return hip_fail(hipErrorLaunchTimeOut);
    // the tiles add into the rows; this run's words carry tags after the
    // last run's
    FI_HIP(fi::launch_zero(d.state, d.C * d.LS, st));
    const uint32_t tag0 = s->tag0;
    s->tag0 = tag0 + (uint32_t)(d.L * s->sc.M);
    const int64_t fuse_max = d.T < fi::kChainFuseMax ? d.T : fi::kChainFuseMax;
    for (int64_t t = 0; t < d.L; ++t) {
        const int64_t i = t + 1;
        const int64_t U = i & -i;
        const bool tile = i < d.L;
        const int fuse = tile && U <= fuse_max ? (int)U : 0;
        FI_HIP(fi::launch_stack_chain(d, s->sc, x0, noise, sigma, y, x_out, t, tag0, fuse, st));
        if (!tile || fuse) continue;
        if (U <= d.T) FI_HIP(fi::launch_tile_direct(d, i, (int)U, st));
        else FI_HIP(fi::launch_tile(d, i, st));
    }
    return FI_OK;
}

void fi_stack_destroy(fi_stack *s) {
    if (!s) return;
    (void)hipStreamSynchronize(s->h.stream);
    free_stack(s);
    delete s;
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

#if FI_PROFILE
int64_t fi_profile_read(fi_handle *s, uint64_t *out, int64_t cap) {
    if (!s || !out || cap < 0) return FI_ERR_INVALID;
    if (!s->d.prof) return 0;
    if (hipStreamSynchronize(s->stream) != hipSuccess) return FI_ERR_HIP;
    const int64_t n = cap < s->d.prof_n ? cap : s->d.prof_n;
    if (n > 0 && hipMemcpy(out, s->d.prof, (size_t)n * 8, hipMemcpyDeviceToHost) != hipSuccess) return FI_ERR_HIP;
    return s->d.prof_n;
}
#endif

}  // extern "C"
