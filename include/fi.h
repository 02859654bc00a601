/*
 * fi.h -- exact online causal long convolution on AMD MI355X (gfx950).
 *
 * Citations name the web page "Flash Inference: Inferenza in Tempo
 * Quasi-Lineare per Modelli di Sequenza a Convoluzione Lunga e Oltre"
 * (lowest.today summary of arXiv 2410.12982), written [FI], and its sections.
 *
 * The operation ([FI] "Definizione del Compito", "Definizione Specifica di
 * LCSM"), 0-indexed: for every channel (b, c), b in [0,B), c in [0,D),
 *
 *     y[b][t][c] = sum_{s=0}^{t} h[t-s][c] * x[b][s][c],     t in [0, L),
 *
 * where x[b][t+1][.] may only be supplied after y[b][t][.] has been returned
 * (online constraint).  The filter h[L][D] is shared by the B batch rows.  The
 * library evaluates it with the relaxed power-of-two tiling of [FI]
 * "Strategia di Tiling (Algoritmo 1)": once position i-1 is complete, with
 * U = largest power of two dividing i, the tile tau(x, [i-U, i), h, [i, i+U))
 * of [FI] "Definizione di Aggregazione di Contribuzione" adds the contribution
 * of x[i-U, i) to y[i, i+U) (clipped to < L).  Small tiles are direct
 * Toeplitz products, larger ones FFT circular convolutions of length 2U with
 * precomputed filter spectra ([FI] "Ottimizzazione della Memoria", "Trucco
 * di Convoluzione Circolare").  fi_step does tiles of side U <= T (the
 * config's small_tile_max) directly; the persistent pass (fi_run_closed_loop,
 * fi_run_prompted) does every tile of side < 256 and, for T < 256, the tile
 * of side 256 directly (on the matrix cores), and the larger ones by FFT.
 * The results agree to fp32 rounding.
 *
 * Layouts: row-major, channels innermost: h[L][D], x[B][L][D], y[B][L][D],
 * per-step vectors [B][D].  Storage dtype of x and h is the config's io_dtype
 * (fp32 or bf16); y is always fp32 and all arithmetic is fp32.
 *
 * Pointers: every array argument is a DEVICE pointer (hipMalloc'ed or a
 * torch CUDA tensor's data_ptr()) unless stated.  Calls other than
 * fi_create / fi_destroy are asynchronous on the config's stream: the caller
 * owns its arrays and must keep them valid until that stream is synchronised.
 *
 * Errors: functions return FI_OK (0) or a negative FI_ERR_* code and never
 * throw.  Arguments are validated before any device work; a rejected call
 * changes nothing.  FI_ERR_HIP records the HIP error, readable through
 * fi_strerror(FI_ERR_HIP) on the same thread.  A handle is not thread-safe;
 * distinct handles are independent.
 */
#ifndef FI_H_
#define FI_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fi_handle fi_handle;  /* opaque; owns all the device memory it allocates */

/* Storage type of x and h (y and every accumulation are always fp32). */
typedef enum { FI_F32 = 0, FI_BF16 = 1 } fi_dtype;

/* Feedback of fi_run_closed_loop. */
typedef enum {
    FI_FEEDBACK_NONE = 0,   /* open loop: x[b][t][c] read from x_in[B][L][D] */
    FI_FEEDBACK_TANH = 1    /* closed loop: x[b][t+1][c] = tanh(y[b][t][c]) */
} fi_feedback;

enum {
    FI_OK = 0,
    FI_ERR_INVALID = -1,      /* bad argument: NULL, size <= 0, overflow, unknown enum */
    FI_ERR_NOMEM = -2,        /* device allocation failed */
    FI_ERR_HIP = -3,          /* HIP runtime error (see fi_strerror) */
    FI_ERR_STATE = -4,        /* call not allowed at the handle's current position */
    FI_ERR_UNSUPPORTED = -5   /* valid but not supported (e.g. no gfx950 device) */
};

/* largest supported L (fi_create returns FI_ERR_UNSUPPORTED beyond it) */
#define FI_MAX_L (1LL << 25)

/* small_tile_max used when the config leaves it 0 */
#define FI_DEFAULT_SMALL_TILE_MAX 64

typedef struct {
    int64_t B;               /* batch rows, >= 1 */
    int64_t D;               /* channels per row, >= 1 */
    int64_t L;               /* positions = filter length, >= 1 (any value; tiles clip to < L) */
    fi_dtype io_dtype;       /* FI_F32 or FI_BF16 (an int-sized enum) */
    void *stream;            /* hipStream_t the handle works on; NULL = the null stream */
    int32_t small_tile_max;  /* T: the largest tile side fi_step does as a direct product, tiles of
                                side > T being FFT tiles: 64, 128 or 256; 0 = the environment's
                                FI_SMALL_TILE_MAX when set (an override for ablations; any other
                                value there gives FI_ERR_INVALID), else FI_DEFAULT_SMALL_TILE_MAX.  The persistent pass (fi_run_closed_loop,
                                fi_run_prompted) does every tile of side < 256 directly whatever T
                                is; it does the tile of side 256 from LDS when T = 256, else on
                                the matrix cores, and the larger ones by FFT. */
} fi_config;

/*
 * fi_create: validate cfg, allocate the handle's device state, copy the
 * filter h[L][D] (device pointer, io_dtype) and precompute, on the device,
 * the filter spectra of every FFT tile level ([FI] "Ottimizzazione della
 * Memoria": the filter DFT is computed ahead for each block size) and the
 * twiddle tables.  Synchronous: returns after the device work finished, so
 * the caller may free h at once.  On success *out receives the handle at
 * position 0; on failure *out is set to NULL and nothing stays allocated.
 * Errors: FI_ERR_INVALID for a NULL pointer, B, D or L < 1, an unknown dtype
 * or small_tile_max, or sizes whose element counts overflow; FI_ERR_UNSUPPORTED
 * for L > FI_MAX_L or when the current device is not gfx950; FI_ERR_NOMEM /
 * FI_ERR_HIP from the device.
 */
int fi_create(const fi_config *cfg, const void *h, fi_handle **out);

/*
 * fi_step: one online step at the handle's position t ([FI] "Strategia di
 * Tiling (Algoritmo 1)", one loop iteration): reads x_t[B][D] (io_dtype),
 * writes y_t[B][D] (fp32) = accumulated tiles + h[0] * x_t (the red cell),
 * then, if t+1 < L, applies the tile of side lowbit(t+1).  Position becomes
 * t+1.  FI_ERR_STATE when the position already is L.
 */
int fi_step(fi_handle *s, const void *x_t, float *y_t);

/*
 * fi_run_closed_loop: all L steps in one call, from position 0 (else
 * FI_ERR_STATE); leaves the position at L.  One persistent device pass: a
 * single kernel launch on the handle's stream, which may be captured into a
 * HIP graph and replayed (the pass clears the state it uses itself; the
 * handle's position is host state and is not replayed).
 *   fb = FI_FEEDBACK_TANH: x_in is x_0[B][D]; x[t+1] = tanh(y[t]) (rounded to
 *        bf16, nearest-even, when io_dtype is FI_BF16).
 *   fb = FI_FEEDBACK_NONE: x_in is x[B][L][D] (the open-loop inputs, consumed
 *        in order through the same online schedule).
 *   y[B][L][D] (fp32) receives every output; x_out[B][L][D] (io_dtype), if not
 *   NULL, receives the inputs that produced them.
 */
int fi_run_closed_loop(fi_handle *s, const void *x_in, fi_feedback fb, float *y, void *x_out);

/*
 * fi_run_prompted: generation from a prompt ([FI] "Definizione del Compito":
 * the prompt x_1 .. x_p is given, later inputs are produced one by one), all
 * L steps in one call from position 0 (else FI_ERR_STATE), leaving the
 * position at L.  Positions t < p read x_prompt[B][p][D] (io_dtype); from
 * position p on, x[t] = tanh(y[t-1]) (rounded to bf16, nearest-even, when
 * io_dtype is FI_BF16).  Every output goes through the same online schedule
 * as fi_run_closed_loop; p = 1 is its closed loop with x_0 = x_prompt[.][0][.]
 * and p = L its open loop.  y[B][L][D] (fp32) receives every output; x_out
 * [B][L][D] (io_dtype), if not NULL, the inputs that produced them (the
 * prompt's values unchanged).  FI_ERR_INVALID for a NULL handle, x_prompt or
 * y, or p outside [1, L].  The caller owns x_prompt, y and x_out, which must
 * stay valid until the stream has passed the call.
 */
int fi_run_prompted(fi_handle *s, const void *x_prompt, int64_t p, float *y, void *x_out);

/*
 * fi_conv_static: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * fi_create + fi_run_closed_loop + fi_destroy in one call that allocates
 * nothing.  Same arguments and results as those calls: cfg, h[L][D]
 * (io_dtype) as for fi_create; x_in, fb, y, x_out as for fi_run_closed_loop.
 * The handle's device buffers (filter rows, accumulator rows, spectra,
 * twiddles, FFT scratch) are carved from one fixed workspace of
 * FI_STATIC_WORKSPACE_BYTES per device, a static device array the library
 * holds until the process ends; no hipMalloc, hipFree or other allocating
 * call is made.  Their size is about 4 LS (D + B D) + 8 D L bytes (LS = L
 * rounded up to 64) plus twiddle tables and, when L > 8192, FFT scratch of
 * 8 * min(B D, resident teams) * (largest tile side) bytes; larger problems
 * get FI_ERR_UNSUPPORTED and nothing is launched.  Asynchronous on
 * cfg->stream (nothing is synchronised): the caller keeps h, x_in, y and
 * x_out valid until the stream has passed the call.  Every call on a device
 * uses that device's one workspace: calls that overlap on one device (on
 * different streams, or from different threads) race and give undefined
 * results; calls in order on one stream are safe.  Errors as fi_create and
 * fi_run_closed_loop (FI_ERR_INVALID, FI_ERR_UNSUPPORTED, FI_ERR_HIP).
 */
#define FI_STATIC_WORKSPACE_BYTES (64LL << 20)
int fi_conv_static(const fi_config *cfg, const void *h, const void *x_in, fi_feedback fb, float *y,
                   void *x_out);

/*
 * The layer stack ([FI] "Algoritmo di Inferenza LCSM (Algoritmo 2)",
 * "Parallelizzazione Cross-Layer (Algoritmo 3)"): M layers, each a long
 * convolution mixer (filter rho^l[L][D], per channel) followed by a block
 * (the synthetic MLP + GELU block of [FI] "Configurazione Sperimentale"),
 * and a sampler that feeds the last layer's output back with added noise.
 * 0-indexed, for every batch row b and position t, with a^0 = x:
 *   z^l_t[c]  = sum_{s<=t} rho^l[t-s][c] a^l_s[c]
 *   a^{l+1}_t = W2^l act(W1^l z^l_t)          (W row j = output j, D x D)
 *   x_{t+1}   = a^M_t + sigma noise[t]
 * The mixers run the relaxed tiling of fi_step on all M B D channels (red
 * cells and blocks of all layers in order at each position, then the gray
 * tiles of all layers in one launch).  fp32 storage and arithmetic.
 */
typedef struct fi_stack fi_stack;   /* opaque; owns its device memory */
typedef enum { FI_ACT_GELU = 0, FI_ACT_TANH = 1, FI_ACT_IDENTITY = 2 } fi_activation;
typedef struct {
    int64_t B;                /* batch rows, >= 1 */
    int64_t D;                /* channels (the blocks are D x D), 1 <= D <= 8192 */
    int64_t L;                /* positions = filter length, >= 1 */
    int64_t M;                /* layers, >= 1 */
    fi_activation act;        /* the blocks' activation: GELU (exact, erf), tanh or identity */
    void *stream;             /* hipStream_t; NULL = the null stream */
    int32_t small_tile_max;   /* T as in fi_config (0 = default) */
} fi_stack_config;

/* fi_stack_create: copies rho[M][L][D], w1[M][D][D] and w2[M][D][D] (device
 * pointers, fp32; W[l][j][k] is the weight of input k in output j) and
 * precomputes every layer's filter spectra.  Synchronous.  Errors as
 * fi_create (FI_ERR_INVALID for an unknown act or M < 1;
 * FI_ERR_UNSUPPORTED for D > 8192). */
int fi_stack_create(const fi_stack_config *cfg, const float *rho, const float *w1, const float *w2,
                    fi_stack **out);

/* fi_stack_run: generates all L positions from x0[B][D]: y[B][L][D]
 * receives a^M_t, x_out[B][L][D] (or NULL) the inputs x_t; noise[B][L][D]
 * (or NULL: no noise) is scaled by sigma.  Each call starts from position 0.
 * It first waits for the stream to pass the handle's earlier runs, then
 * queues one launch per position (two where the position completes a tile
 * of side > 16) and returns: device pointers, owned by the caller until the
 * stream has passed the call.  A position's layers run on up to 16
 * workgroups that wait for each other's partial products; a wait past its
 * limit (about a second: the workgroups could not all be resident) leaves
 * garbage in that run's outputs and makes this and every later call on the
 * handle return FI_ERR_HIP.  L M must not exceed 2^30 (FI_ERR_UNSUPPORTED
 * at fi_stack_create). */
int fi_stack_run(fi_stack *s, const float *x0, const float *noise, float sigma, float *y, float *x_out);

/* fi_stack_destroy: synchronise the stream and free everything; NULL is a no-op. */
void fi_stack_destroy(fi_stack *s);

/* fi_reset: position := 0; the accumulators are cleared on the stream before
 * the next fi_step (fi_run_closed_loop clears the rows it uses itself). */
int fi_reset(fi_handle *s);

/* fi_destroy: synchronise the stream and free everything; NULL is a no-op. */
void fi_destroy(fi_handle *s);

/* fi_position: the handle's current position (host value), or -1 for NULL. */
int64_t fi_position(const fi_handle *s);

/* fi_strerror: static description of a status code (host; thread-local text
 * for FI_ERR_HIP includes the last HIP error seen on this thread). */
const char *fi_strerror(int status);

/*
 * Schedule helper (host, integer only): the tile applied once position i-1
 * is complete, for 1 <= i < L ([FI] "Strategia di Tiling (Algoritmo 1)",
 * "Analisi di Complessita (Proposizione 1)"): U = largest power of two dividing
 * i, inputs [in_lo, in_hi) = [i-U, i), outputs [out_lo, out_hi) =
 * [i, min(i+U, L)).  FI_ERR_INVALID for i outside [1, L) or a NULL out.
 */
typedef struct {
    int64_t U, in_lo, in_hi, out_lo, out_hi;
} fi_tile;
int fi_tile_at(int64_t L, int64_t i, fi_tile *out);

#ifdef __cplusplus
}
#endif
#endif /* FI_H_ */
