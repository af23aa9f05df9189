/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD selective-scan library.
 *
 * The operation ("Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching for Inference", abstract; recurrence as in
 * "Engineering hybrid state-space models", innvotechnologies blog, section 2):
 * per sequence, head h (group g = h / (H/G)) and token t,
 *
 *     S_t = exp(dt[t,h] * A[h]) * S_{t-1} + dt[t,h] * x[t,h,:] (outer) B[t,g,:]
 *     y[t,h,:] = S_t C[t,g,:]  +  D[h] * x[t,h,:]
 *
 * with S a (P x N) fp32 state per (sequence, head).  Two entry points:
 *   ssd_chunked_scan  -- prefill over whole sequences, computed chunk by chunk
 *                        (the paper's fixed-size chunking); returns y and the
 *                        state after each sequence's last token;
 *   ssd_decode_step   -- the O(1) cached single-token step, updating the state
 *                        in place (the paper's cached decode).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory, never synchronizes, and keeps no
 *     global state: calls are reentrant and asynchronous on `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream).
 *   - Tensors are dense row-major with the innermost index last, as listed per
 *     argument.  Tensor pointers must be 16-byte aligned, except the fp32
 *     vectors dt, A, D and dt_bias, which the kernels read one element at a
 *     time and which need only 4-byte alignment (so a per-step slice of a
 *     [steps, batch, H] dt buffer can be passed as is).
 *   - Validation runs on the host before any launch.  On any error nothing is
 *     launched and nothing is written; the returned code says why and
 *     ssd_last_error_detail() gives a sentence (thread-local).
 *   - Inputs are not checked for NaN/Inf; such values propagate.
 *   - dtype of x, B and C is ssd_shape.dtype (fp32 or bf16); dtype of y is
 *     ssd_shape.ydtype (fp32 by default); dt, A, D and every state tensor are
 *     always fp32.  Accumulation is fp32; bf16 inputs are widened exactly; a
 *     bf16 y is rounded to nearest even.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    SSD_ERR_DTYPE = -3,       /* unknown dtype code */
    SSD_ERR_ALIGN = -4,       /* a tensor pointer is not aligned as required */
    SSD_ERR_CHUNK = -5,       /* chunk not in {32, 64, 128, 256} */
    SSD_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the query says */
    SSD_ERR_HIP = -7,         /* the HIP runtime reported an error at launch */
    SSD_ERR_UNSUPPORTED = -8, /* valid but outside what the kernels implement */
    SSD_ERR_SEQLENS = -9,     /* host copy of cu_seqlens is not a valid offset list */
    SSD_ERR_VALUE = -10       /* a scalar argument is out of its range */
} ssd_status;

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/*
 * Problem description.
 *   Dense batch (cu_seqlens == NULL): `batch` sequences of `seqlen` tokens;
 *     token rows are indexed [batch, seqlen].
 *   Packed variable-length batch (cu_seqlens != NULL): `batch` sequences packed
 *     into one stream of `seqlen` = T tokens; sequence s owns rows
 *     [cu_seqlens[s], cu_seqlens[s+1]).  Chunks restart at every sequence start
 *     and never straddle two sequences; a zero-length sequence passes its
 *     initial state through unchanged.
 *   headdim P in [8, 128] and dstate N in [8, 256], both multiples of 8;
 *   ngroups G >= 1 divides nheads H; head h reads B/C group h / (H/G).
 *   path: which kernels compute the chunk states, their passing and y
 *     (ssd_path; SSD_PATH_AUTO, i.e. 0, lets the library choose).  Every path
 *     computes the same result up to fp32 rounding order; the others exist
 *     for tests and measurements.  The workspace size depends on the path:
 *     query it with the same shape the call uses.
 *   reserved: must be zero.
 */
typedef enum ssd_path {
    SSD_PATH_AUTO = 0,
    SSD_PATH_CHUNK_PARALLEL = 1, /* chunk states, state passing and outputs as three
                                    launches, each parallel over chunks */
    SSD_PATH_STATE_WALK = 2,     /* one walk per (sequence, head, 32-column tile) for the
                                    states and their passing, then the outputs */
    SSD_PATH_SCAN_WALK = 3       /* one walk per (sequence, group, slice of heads) that also
                                    writes y, so no per-chunk state leaves the chip; bf16
                                    inputs, chunk 256 and dstate in (64, 128] only
                                    (SSD_ERR_UNSUPPORTED otherwise) */
} ssd_path;

typedef struct ssd_shape {
    int64_t batch;
    int64_t seqlen;
    int32_t nheads;
    int32_t headdim;
    int32_t dstate;
    int32_t ngroups;
    int32_t dtype;               /* ssd_dtype of x, B, C */
    int32_t ydtype;              /* ssd_dtype of y (0 = SSD_F32, the default) */
    int32_t path;                /* ssd_path (0 = the library's choice) */
    int32_t reserved;            /* must be 0 */
    const int32_t* cu_seqlens;      /* device int32 [batch+1], or NULL (dense) */
    const int32_t* cu_seqlens_host; /* optional host copy; validated when given */
} ssd_shape;

/*
 * Workspace bytes that ssd_chunked_scan needs for this shape and chunk size.
 * Writes *bytes and returns SSD_OK, or an error code for an invalid shape.
 */
ssd_status ssd_chunked_scan_workspace_size(const ssd_shape* shape, int32_t chunk, size_t* bytes);

/*
 * Chunked prefill.  ("Compiler-First State Space Duality...", abstract:
 * fixed-size chunking, einsum-dominated compute; chunk algebra as in the
 * blog's section 2 duality Y = (M o CB^T) X with a 1-semiseparable mask M.)
 *
 *   x          [rows, H, P]  dtype      rows = batch*seqlen (dense) or T (packed)
 *   dt         [rows, H]     fp32       step sizes, used as given (no activation)
 *   A          [H]           fp32       per-head scalar decay rate
 *   B, C       [rows, G, N]  dtype
 *   D          [H]           fp32       skip coefficient
 *   chunk      32, 64, 128 or 256 tokens
 *   init_state [nseq, H, P, N] fp32, or NULL for zero initial states
 *   y          [rows, H, P]  ydtype     output; must not alias any input
 *   final_state[nseq, H, P, N] fp32, or NULL (not written); may alias
 *              init_state (each element is read before it is written)
 *   workspace  device scratch of at least the queried size, owned by the
 *              caller, contents undefined on entry and exit.  It holds the
 *              per-chunk decay tables and C.B^T, and (every path but the scan
 *              walk) one fp32 (P x N) state per (chunk, head), about
 *              4*P*N*H/chunk bytes per token.
 *   stream     hipStream_t (as void*) the kernels are queued on
 * Returns SSD_OK once the kernels are queued (asynchronous).
 */
ssd_status ssd_chunked_scan(const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D, int32_t chunk,
                            const float* init_state, void* y, float* final_state,
                            const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * O(1) cached decode step, in place.  ("Compiler-First State Space
 * Duality...", abstract: registered cache + cached decode whose cost does not
 * depend on the sequence length; the state is a fixed (batch, heads,
 * head_dim, state_dim) buffer as in the blog's section 3.)
 *
 *   state [batch, H, P, N] fp32   read and overwritten with the new state
 *   x     [batch, H, P]  dtype    one token per sequence
 *   dt    [batch, H]     fp32
 *   A, D  [H]            fp32
 *   B, C  [batch, G, N]  dtype
 *   y     [batch, H, P]  ydtype   output; must not alias any input
 * shape->seqlen and shape->cu_seqlens are ignored.  batch * H may be at most
 * 2^31 - 8 (one launch grid, one wave per (sequence, head)); larger batches
 * return SSD_ERR_SHAPE.
 */
ssd_status ssd_decode_step(float* state, const void* x, const float* dt, const float* A,
                           const void* B, const void* C, const float* D, void* y,
                           const ssd_shape* shape, void* stream);

/*
 * Fused dt activation.  The step size comes from a softplus of the projected
 * input plus a per-head bias ("Engineering hybrid state-space models",
 * section 3, architecture figure of the Mamba-2 block).  The *_dt_act entry
 * points take that raw dt and use, for every (token, head),
 *
 *     dt = min(max(softplus(dt_raw[., h] + dt_bias[h]), dt_min), dt_max)
 *     softplus(v) = log(1 + exp(v)), taken as v itself for v > 20,
 *
 * evaluated in fp32 where dt enters the kernels (the cumsum stage of the
 * prefill, the decode step).  Everything else is exactly ssd_chunked_scan /
 * ssd_decode_step; the `dt` argument holds dt_raw.
 *
 *   dt_bias  [H] fp32 device pointer, 4-byte aligned, or NULL for no bias
 *   dt_min   lower clamp: finite and >= 0
 *   dt_max   upper clamp: >= dt_min (INFINITY: no upper clamp)
 * Errors as the plain entry points, plus SSD_ERR_NULL for a NULL `act` and
 * SSD_ERR_VALUE for a clamp range outside the above (NaN included).
 */
typedef struct ssd_dt_activation {
    const float* dt_bias;
    float dt_min;
    float dt_max;
} ssd_dt_activation;

ssd_status ssd_chunked_scan_dt_act(const void* x, const float* dt_raw, const float* A, const void* B,
                                   const void* C, const float* D, int32_t chunk,
                                   const float* init_state, void* y, float* final_state,
                                   const ssd_dt_activation* act, const ssd_shape* shape,
                                   void* workspace, size_t workspace_bytes, void* stream);

ssd_status ssd_decode_step_dt_act(float* state, const void* x, const float* dt_raw, const float* A,
                                  const void* B, const void* C, const float* D, void* y,
                                  const ssd_dt_activation* act, const ssd_shape* shape, void* stream);

/*
 * Exact windowed decode step ("SketchSSM: Write to the Full State, Read from
 * a Compact Sketch", Fig. 3(a), Fig. 4 and Table 4: ReplaySSM reads the full
 * state at every step and writes it once per window of W tokens, D + D/W
 * state traffic per step instead of 2D).
 *
 * The caller keeps the state S0 as of the last flush and the tokens since
 * then in window slots 0..t; slot t holds the current token.  The call writes
 * the current token's output
 *     y_t = exp(cs_t) S0 C_t + sum_{s<=t} exp(cs_t - cs_s) dt_s (B_s . C_t) x_s + D x_t,
 *     cs_s = A sum_{u<=s} dt_u,
 * which equals what t+1 ssd_decode_step calls from S0 would give, and, when
 * `flush` is 1, replaces S0 by the state after token t (the caller then
 * starts a new window at slot 0).  With flush = 0 the state is only read.
 *
 *   state  [batch, H, P, N] fp32   S0 (rewritten only when flush = 1)
 *   x      [batch, W, H, P] dtype  window slots; slots > t are not read
 *   dt     [batch, W, H]    fp32   (raw when act is given)
 *   A, D   [H]              fp32
 *   B, C   [batch, W, G, N] dtype
 *   y      [batch, H, P]    ydtype output of token t; must not alias an input
 *   window W in [1, 16]; t in [0, W); flush 0 or 1
 *   act    NULL, or the dt activation of ssd_decode_step_dt_act
 * shape->seqlen and shape->cu_seqlens are ignored.  Errors (and the batch * H
 * limit) as ssd_decode_step, plus SSD_ERR_VALUE for window, t or flush out of
 * range (and the activation errors).
 */
ssd_status ssd_decode_window_step(float* state, const void* x, const float* dt, const float* A,
                                  const void* B, const void* C, const float* D, void* y, int32_t window,
                                  int32_t t, int32_t flush, const ssd_dt_activation* act,
                                  const ssd_shape* shape, void* stream);

/*
 * Causal depthwise conv1d with optional SiLU, the step before the scan in the
 * Mamba-2 block ("Engineering Hybrid State-Space Models", section 3,
 * architecture figure: a width-4 1D convolution + SiLU), with its cache of
 * the K-1 most recent inputs per channel (same page, section 4: the conv state
 * [dConv - 1, channels] of each layer's state buffer).  Per sequence, channel
 * c and token t, over the padded sequence xp = [conv state (K-1 rows, oldest
 * first); x]:
 *
 *     v[t, c] = bias[c] + sum_{k<K} weight[c, k] * xp[t + k, c]
 *     out[t, c] = activation ? v / (1 + exp(-v)) : v
 *
 * so weight[c, K-1] multiplies the current token.  The state after a
 * sequence is the last K-1 rows of xp.
 *
 * Shape:
 *   batch        sequences (>= 0)
 *   seqlen       dense (cu_seqlens == NULL): tokens per sequence, rows =
 *                batch*seqlen in [batch, seqlen] order; packed: total tokens T,
 *                sequence s owns rows [cu_seqlens[s], cu_seqlens[s+1])
 *   channels     C, a multiple of 8, at most 2^20
 *   width        K in [2, 4]
 *   dtype        ssd_dtype of x and of the conv states
 *   ydtype       ssd_dtype of the outputs
 *   activation   0: none; 1: SiLU
 *   reserved     must be 0
 *
 * Outputs: the C channels of a row are split into nparts (1 to 3) contiguous
 * channel ranges, in order, each written to its own dense buffer: part p is
 * [rows, channels[p]] in ydtype, channels[p] a multiple of 8, the channels
 * summing to C.  (With the Mamba-2 channel order x | B | C, the three parts
 * are the scan's x, B and C inputs, written with no separate split pass.)
 * Unused entries must be 0 / NULL.
 */
typedef struct ssd_conv_shape {
    int64_t batch;
    int64_t seqlen;
    int32_t channels;
    int32_t width;
    int32_t dtype;
    int32_t ydtype;
    int32_t activation;
    int32_t reserved;
    const int32_t* cu_seqlens;      /* device int32 [batch+1], or NULL (dense) */
    const int32_t* cu_seqlens_host; /* optional host copy; validated when given */
} ssd_conv_shape;

typedef struct ssd_conv_outputs {
    int32_t nparts;
    int32_t channels[3];
    void* out[3];
} ssd_conv_outputs;

/*
 *   x              [rows, C]        dtype
 *   weight         [C, K]           fp32
 *   bias           [C]              fp32, or NULL (zero)
 *   conv_state_in  [batch, K-1, C]  dtype, or NULL (zero history)
 *   conv_state_out [batch, K-1, C]  dtype, or NULL (not written); may equal
 *                  conv_state_in (it is written after every read of it)
 *   out            the output parts (above); no part may alias an input
 * Errors: SSD_ERR_NULL, SSD_ERR_ALIGN, SSD_ERR_DTYPE, SSD_ERR_SHAPE (sizes,
 * parts, aliasing), SSD_ERR_VALUE (activation), SSD_ERR_SEQLENS (host copy
 * of cu_seqlens), SSD_ERR_HIP.
 */
ssd_status ssd_causal_conv1d(const void* x, const float* weight, const float* bias,
                             const void* conv_state_in, void* conv_state_out,
                             const ssd_conv_outputs* out, const ssd_conv_shape* shape, void* stream);

/*
 * One decode token per sequence, the conv state updated in place (oldest row
 * dropped, the token appended):
 *   conv_state [batch, K-1, C] dtype, read and overwritten
 *   x          [batch, C]      dtype
 *   weight, bias, out as ssd_causal_conv1d, with rows = batch
 * shape->seqlen and shape->cu_seqlens are ignored.  Same errors.
 */
ssd_status ssd_causal_conv1d_step(void* conv_state, const void* x, const float* weight, const float* bias,
                                  const ssd_conv_outputs* out, const ssd_conv_shape* shape, void* stream);

/*
 * Measurement helper, for benchmarks only: does what ssd_chunked_scan does,
 * with a HIP event recorded on `stream` before and after every kernel stage,
 * then waits for the last event and writes each stage's elapsed time in
 * milliseconds to stage_ms[SSD_PREFILL_STAGES], in the order plan, cumsum,
 * cb, chunk_state, state_passing, chunk_scan, scan_walk.  A stage the path
 * does not run reads exactly 0:
 *   SSD_PATH_CHUNK_PARALLEL  scan_walk
 *   SSD_PATH_STATE_WALK      state_passing (the passing runs inside the
 *                            chunk_state stage), scan_walk
 *   SSD_PATH_SCAN_WALK       chunk_state, state_passing, chunk_scan
 * With SSD_PATH_AUTO the library takes a walk when there are enough
 * (sequence, head, 32-column tile) walks, 256 or more, and sequences of
 * similar length (with a host copy of a packed batch's offsets, no sequence
 * over 1.5 times the mean chunk count), else the chunk-parallel path.  The
 * walk it takes is the scan walk where that path applies, else the state
 * walk.  For a packed batch of at most 256 sequences with a host copy of
 * its offsets, where the scan walk applies, the library instead estimates
 * the scan walk (which runs the longest sequences first) against the
 * chunk-parallel path and takes the walk when it expects it to be at least
 * 10% faster.
 * Unlike ssd_chunked_scan it blocks the calling thread until the kernels
 * finish.  Same arguments and errors as ssd_chunked_scan, plus SSD_ERR_NULL
 * when stage_ms is NULL.
 */
#define SSD_PREFILL_STAGES 7
ssd_status ssd_chunked_scan_profiled(const void* x, const float* dt, const float* A,
                                     const void* B, const void* C, const float* D, int32_t chunk,
                                     const float* init_state, void* y, float* final_state,
                                     const ssd_shape* shape, void* workspace,
                                     size_t workspace_bytes, void* stream, float* stage_ms);

/*
 * Allocation-free prefill, for callers that cannot allocate device memory:
 * code under stream capture, tight serving loops, harnesses that forbid
 * allocation.  It does exactly what ssd_chunked_scan does, with the
 * workspace taken from a device array inside the library instead of an
 * argument: SSD_NOALLOC_SCRATCH_BYTES bytes on every device it runs on, held
 * until the process ends.
 *   - The array of the current device (hipGetDevice) is used; `stream` must
 *     belong to that device.  Its address is looked up (hipGetSymbolAddress)
 *     on the first call with a device current and kept.
 *   - Every call on a device shares that device's array.  Calls that overlap
 *     on one device (other host threads, or streams with no ordering between
 *     them) race; the caller orders them.  Nothing in the array has to start
 *     at zero.
 *   - A shape whose workspace (ssd_chunked_scan_workspace_size with the same
 *     shape and chunk) exceeds the array returns SSD_ERR_WORKSPACE before
 *     anything is launched.
 *   - It calls nothing that allocates or frees device memory.
 * Same arguments as ssd_chunked_scan without workspace and workspace_bytes;
 * same errors, plus SSD_ERR_HIP if the device or the array's address cannot
 * be queried.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_chunked_scan_noalloc(const void* x, const float* dt, const float* A, const void* B,
                                    const void* C, const float* D, int32_t chunk,
                                    const float* init_state, void* y, float* final_state,
                                    const ssd_shape* shape, void* stream);

/* Static English name of a status code. */
const char* ssd_status_string(int32_t status);

/* Thread-local sentence describing the last error returned on this thread. */
const char* ssd_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
