/*
 * flce.h - C ABI of the MI355X (gfx950) fused linear + cross-entropy library (libflce.so).
 *
 * What one call computes (forward and backward in one pass over the data):
 *
 *   z   = hidden[BT, H] . W[V, H]^T          the LM-head linear layer, W in nn.Linear(H, V, bias=False)
 *                                            layout (the test in PyTorch PR #126348, "[AOTAutograd]
 *                                            tweak min-cut partitioner to avoid saving softmax output")
 *   s   = softcap * tanh(z / softcap)        Gemma2-style logit softcap when softcap > 0 (named in
 *                                            Liger-Kernel issue #227, "Torch compiled FLCE is 2x faster
 *                                            than the current FLCE"; the formula is this library's reading)
 *   lse = log sum_v exp(s_v)                 per row: the row max and row sum-of-exponentials of the
 *                                            PR #126348 description, here formed online over V tiles
 *   loss = sum over valid rows of (lse - s[label]) / N    (FLCE_MEAN, N = number of valid rows)
 *        = sum over valid rows of (lse - s[label])        (FLCE_SUM)
 *   grad_hidden = dZ . W,   grad_W = dZ^T . hidden,
 *   dZ = g * (softmax(s) - onehot(label)) * (1 - (s/softcap)^2 if softcap > 0),
 *   g = 1/N (mean) or 1 (sum) on valid rows, 0 on rows whose label is ignore_index.
 *
 * The softmax is never stored: as the PR #126348 description proposes, the backward rebuilds it from
 * the logits and the small per-row max/sum statistics. Per chunk of rows the workspace holds one
 * 16-bit [chunk_rows, V] buffer of softmax numerators exp(s - c) (c a per-row reference); the backward
 * GEMMs read it as it is and apply the per-row normalisation by linearity, so dlogits are never
 * written. No [BT, V] buffer is allocated by the library or required of the caller.
 * B*T may be any value (ragged batches, as in the benchmark comment of Liger-Kernel issue #227): the
 * library splits the rows into balanced chunks (flce_chunk_plan) with one code object.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers on the handle's device; "host" pointers are
 *     ordinary host memory. The caller owns every buffer passed in; the library never frees them.
 *   - Row-major, contiguous, densely packed: hidden and grad_hidden are [BT][H], W and grad_W are
 *     [V][H], labels is [BT]. Device pointers must be 16-byte aligned (labels: 8-byte). The *_rows
 *     entry points take hidden, grad_hidden and labels as batches of sequences at given strides
 *     (see flce_rows).
 *   - Errors are reported synchronously by the return code before anything is enqueued; the
 *     outputs are then untouched. The compute entry points never allocate, never synchronise and
 *     enqueue all their work on `stream`.
 *   - A handle may be used by one stream at a time (it holds a small device status word).
 *   - Since the compute entry points only launch kernels (no allocation, no memset, no copy, no
 *     synchronisation), a caller may capture them into a HIP graph on `stream` and replay it; each
 *     replay reads the buffers' current contents. flce_status and flce_profile_* are not capturable.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct flce_ctx* flce_handle;

/* Element type of hidden, W and grad_hidden. grad_W is always fp32 (it is the accumulator). */
typedef enum { FLCE_BF16 = 0, FLCE_FP32 = 1 } flce_dtype;

/* Loss reduction. FLCE_NONE (per-row losses) is offered by flce_forward only: the fused forward +
 * backward assumes a scalar upstream gradient. */
typedef enum { FLCE_NONE = 0, FLCE_MEAN = 1, FLCE_SUM = 2 } flce_reduction;

/* Return codes. */
enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = -1,        /* null pointer, bad size, bad enum, misaligned pointer, bad softcap */
  FLCE_ERR_UNSUPPORTED = -2,        /* a valid request this library does not implement (e.g. H % 8 != 0) */
  FLCE_ERR_WORKSPACE_TOO_SMALL = -3,/* workspace_bytes < flce_workspace_size(...) */
  FLCE_ERR_HIP = -4,                /* a HIP runtime call or kernel launch failed */
  FLCE_ERR_LABEL_RANGE = -5         /* (flce_status) a label outside [0, V) that is not ignore_index */
};

/* Configuration passed to flce_create; a NULL pointer or zero fields select the defaults. */
typedef struct {
  int64_t chunk_rows_max; /* row cap of a chunk (0 = automatic, see flce_chunk_plan); rounded up to a
                           * multiple of 256 */
  int64_t reserved[3];    /* must be zero */
} flce_config;

/* Create a handle on HIP device `device`. Allocates a few hundred bytes of device memory for the
 * status word (freed by flce_destroy). *out receives the handle. Returns FLCE_OK, or
 * FLCE_ERR_INVALID_ARG (out == NULL, nonzero reserved fields, negative chunk_rows_max) or
 * FLCE_ERR_HIP (no such device / allocation failed). */
int flce_create(flce_handle* out, int device, const flce_config* cfg);

/* Release the handle and its device memory. NULL is accepted. Pending work that uses the handle
 * must have completed. */
int flce_destroy(flce_handle h);

/* Bytes of device workspace flce_forward_backward needs for this problem (host-only arithmetic, no
 * device call). h may be NULL (default configuration). The workspace holds one chunk of
 * logits-derived values ([chunk_rows][V rounded up to 256], bf16 for FLCE_BF16, fp32 for
 * FLCE_FP32), per-(row, 128-wide V segment) statistics, per-row data, split-K partials of
 * grad_hidden, two [chunk_rows][H] copies of the chunk's hidden rows (transposed; scaled by the
 * per-row factor of the backward) and, for plans of several chunks whose grad_W grid leaves its last
 * wave of 256 x 256 tiles under half full, fp32 partial tiles of that wave (at most one per compute
 * unit). It never grows with BT beyond O(BT) bytes of per-row data.
 * Returns FLCE_OK and writes *bytes, or FLCE_ERR_INVALID_ARG. */
int flce_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, size_t* bytes);

/* Chunk plan for BT rows of a problem with hidden size H, vocabulary V and dtype (host-only):
 * n = ceil(BT / cap) chunks of chunk_rows rows (a multiple of 256, at most cap), the last one holding
 * BT - (n-1)*chunk_rows rows. cap is the handle's chunk_rows_max if configured; otherwise (also for
 * h == NULL) it is automatic: max(4096, min(2^24 / H rounded up to 256, the largest multiple of 256
 * whose [rows][V rounded up to 256] buffer of the dtype fits 2 GiB)). The 2^24 / H term gives one
 * chunk's grad_hidden product (rows x H) at least 256 output tiles of 256 x 256, one per compute unit,
 * for narrow hidden sizes (H = 768: 16384-row chunks at BT = 32768). Every entry point that chunks
 * rows follows this plan. Returns FLCE_OK, FLCE_ERR_INVALID_ARG (NULL outputs, BT < 0, H or V <= 0,
 * bad dtype) or FLCE_ERR_UNSUPPORTED for sizes the library rejects. */
int flce_chunk_plan(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, int64_t* n_chunks,
                    int64_t* chunk_rows);

/* The fused forward + backward.
 *   hidden       device, [BT][H] of dtype          (read)
 *   W            device, [V][H] of dtype           (read)
 *   labels       device, [BT] int64                (read); ignore_index marks rows left out
 *   BT >= 0, 0 < H <= 65536 with H % 8 == 0, 0 < V <= 2^20 (larger sizes: FLCE_ERR_UNSUPPORTED)
 *   dtype        FLCE_BF16 or FLCE_FP32
 *   softcap      0 = off, > 0 = cap; negative or NaN is FLCE_ERR_INVALID_ARG
 *   reduction    FLCE_MEAN or FLCE_SUM (dLoss/dloss = 1 is assumed; scale the grads for other upstream
 *                grads); FLCE_NONE is FLCE_ERR_UNSUPPORTED here (see flce_forward)
 *   loss         device, 1 float (written)
 *   grad_hidden  device, [BT][H] of dtype (overwritten)
 *   grad_W       device, [V][H] fp32 (overwritten)
 *   workspace    device, >= flce_workspace_size bytes, 256-byte aligned; contents are scratch
 *   stream       a hipStream_t (NULL = the null stream)
 * Mean over zero valid rows gives loss 0 and zero gradients. A label outside [0, V) that is not
 * ignore_index is treated as ignored and flagged in the handle's status word (see flce_status).
 * BT == 0 writes loss = 0 and grad_W = 0. Returns FLCE_OK or an error code before enqueueing. */
int flce_forward_backward(flce_handle h,
                          const void* hidden, const void* W, const int64_t* labels,
                          int64_t BT, int64_t H, int64_t V, int dtype,
                          int64_t ignore_index, float softcap, int reduction,
                          float* loss, void* grad_hidden, float* grad_W,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The recompute mode: the result of flce_forward_backward with no [rows][V] buffer and more work.
 * The PR #126348 description rebuilds the softmax in the backward pass from the softmax input and
 * the per-row max/sum; here the softmax input itself is rebuilt too. One pass covers all BT rows
 * (the handle's chunk_rows_max does not apply): a forward pass over the whole vocabulary gives each
 * row's log-sum-exp; then, per vocabulary slice of v_slice columns, outermost, the logits of all
 * rows are computed again and turned into dZ against that lse. That dZ is used at once for the
 * slice's rows of grad_W, written once, and for an fp32 [BT][H] running sum of grad_hidden. The
 * logits GEMM runs twice: 8 * BT * H * V flop instead of 6. The workspace holds one [BT][v_slice]
 * slice of dZ numerators (16-bit for bf16, fp32 for fp32), per-row statistics of 128-wide vocabulary
 * segments ([BT][V/128], twice, fp32), the fp32 [BT][H] accumulator and two [BT][H] copies of hidden
 * (transposed, and scaled per row) in the input dtype: linear in BT, independent of V but for the
 * segment statistics.
 *   v_slice      vocabulary columns per slice: 0 = 8192; rounded up to a multiple of 256; at most V
 *                rounded up; negative is FLCE_ERR_INVALID_ARG
 * Everything else as for flce_forward_backward. The loss is bitwise that of flce_forward_backward on
 * the same inputs. grad_W is bitwise that of flce_forward_backward on a handle whose chunk plan puts
 * all BT rows in one chunk, as long as no counted row's largest logit exceeds its label logit by more
 * than 48 (such rows have their stored numerators rescaled by the fused call and formed against the
 * final maximum here: the two agree to rounding). grad_hidden differs from the fused call's only by
 * the order of its fp32 sums (one per slice, added in slice order). */
int flce_recompute_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype,
                                  int64_t v_slice, size_t* bytes);
int flce_forward_backward_recompute(flce_handle h,
                                    const void* hidden, const void* W, const int64_t* labels,
                                    int64_t BT, int64_t H, int64_t V, int dtype,
                                    int64_t ignore_index, float softcap, int reduction,
                                    int64_t v_slice,
                                    float* loss, void* grad_hidden, float* grad_W,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace flce_forward needs (host-only arithmetic; h may be NULL). The forward
 * path keeps no logits: the workspace holds the per-(row, 128-wide V segment) statistics of one
 * chunk, per-row label data and one chunk of hidden transposed. Returns FLCE_OK or
 * FLCE_ERR_INVALID_ARG / FLCE_ERR_UNSUPPORTED for sizes flce_forward rejects. */
int flce_forward_workspace_size(flce_handle h, int64_t BT, int64_t H, int64_t V, int dtype, size_t* bytes);

/* Forward only (evaluation, per-row verification): the loss of the same model as
 * flce_forward_backward without any gradient, and optionally the per-row terms.
 *   hidden, W, labels, BT, H, V, dtype, ignore_index, softcap   as for flce_forward_backward
 *   reduction    FLCE_MEAN or FLCE_SUM (loss required), or FLCE_NONE (loss_rows required)
 *   loss         device, 1 float (written for MEAN/SUM; may be NULL for NONE)
 *   loss_rows    device, [BT] float or NULL (required for FLCE_NONE when BT > 0): row t gets
 *                lse_t - s_t[label_t] (the NLL term of the
 *                PR #126348 description), 0 where the label is ignore_index or out of range
 *   lse_rows     device, [BT] float or NULL: row t gets lse_t = log sum_v exp(s_tv), for every row
 *   workspace    device, >= flce_forward_workspace_size bytes, 256-byte aligned; contents are scratch
 *   stream       a hipStream_t (NULL = the null stream)
 * The loss and the per-row terms are bitwise those of flce_forward_backward on the same inputs.
 * Labels outside [0, V) that are not ignore_index are flagged as for flce_forward_backward. Never
 * allocates or synchronises. Returns FLCE_OK or an error code before enqueueing. */
int flce_forward(flce_handle h,
                 const void* hidden, const void* W, const int64_t* labels,
                 int64_t BT, int64_t H, int64_t V, int dtype,
                 int64_t ignore_index, float softcap, int reduction,
                 float* loss, float* loss_rows, float* lse_rows,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Rows given as a batch of sequences (the *_rows entry points). hidden and grad_hidden hold B
 * sequences of T positions, each position a row of H contiguous elements, at arbitrary
 * non-negative element strides; labels hold B x T int64 values at their own strides. With
 * shift = 1, position t < T-1 of sequence b is scored against the label at position t+1 and
 * position T-1 is not a row: the next-token shift of a causal LM, which torchtune issue #1228
 * ("[FEATURE REQUEST] Compile model+loss_fn together") shows being done with sliced .contiguous()
 * copies of the logits and labels. Here no copy is made: rows are addressed where they lie.
 * Row r = b * (T - shift) + t, so BT = B * (T - shift); loss_rows / lse_rows are indexed by r. */
typedef struct {
  int64_t batch;                 /* B >= 0 */
  int64_t seq;                   /* T >= 0 positions per sequence */
  int64_t shift;                 /* 0 or 1 */
  int64_t hidden_stride[2];      /* elements from (b, t) to (b+1, t) and to (b, t+1); multiples of
                                    8 (FLCE_BF16) or 4 (FLCE_FP32) elements, so rows stay 16-byte aligned */
  int64_t grad_hidden_stride[2]; /* the same for grad_hidden; its B x T rows must be disjoint, with
                                    the larger stride stepping past the whole span of the smaller */
  int64_t label_stride[2];       /* elements from (b, t) to (b+1, t) and to (b, t+1) of labels */
} flce_rows;

/* Flags of flce_forward_backward_rows. FLCE_NO_GRAD_HIDDEN / FLCE_NO_GRAD_W leave one gradient out
 * (a frozen input or a frozen LM-head weight, e.g. the frozen base weights of the QLoRA recipe in the
 * torchtune issue #1228 discussion): its GEMM is not run and its pointer may be NULL. Setting both
 * is FLCE_ERR_INVALID_ARG (use flce_forward_rows), and so is accumulating into a gradient that is
 * left out. */
enum { FLCE_ACCUMULATE_GRAD_HIDDEN = 1, FLCE_ACCUMULATE_GRAD_W = 2, FLCE_NO_GRAD_HIDDEN = 4, FLCE_NO_GRAD_W = 8 };

/* Bytes of device workspace flce_forward_backward_rows needs (host-only arithmetic; h may be NULL):
 * flce_workspace_size for BT = B * (T - shift), whatever the strides.
 * Returns FLCE_OK, FLCE_ERR_INVALID_ARG or FLCE_ERR_UNSUPPORTED. */
int flce_workspace_size_rows(flce_handle h, const flce_rows* rows, int64_t H, int64_t V, int dtype,
                             size_t* bytes);

/* flce_forward_backward over rows described by `rows` (see flce_rows), with two more options:
 *   grad_scale   multiplies grad_hidden and grad_W (not the loss): the upstream gradient of the
 *                loss, e.g. 1 / gradient-accumulation steps as in the training loop of the
 *                torchtune issue #1228 discussion; finite, else FLCE_ERR_INVALID_ARG
 *   flags        FLCE_ACCUMULATE_GRAD_HIDDEN: grad_hidden rows get += instead of =
 *                FLCE_ACCUMULATE_GRAD_W: grad_W gets += instead of =
 *                FLCE_NO_GRAD_HIDDEN / FLCE_NO_GRAD_W: that gradient is not computed (NULL allowed)
 *                other bits FLCE_ERR_INVALID_ARG
 *   grad_hidden  device, B x T rows at grad_hidden_stride (written): the rows of the call get their
 *                gradient; with shift = 1 the last position of each sequence gets 0 (or is left as it
 *                is with FLCE_ACCUMULATE_GRAD_HIDDEN)
 * Everything else as for flce_forward_backward (BT there is B * (T - shift) here). With B = 1,
 * T = BT, shift = 0, hidden/grad strides {0, H}, label strides {0, 1}, grad_scale = 1 and no flags
 * it computes exactly what flce_forward_backward computes. */
int flce_forward_backward_rows(flce_handle h,
                               const void* hidden, const void* W, const int64_t* labels,
                               const flce_rows* rows, int64_t H, int64_t V, int dtype,
                               int64_t ignore_index, float softcap, int reduction,
                               float grad_scale, int flags,
                               float* loss, void* grad_hidden, float* grad_W,
                               void* workspace, size_t workspace_bytes, void* stream);

/* flce_forward over rows described by `rows` (grad_hidden_stride is not used). The workspace is
 * flce_forward_workspace_size for BT = B * (T - shift). */
int flce_forward_rows(flce_handle h,
                      const void* hidden, const void* W, const int64_t* labels,
                      const flce_rows* rows, int64_t H, int64_t V, int dtype,
                      int64_t ignore_index, float softcap, int reduction,
                      float* loss, float* loss_rows, float* lse_rows,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Synchronise `stream` and report the status word of the last flce_forward_backward or flce_forward on it:
 * FLCE_OK, or FLCE_ERR_LABEL_RANGE if some label was outside [0, V) and not ignore_index. */
int flce_status(flce_handle h, void* stream);

/* Kernel timing (diagnostics). Between flce_profile_begin and flce_profile_end, every kernel that
 * flce_forward_backward or flce_forward enqueues on the handle is bracketed by a pair of HIP events recorded on the
 * same stream, for at most max_launches launches. flce_profile_end synchronises `stream`, writes for
 * each kernel kind k (FLCE_K_*) the summed duration in ms_out[k] and the launch count in count_out[k]
 * (arrays of FLCE_K_COUNT entries, host memory), and releases the events. Events are created in
 * flce_profile_begin, never inside flce_forward_backward. Returns FLCE_OK, FLCE_ERR_INVALID_ARG or
 * FLCE_ERR_HIP. */
enum { FLCE_K_PREPASS = 0, FLCE_K_FWD = 1, FLCE_K_LSE = 2, FLCE_K_DX = 3, FLCE_K_DX_REDUCE = 4,
       FLCE_K_DW = 5, FLCE_K_FINALIZE = 6, FLCE_K_TRANSPOSE = 7, FLCE_K_ROWS = 8, FLCE_K_ZERO = 9,
       FLCE_K_ROWREF = 10, FLCE_K_ROWFIX = 11, FLCE_K_COUNT = 12 };
int flce_profile_begin(flce_handle h, int max_launches);
int flce_profile_end(flce_handle h, void* stream, double* ms_out, int64_t* count_out);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): flce_forward_backward with no workspace argument. The work runs
 * in a static device array of FLCE_STATIC_SCRATCH_BYTES bytes that the library's code object carries:
 * every device the library is loaded on holds one copy until the process ends; flce_create looks up
 * its address on the handle's device. The call allocates nothing (no hipMalloc, no allocating
 * library routine) and, like flce_forward_backward, never synchronises.
 *   Arguments as for flce_forward_backward, without workspace and workspace_bytes.
 *   Chunk plan: the largest chunk_rows_max' <= the handle's row cap (flce_chunk_plan), a multiple of 256, for
 *   which flce_workspace_size (with chunk_rows_max') fits FLCE_STATIC_SCRATCH_BYTES; the result is
 *   bitwise that of flce_forward_backward on a handle configured with chunk_rows_max'.
 *   Sizes whose workspace exceeds the scratch even with 256-row chunks (e.g. V above ~2^19, or a very
 *   large BT) return FLCE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 * Every call on a device shares that device's one array, and nothing in it needs to start at zero
 * (each call writes every byte it reads): calls on one device that overlap in time (on different
 * streams, or from different handles or threads without ordering between them) race and give wrong
 * results. Order them, e.g. by issuing them on one stream. */
#define FLCE_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int flce_forward_backward_static(flce_handle h,
                                 const void* hidden, const void* W, const int64_t* labels,
                                 int64_t BT, int64_t H, int64_t V, int dtype,
                                 int64_t ignore_index, float softcap, int reduction,
                                 float* loss, void* grad_hidden, float* grad_W, void* stream);

/* Static description of a return code. */
const char* flce_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
