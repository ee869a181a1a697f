/*
 * flce.h - C ABI of the MI355X (gfx950) fused linear cross-entropy library.
 *
 * Fused linear cross-entropy (FLCE) projects token hidden states through the
 * LM-head weight and applies softmax cross-entropy, forward and backward in
 * one call, without materialising the [N,V] logits: tokens are processed in
 * chunks, each chunk's logits buffer is overwritten in place by its
 * gradient, dx is produced per chunk and dW is accumulated across chunks
 * (the four-step loop of the core-idea section of the "Fused Linear
 * Cross-Entropy" page, 42jerrykim.github.io).  Because it is the last layer,
 * the gradients are finished inside the forward call.
 *
 * For x[N,H], W[V,H] and targets t[N] the call returns
 *   loss = (1/N) sum_n ( lse_n - z[n,t_n] ),  z = x W^T,  lse_n = ln sum_v e^{z[n,v]}
 *   dx   = G W,   dW = G^T x,   G = (softmax(z) - onehot(t)) / N
 * (loss and gradient equations of the "Unsloth deep architecture" page,
 * techknowgenie.com, streaming Fast CrossEntropy section; mean reduction and
 * the 1/N on both gradients as in the code sample of the FLCE page).
 *
 * Conventions shared by every entry point:
 *  - All tensors are caller-owned DEVICE pointers on the handle's device,
 *    row-major and contiguous, 16-byte aligned.
 *  - `stream` is a hipStream_t (passed as void*).  Every kernel of a call is
 *    enqueued on it and the call returns after enqueueing: the call itself
 *    neither synchronises the host nor enqueues anything on the null stream
 *    (the stream and event ordering rules of the async continuous-batching
 *    page, pogovet.com, "default stream" and "events" sections).  Results
 *    are valid once the stream reaches that point.  What does synchronise:
 *    growing the workspace (hipMalloc/hipFree: flce_reserve, or the first call
 *    that needs more), flce_check (the given stream), flce_profile_read (the
 *    recorded events, then a blocking copy of the clock counters) and
 *    flce_destroy (hipFree).
 *  - No output may overlap an input or another output (byte ranges are
 *    compared; INVALID_ARG otherwise): later chunks read x and W after
 *    earlier chunks have written dx and dW.
 *  - Validation happens before any launch; a call that returns an error
 *    writes nothing.  Nothing aborts and no exception crosses the ABI.
 *  - A handle owns one workspace, shared by all its calls: calls on one
 *    handle must be ordered on the device (the same stream, or streams
 *    ordered by events), and a handle must not be used by two host threads
 *    at the same time.  Distinct handles share nothing.
 *  - Graph capture: a call captured into a HIP graph enqueues kernels only
 *    (no memset, no allocation).  Under capture nothing may be allocated, so
 *    a captured call whose workspace is not yet large enough (flce_reserve it
 *    first, or run the call once eagerly) fails with UNSUPPORTED.  A graph
 *    holds the handle's workspace address: after the first captured call the
 *    workspace is pinned for the handle's lifetime, and a later call or
 *    flce_reserve that would need a larger one fails with UNSUPPORTED instead
 *    of moving it.  A captured graph must not be replayed after flce_destroy.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = 1,   /* null pointer, N/H/V < 1, bad enum value */
  FLCE_ERR_UNSUPPORTED = 2,   /* H % 8 != 0, misaligned pointer, dtype combination not built, size limits */
  FLCE_ERR_OOM = 3,           /* workspace allocation failed or exceeds cfg.workspace_limit */
  FLCE_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
  FLCE_ERR_DATA = 5           /* flce_check: a target id was outside [0, V) */
} flce_status_t;

typedef enum { FLCE_BF16 = 0, FLCE_FP32 = 1 } flce_dtype_t;

typedef enum {
  FLCE_CHUNKED = 0,           /* token chunks; one [C,V] buffer overwritten in place by dlogits */
  FLCE_FUSED = 1              /* two passes, logits recomputed: pass 1 per-token log-sum-exp (no
                                 logits stored); pass 2 cuts the (token x vocabulary) plane into
                                 blocks (planned per launch, at most 1536 tiles of 256 x 256) and
                                 runs in steps: one kernel recomputes the logits of up to 1.5 GiB
                                 of blocks and stores them as dlogits in workspace slots, a second
                                 forms the blocks' dx and dW tile products and adds them into
                                 fp32 accumulators with atomics.  With fp32 dx and dW, pass 2 runs
                                 once over all N tokens after every chunk's pass 1 (dx and dW are
                                 their own accumulators).  Otherwise it runs once per chunk: bf16
                                 dx through an fp32 [chunk, H] accumulator; bf16 dW with one token
                                 block per launch, so that each dW tile has one product per chunk
                                 and is stored (added after the first chunk) with no accumulator.
                                 bf16 inputs only.  Results are not bitwise repeatable.  Size
                                 limit: (V + 256) * H * 4 and (chunk + 256) * H * 4 below 4 GiB
                                 (32-bit offsets into the accumulators), else UNSUPPORTED. */
} flce_variant_t;

typedef struct {
  int32_t in_dtype;           /* dtype of x and W: FLCE_BF16 or FLCE_FP32 */
  int32_t dx_dtype;           /* dtype of dx: FLCE_BF16 (bf16 inputs only) or FLCE_FP32 */
  int32_t dw_dtype;           /* dtype of dW: FLCE_BF16 (bf16 inputs only) or FLCE_FP32 */
  int32_t variant;            /* flce_variant_t */
  int32_t device;             /* HIP device ordinal the handle and its workspace belong to */
  int32_t reserved;           /* must be 0 */
  int64_t workspace_limit;    /* bytes; 0 = no limit.  A plan needing more fails with FLCE_ERR_OOM */
} flce_config_t;

typedef struct flce_handle_s* flce_handle_t;

/* Creates a handle: the configuration (dtypes, variant, device) and, later, the workspace that
 * holds the chunk's logits buffer of the FLCE page's core idea (one [C,V] buffer reused by every
 * chunk).  The pages define no handle; it is the plumbing of this C interface, which keeps that
 * buffer between calls instead of allocating it per call.  No device memory is allocated yet.
 * `*out` receives the handle, owned by the caller until flce_destroy.
 * Errors: INVALID_ARG (null cfg/out, bad enum, reserved != 0, negative limit or device),
 *         UNSUPPORTED (fp32 inputs with a bf16 output, or the fused variant with fp32 inputs),
 *         HIP (device ordinal not usable). */
flce_status_t flce_create(const flce_config_t* cfg, flce_handle_t* out);

/* Frees the handle's workspace and the handle (hipFree: synchronises the device).  Interface
 * plumbing, like flce_create.  NULL is a no-op.  Always returns FLCE_OK. */
flce_status_t flce_destroy(flce_handle_t h);

/* One fused forward+backward pass.
 *   x       [N,H]  cfg.in_dtype, read-only
 *   W       [V,H]  cfg.in_dtype, read-only
 *   targets [N]    int64, each expected in [0,V).  An id outside that range never faults: that
 *                  token's loss is NaN (so `loss` is NaN), its gradient row is the plain softmax,
 *                  and a device flag is raised that flce_check reports as FLCE_ERR_DATA.
 *   chunk          tokens per chunk; <= 0 selects the automatic size (flce_effective_chunk)
 *   loss    [1]    fp32, overwritten with the mean loss over the N tokens
 *   dx      [N,H]  cfg.dx_dtype, overwritten
 *   dW      [V,H]  cfg.dw_dtype, overwritten
 * The workspace grows on demand (hipMalloc/hipFree, which synchronise the device); call
 * flce_reserve beforehand to keep allocation out of timed or captured regions.
 * Errors: INVALID_ARG, UNSUPPORTED (also: a captured call or a pinned workspace that would
 * need to grow), OOM (allocation failed or cfg.workspace_limit exceeded; outputs untouched),
 * HIP. */
flce_status_t flce_forward_backward(flce_handle_t h, const void* x, const void* W,
                                    const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                    int64_t chunk, float* loss, void* dx, void* dW, void* stream);

/* As flce_forward_backward, and additionally writes the per-token log-sum-exp
 * lse_n = ln sum_v exp(z[n,v]) (fp32, [N]) to `lse` when it is not NULL. */
flce_status_t flce_forward_backward_ex(flce_handle_t h, const void* x, const void* W,
                                       const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                       int64_t chunk, float* loss, void* dx, void* dW, float* lse,
                                       void* stream);

/* Options of flce_forward_backward_opt: the loss reduction, masked tokens, accumulation into
 * the gradient outputs, and a forward-only (loss) mode.  These are the conventions of PyTorch's
 * cross_entropy(reduction=..., ignore_index=...); the FLCE page's interface fixes none of them
 * (its listing is the mean over all tokens, overwriting dx and dW, which is the default). */
typedef enum {
  FLCE_MEAN = 0,              /* loss and gradients divided by the number of counted tokens */
  FLCE_SUM = 1                /* not divided */
} flce_reduction_t;

enum {
  FLCE_ACCUMULATE = 1,        /* dx += d loss / d x and dW += d loss / d W (sum in fp32, one rounding
                                 to the output dtype per call); default: overwrite */
  FLCE_FORWARD_ONLY = 2       /* loss (and lse) only: dx, dW are not touched and may be NULL, and the
                                 chunked variant needs no logits buffer */
};

typedef struct {
  int32_t reduction;          /* flce_reduction_t */
  int32_t flags;              /* FLCE_ACCUMULATE | FLCE_FORWARD_ONLY (not both) */
  int32_t ignore_on;          /* 1: tokens whose target equals ignore_index count for nothing: no loss,
                                 a zero gradient row, not in the mean's denominator.  A mean over
                                 zero counted tokens is NaN (0/0) with zero gradients. */
  int32_t reserved;           /* must be 0 */
  int64_t ignore_index;       /* e.g. -100; any value, inside [0, V) or not */
} flce_options_t;

/* flce_forward_backward_ex with options; opt == NULL gives the defaults (mean, overwrite, no
 * ignored tokens, gradients).  The count of counted tokens is taken on the device.
 * Errors: as flce_forward_backward, and INVALID_ARG for an unknown reduction or flag, both
 * flags at once, ignore_on outside {0, 1}, reserved != 0, or NULL dx / dW with gradients. */
flce_status_t flce_forward_backward_opt(flce_handle_t h, const void* x, const void* W,
                                        const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                        int64_t chunk, const flce_options_t* opt, float* loss, void* dx,
                                        void* dW, float* lse, void* stream);

/* flce_forward_backward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It calls no hipMalloc, hipFree
 * or allocating library routine: the call's workspace lives in a library-owned array of 256 MiB
 * per device (a static __device__ array, `scratch`; each GPU the library runs on holds its own
 * copy until the process ends), whose address is looked up once per device by the first such
 * call on it (hipGetSymbolAddress; make that first call outside graph capture).
 *   Arguments, layouts, results and errors as for flce_forward_backward; chunked variant only
 *   (UNSUPPORTED for a fused handle).  The handle's own workspace is not used.
 *   chunk > 0: used as given (clamped to N); the call fails with UNSUPPORTED, writing nothing, if
 *     its workspace (flce_workspace_bytes for that chunk) exceeds 256 MiB - 256 bytes.
 *   chunk <= 0: the automatic chunk (flce_effective_chunk), halved until the workspace fits (512
 *     tokens at V = 128,256, H = 4,096; a smaller chunk re-reads W more often, so such calls are
 *     slower); UNSUPPORTED if not even one token fits (12 bytes per token of N are needed too).
 * Every call on a GPU uses that GPU's one array and leaves its contents behind: calls on the
 * same device that overlap in time (on different streams, through any handle) race and give
 * wrong results; order them on the device.  An out-of-range target raises a flag in the array
 * that flce_check of any handle on that device reports (and clears).  No profiling events. */
flce_status_t flce_forward_backward_noalloc(flce_handle_t h, const void* x, const void* W,
                                            const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                            int64_t chunk, float* loss, void* dx, void* dW, void* stream);

/* Workspace bytes a flce_forward_backward_opt call with these sizes and options needs (0 for
 * invalid sizes or options); forward only needs no logits buffer and no gradient accumulators. */
size_t flce_workspace_bytes_opt(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk,
                                const flce_options_t* opt);

/* The final RMSNorm of the model in front of the head, then the loss (an upstream
 * fusion).  From the "Unsloth deep architecture" page, section on RMSNorm and its backward as
 * one kernel:
 *   x = hidden / RMS(hidden) * gamma,  RMS(h) = sqrt(mean_k h_k^2 + eps)  (per token row),
 * then the loss of flce_forward_backward_opt on x.  Returns dhidden = d loss / d hidden,
 * dgamma = d loss / d gamma (sum over tokens of dx * hidden / RMS) and dW.  Processed per token
 * chunk: the chunk's x (input dtype, rounded once) and its fp32 d loss / d x live only in the
 * workspace; neither reaches HBM for all N.
 *   hidden  [N,H]  cfg.in_dtype, read-only         gamma   [H]  cfg.in_dtype, read-only
 *   dhidden [N,H]  cfg.dx_dtype                    dgamma  [H]  cfg.dw_dtype
 *   dW      [V,H]  cfg.dw_dtype                    eps >= 0 (finite)
 * Options as for flce_forward_backward_opt (accumulate adds into dhidden, dgamma and dW;
 * forward only needs none of them).  Chunked variant only; H <= 32768.
 * Errors: INVALID_ARG (NULL pointers, bad options, eps < 0 or NaN, overlapping tensors),
 * UNSUPPORTED (fused variant, H > 32768, alignment, size limits), OOM, HIP. */
flce_status_t flce_rmsnorm_forward_backward(flce_handle_t h, const void* hidden, const void* gamma, float eps,
                                            const void* W, const int64_t* targets, int64_t N, int64_t H,
                                            int64_t V, int64_t chunk, const flce_options_t* opt, float* loss,
                                            void* dhidden, void* dgamma, void* dW, float* lse, void* stream);

/* Workspace bytes flce_rmsnorm_forward_backward needs for these sizes and options (0 if invalid). */
size_t flce_rmsnorm_workspace_bytes(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk,
                                    const flce_options_t* opt);

/* Token chunk the call would use (for bf16 inputs): chunk clamped to [1, N] when positive; for
 * chunk <= 0 the size rule of the FLCE page's trade-offs section, next_pow2(ceil(N / ceil(V/H))),
 * raised to at least 4096 tokens (on MI355X the chunk's GEMMs run faster with the longer token
 * contraction, and below ~2048 the per-chunk re-read of W dominates), capped at 8192 and so that
 * the chunk's logits buffer stays within 1.5 GB, then clamped to N.  Returns 0 for invalid sizes. */
int64_t flce_effective_chunk(int64_t N, int64_t H, int64_t V, int64_t chunk);

/* Workspace bytes a call with these sizes needs (0 for invalid sizes or a NULL handle): the
 * chunk's logits buffer (C x ceil(V/256)*256 elements of the input dtype; the buffer the FLCE
 * page's core idea overwrites in place with dlogits), the per-row log-sum-exp partials of the
 * online softmax (the streaming CE kernel of the "Unsloth deep architecture" page: a running
 * maximum and sum per row and 256-wide vocabulary tile, 8 bytes each), 12 bytes per token (target
 * logit, lse, loss), and split-K partials of the dx product when the chunk has few output tiles. */
size_t flce_workspace_bytes(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk);

/* Allocates the workspace for these sizes now (no-op if already large enough); synchronises the
 * device when it allocates.  Interface plumbing: keeps allocation out of timed or captured calls.
 * Errors: INVALID_ARG, UNSUPPORTED (sizes; or a pinned workspace that would need to grow), OOM,
 * HIP. */
flce_status_t flce_reserve(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk);

/* Synchronises `stream`, then reports and clears the device-side data flag:
 * FLCE_ERR_DATA if any call since the last check saw a target outside [0,V), else FLCE_OK.
 * Targets are class ids in [0, V) (the cross-entropy equation of the "Unsloth deep architecture"
 * page indexes the logits by the target); a kernel cannot return an error without a host
 * synchronisation, so an out-of-range id is recorded on the device and reported here.
 * Errors: INVALID_ARG (NULL handle), HIP. */
flce_status_t flce_check(flce_handle_t h, void* stream);

/* ---- per-kernel timing (tracing) ----------------------------------------------------
 * When enabled, every launch a call makes is bracketed by HIP events recorded on the
 * caller's stream, so each kernel's duration is the time between the event before it and
 * the event after it on that stream.  The GEMM kernels (logits_lse, dx, dw) also time each of
 * their workgroups with the shader-clock counter and the 100 MHz real-time counter, whose ratio
 * is the shader clock the GEMMs actually ran at.  Enabling (or disabling) resets the statistics;
 * enabling allocates 2 * 8 bytes of device memory per kernel kind once per handle, which the next
 * call clears on its stream.  Measurement plumbing (the per-kernel times and flops feed the
 * roofline: 2 N H V flops per GEMM launch, the forward 2PD and backward 4PD of the compute
 * section of "Transformer Math 101"). */
typedef struct {
  char name[32];          /* kernel name, e.g. "logits_lse", "dx", "dw" */
  int64_t launches;       /* launches timed since the last reset */
  double total_ms;        /* summed durations of those launches */
  double flops;           /* summed algorithmic flops: 2*rows*V*H for each GEMM launch, 0 otherwise */
  double bytes;           /* summed algorithmic HBM bytes (each operand read once, each result written once) */
  double sclk_mhz;        /* GEMM kernels: mean shader clock over their workgroups' lifetimes, MHz (0: not timed) */
} flce_kernel_stat_t;

/* Errors: INVALID_ARG (null handle), OOM, HIP. */
flce_status_t flce_profile_enable(flce_handle_t h, int enable);

/* Synchronises on the recorded events, folds them into the statistics and copies up to
 * `capacity` entries (one per kernel that ran) into `out`; `*count` receives the number of
 * entries available.  The clock counters come back by a blocking device-to-host copy.
 * Errors: INVALID_ARG, HIP. */
flce_status_t flce_profile_read(flce_handle_t h, flce_kernel_stat_t* out, int capacity, int* count);

/* Static description of a status code (never NULL; "unknown flce status" for other values).
 * Interface plumbing: the error convention of this C interface (status codes, no aborts). */
const char* flce_status_string(flce_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
