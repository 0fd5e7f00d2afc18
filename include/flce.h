/*
 * flce.h - C ABI of the MI355X (gfx950) fused linear + cross-entropy library.
 *
 * The operation (fused linear + cross-entropy, FLCE):
 *   z      = x . W^T                     logits, [N, V], never stored in memory
 *   lse_i  = log sum_v exp(z_iv)         per-token log-sum-exp
 *   l_i    = lse_i - z_{i, t_i}          per-token cross-entropy
 *   loss   = sum_i l_i  (FLCE_SUM)  or  (1/N) sum_i l_i  (FLCE_MEAN)
 *   D      = s (softmax(z) - onehot(t)), s = grad_loss / N (mean) or grad_loss (sum)
 *   grad_x = D . W        [N, H]
 *   grad_W = D^T . x      [V, H]
 *
 * Sources (pages on fused linear + cross-entropy):
 *   - "Fused linear + cross-entropy" (KernelIndex operation page), description and
 *     Semantics table: x float [tokens, hidden], weight float [vocab, hidden],
 *     target int64 [tokens], loss float [1]; no mutation or aliasing.
 *   - "[example] fused_linear_cross_entropy kernel" (pytorch/helion PR #1268), PR
 *     description: the forward is a tiled matmul with an online softmax that yields
 *     the log-sum-exp and the target logit and keeps the log-sum-exp for the
 *     backward; the backward recomputes the logits and accumulates the input and
 *     weight gradients.
 *   - "feat(FLCE): add helion version of fused linear cross entropy"
 *     (linkedin/Liger-Kernel PR #928), test log: reductions sum and mean; ragged
 *     shapes where out-of-range dlogits must not leak into the weight gradient.
 *
 * Conventions shared by every entry point:
 *   - Pointers named x, W, target, lse, grad_loss, loss, grad_x, grad_W, ws are
 *     DEVICE pointers (memory of the current HIP device).  The library never
 *     allocates, frees or synchronises: the caller owns every buffer, and all work
 *     is enqueued on `hip_stream` (a hipStream_t passed as void*, NULL = default
 *     stream).  Outputs are ready when the stream reaches them.
 *   - Layout: every tensor is contiguous and row-major.  x is [N, H], W is [V, H]
 *     (the nn.Linear weight layout, hidden contiguous), target is [N] int64.
 *   - x and W have the element type `dt`; loss, lse and target_logit are float32;
 *     grad_x and grad_W have the element type `dt` and are overwritten (not
 *     accumulated into).
 *   - Inputs are never written.  No output may overlap an input or another output
 *     (FLCE_ERR_ALIAS), and the workspace may overlap nothing.
 *   - x and W base pointers must be 16-byte aligned and H * sizeof(dt) must be a
 *     multiple of 16 (FLCE_ERR_ALIGN otherwise).
 *   - N, H and V lie in [1, 2^30]; H * sizeof(dt) and V (rounded up to 256) *
 *     sizeof(dt) are at most 8 MiB; each of N x V, N x H and V x H has fewer
 *     than 2^31 tiles of 256 x 256 (FLCE_ERR_SHAPE otherwise; workspace size
 *     functions return 0).
 *   - Targets must lie in [0, V).  The kernels never read out of bounds for other
 *     values: such a token gets a NaN loss term and no one-hot term in D.
 *   - A status other than FLCE_OK means nothing was enqueued, except FLCE_ERR_HIP,
 *     which reports a failed kernel launch.  The library never prints.
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x, W, grad_x and grad_W. */
typedef enum { FLCE_F32 = 0, FLCE_BF16 = 1 } flce_dtype;

/* Reduction of the per-token losses (Liger-Kernel PR #928 test matrix: sum, mean). */
typedef enum { FLCE_MEAN = 0, FLCE_SUM = 1 } flce_reduction;

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_NULL = 1,      /* a required pointer is NULL                          */
  FLCE_ERR_SHAPE = 2,     /* N, H or V <= 0, or a size too large to index         */
  FLCE_ERR_DTYPE = 3,     /* unknown flce_dtype                                   */
  FLCE_ERR_REDUCTION = 4, /* unknown flce_reduction                               */
  FLCE_ERR_ALIAS = 5,     /* an output overlaps an input, another output or ws    */
  FLCE_ERR_ALIGN = 6,     /* misaligned x/W, or H * sizeof(dt) not a multiple of 16 */
  FLCE_ERR_WORKSPACE = 7, /* ws is NULL or smaller than required                  */
  FLCE_ERR_HIP = 8,       /* a HIP launch failed                                  */
  FLCE_ERR_SCRATCH = 9    /* sizes beyond flce_forward_noalloc's static scratch    */
} flce_status;

/* Human-readable name of a status code; never NULL, static storage. */
const char* flce_status_string(flce_status status);

/* Bytes of device workspace flce_forward needs for these sizes (a pure function
 * of its arguments; 0 for invalid arguments). */
size_t flce_forward_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt);

/*
 * Forward pass.  Source: helion PR #1268, PR description (tiled matmul plus an
 * online softmax give the log-sum-exp and the target logit; the log-sum-exp is
 * kept for the backward); KernelIndex Semantics table (shapes, dtypes).
 *
 *   x            [N, H] dt         input activations
 *   W            [V, H] dt         LM-head weight
 *   target       [N] int64         class index per token, in [0, V)
 *   loss         [1] float32       out: sum or mean of the per-token losses
 *   lse          [N] float32       out: per-token log-sum-exp (input to the backward)
 *   target_logit [N] float32       out, may be NULL: z_{i, t_i} per token (NaN for a
 *                                  target outside [0, V))
 *   ws, ws_bytes                   device workspace, >= flce_forward_workspace_bytes
 *
 * The logits are never written to memory.  The result is bitwise reproducible
 * run to run (fixed reduction order, no atomics).
 */
flce_status flce_forward(const void* x, const void* W, const int64_t* target, int64_t N,
                         int64_t H, int64_t V, flce_dtype dt, flce_reduction reduction,
                         float* loss, float* lse, float* target_logit, void* ws,
                         size_t ws_bytes, void* hip_stream);

/*
 * Forward pass without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments and the
 * same results, bit for bit, as flce_forward without `ws`/`ws_bytes`: the
 * forward's workspace is a static device array of FLCE_STATIC_SCRATCH_BYTES
 * inside the library (one per GPU, held until the process ends).  Sizes whose
 * forward workspace (flce_forward_workspace_bytes) exceeds it are refused with
 * FLCE_ERR_SCRATCH before anything is enqueued; for every V, N up to
 * flce_forward_noalloc_max_tokens(V) fits (464384 tokens for V > 256).  The first call on
 * a device looks the array's device address up (hipGetSymbolAddress); a failure
 * there is FLCE_ERR_HIP.  Every call on one GPU shares that GPU's array: calls
 * whose kernels overlap in time on one GPU (e.g. on different streams without
 * ordering) race and give undefined results; calls ordered on one stream are safe.
 * Nothing in the array needs clearing between calls.
 */
#define FLCE_STATIC_SCRATCH_BYTES (16u << 20)
int64_t flce_forward_noalloc_max_tokens(int64_t V);
flce_status flce_forward_noalloc(const void* x, const void* W, const int64_t* target, int64_t N,
                                 int64_t H, int64_t V, flce_dtype dt, flce_reduction reduction,
                                 float* loss, float* lse, float* target_logit, void* hip_stream);

/* Bytes of device workspace flce_backward needs for these sizes (a pure function
 * of its arguments; 0 for invalid arguments): the dlogit panel of its default
 * plan (at most 128 MiB, its shape chosen for these sizes), two of them when all
 * tokens form one chunk and the vocabulary takes several panels (grad_x then runs
 * once per pair), float32 accumulators where a gradient is summed over several
 * launches, and float32 partial tiles: for the split tails (the tiles of a
 * launch's partial last round, cut along K and summed in a fixed order) and, for
 * balanced gradient launches, one partial-sum slot per workgroup plus a 4-byte
 * flag each (the slots and flags of a shape whose launches all fill whole
 * rounds are absent); at most 256 tiles of 256 KiB.  A smaller workspace, down to
 * flce_backward_min_workspace_bytes, makes the backward keep one panel at a time
 * or use smaller panels (more passes); a larger one changes nothing. */
size_t flce_backward_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt);
size_t flce_backward_min_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt);

/*
 * Backward pass.  Source: helion PR #1268, PR description (the backward
 * recomputes the logits and accumulates the input and weight gradients);
 * Liger-Kernel PR #928 (out-of-range dlogit entries must be zero so the weight
 * gradient never picks up NaN or garbage on ragged shapes).
 *
 *   x, W, target, N, H, V, dt, reduction   as for flce_forward (same values)
 *   lse        [N] float32       the lse written by flce_forward for these inputs
 *   grad_loss  [1] float32       device scalar: upstream gradient of loss
 *   grad_x     [N, H] dt         out: D . W
 *   grad_W     [V, H] dt         out: D^T . x
 *   ws, ws_bytes                 device workspace, >= flce_backward_min_workspace_bytes
 *
 * The logit tiles are recomputed from x and W; the dlogits exist only as
 * bounded panels inside `ws` (never the N x V matrix).  Deterministic: no
 * atomic accumulation, every sum in a fixed order (of a tile whose K range two
 * workgroups share, the one taking the head of the range starts from the
 * other's partial sums, handed over through the workspace behind a flag), so
 * repeated calls on one device give identical bits.  The hand-over waits for a
 * workgroup of the same launch; with one or two launches of this kind running
 * on a GPU at once the wait always ends.  Should so many run concurrently (from
 * other streams or processes) that their waiting workgroups hold every CU, the
 * wait gives up after about a second of polling and those tiles' gradients are
 * wrong; callers that share a GPU that widely should not overlap backward calls.
 */
flce_status flce_backward(const void* x, const void* W, const int64_t* target,
                          const float* lse, const float* grad_loss, int64_t N, int64_t H,
                          int64_t V, flce_dtype dt, flce_reduction reduction, void* grad_x,
                          void* grad_W, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Forward and backward in one call, for training steps that always need both
 * (Liger-Kernel PR #928 thread: the gradients can be produced in the same call
 * as the loss).  Same results, bit for bit, as flce_forward followed by
 * flce_backward with the same arguments; the two phases share one workspace.
 *
 *   grad_loss   [1] float32 device scalar, or NULL for 1 (the gradient of loss
 *               with respect to itself)
 *   loss, lse   as for flce_forward; lse is also the backward's input
 *   grad_x, grad_W  as for flce_backward
 *   ws, ws_bytes    >= flce_forward_backward_workspace_bytes (smaller, down to the
 *               backward's minimum plus 256 bytes, also works with smaller panels)
 */
size_t flce_forward_backward_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt);
flce_status flce_forward_backward(const void* x, const void* W, const int64_t* target, int64_t N,
                                  int64_t H, int64_t V, flce_dtype dt, flce_reduction reduction,
                                  const float* grad_loss, float* loss, float* lse, void* grad_x,
                                  void* grad_W, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Kernel timing, for benchmarks: the *_timed variants behave exactly like the
 * calls above and, in addition, record caller-created HIP events (hipEvent_t
 * handles passed as void*) on `hip_stream`: events[0] before the first kernel and
 * events[k + 1] right after kernel k, for the first n_events - 1 kernels.  kinds[k]
 * receives the flce_kernel of launch k, n_launches the number of kernels enqueued
 * (also those beyond the event capacity).  `timing` may be NULL.  A failed event
 * record is reported as FLCE_ERR_HIP.
 */
typedef enum {
  FLCE_K_FWD_PARTIAL = 0, /* logit tiles + online (max, sum-exp) per vocabulary split */
  FLCE_K_FWD_COMBINE = 1, /* split merge -> lse, per-token loss, scalar loss         */
  FLCE_K_FWD_LOSS = 2,    /* (no longer launched: fwd_combine writes the loss)     */
  FLCE_K_BWD_DLOGITS = 3, /* logit tile recompute -> dlogit panel                   */
  FLCE_K_BWD_GRAD_W = 4,  /* grad_W rows of one panel                              */
  FLCE_K_BWD_GRAD_X = 5,  /* grad_x rows of one token chunk, one panel or a pair    */
  FLCE_K_FILL = 6,        /* writes the implicit grad_loss of 1                    */
  FLCE_K_BWD_GX_REDUCE = 7, /* adds the K-split partial sums of a grad_x launch      */
  FLCE_K_BWD_ATOMIC = 8,  /* fused dlogit tile + float32 atomic gradient partials  */
  FLCE_K_ZERO = 9,        /* zeroes a float32 accumulator                          */
  FLCE_K_CAST = 10,       /* float32 accumulator -> bfloat16 output                */
  FLCE_K_TAIL_FIXUP = 11, /* adds the K pieces of a launch's split tail tiles (and, for
                             dlogits, forms the dlogits from the summed logits)     */
  FLCE_K_TAIL_PIECES = 12 /* K pieces of the split tail tiles of a backward launch   */
} flce_kernel;

typedef struct {
  void* const* events; /* in: hipEvent_t handles                          */
  int n_events;        /* in: number of handles                           */
  int* kinds;          /* out: flce_kernel per launch, >= n_events - 1     */
  int n_launches;      /* out: kernels enqueued by the call                */
} flce_timing;

flce_status flce_forward_timed(const void* x, const void* W, const int64_t* target, int64_t N,
                               int64_t H, int64_t V, flce_dtype dt, flce_reduction reduction,
                               float* loss, float* lse, float* target_logit, void* ws,
                               size_t ws_bytes, void* hip_stream, flce_timing* timing);

flce_status flce_backward_timed(const void* x, const void* W, const int64_t* target,
                                const float* lse, const float* grad_loss, int64_t N, int64_t H,
                                int64_t V, flce_dtype dt, flce_reduction reduction, void* grad_x,
                                void* grad_W, void* ws, size_t ws_bytes, void* hip_stream,
                                flce_timing* timing);

/*
 * Token-chunked backward, for comparison with flce_backward's bounded panels.
 * Source: Liger-Kernel PR #928 thread, where the author replaces the fully fused
 * backward by a chunk backward that recomputes the logits of one chunk of tokens
 * over the whole vocabulary and then accumulates the input and weight gradients.
 * Arguments and results (up to rounding order) as for flce_backward_timed, plus
 *
 *   chunk_tokens  tokens per chunk, >= 1 (FLCE_ERR_SHAPE otherwise); rounded up to
 *                 a multiple of 256 and capped at N rounded up to 256.  Each
 *                 chunk's dlogits [chunk, V] go to the workspace; grad_x rows of
 *                 the chunk come from one contraction over V; grad_W is summed
 *                 over the chunks (through a float32 [V, H] buffer in the
 *                 workspace for bfloat16, in place for float32).
 *   ws, ws_bytes  >= flce_backward_chunked_workspace_bytes(N, H, V, dt, chunk_tokens)
 *                 (0 for invalid arguments); no smaller-panel fallback
 *   timing        as for the *_timed variants; may be NULL
 */
size_t flce_backward_chunked_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt,
                                             int64_t chunk_tokens);
flce_status flce_backward_chunked(const void* x, const void* W, const int64_t* target,
                                  const float* lse, const float* grad_loss, int64_t N, int64_t H,
                                  int64_t V, flce_dtype dt, flce_reduction reduction,
                                  int64_t chunk_tokens, void* grad_x, void* grad_W, void* ws,
                                  size_t ws_bytes, void* hip_stream, flce_timing* timing);

/*
 * Backward with float32 atomics, for comparison with flce_backward's bounded
 * dlogit panels.  Source: helion PR #1268, PR description (the backward
 * recomputes the logits, and the weight gradient is accumulated with an atomic
 * add); Liger-Kernel PR #928 thread (the two in-loop atomic adds are discussed as
 * a possible bottleneck of the fused backward).  One fused kernel walks the
 * (256-token tile, 256-vocabulary tile) pairs: it recomputes the logit tile,
 * forms the dlogit tile (kept in a 256 x 256 slot of `ws` per workgroup, never the
 * N x V matrix), contracts it with the tile's rows of W and x over the hidden
 * size and adds both gradients' partial sums into float32 buffers with atomic
 * adds (grad_x and grad_W themselves for float32; buffers in `ws`, then cast to
 * bfloat16, for bfloat16).  Arguments and results (up to rounding order) as for
 * flce_backward_timed; not bitwise reproducible (atomic order).
 *
 *   ws, ws_bytes  >= flce_backward_atomic_workspace_bytes(N, H, V, dt) (0 for
 *                 invalid arguments): 256 dlogit tiles of 256 x 256 plus, for
 *                 bfloat16, float32 [N, H] and [V, H] accumulators
 *   timing        as for the *_timed variants; may be NULL
 */
size_t flce_backward_atomic_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt);
flce_status flce_backward_atomic(const void* x, const void* W, const int64_t* target,
                                 const float* lse, const float* grad_loss, int64_t N, int64_t H,
                                 int64_t V, flce_dtype dt, flce_reduction reduction, void* grad_x,
                                 void* grad_W, void* ws, size_t ws_bytes, void* hip_stream,
                                 flce_timing* timing);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
