/*
 * muon_mi355x.h - C ABI of the MI355X (gfx950) Muon + AdamW optimizer step.
 *
 * The library updates optimizer state and parameters that the caller owns, on
 * the caller's HIP stream, with hand-written CDNA4 kernels. It never allocates
 * or frees device memory inside a step; scratch memory is a caller-provided
 * workspace whose size the *_workspace_size queries return. The memory it owns
 * is a small pinned host staging area for the per-call descriptor tables
 * (allocated on first use), while profiling is on a pool of HIP events, and
 * for repeated Muon calls (below) the plans and HIP graphs of the last 16 call
 * structures plus one private capture stream per device.
 *
 * Repeated calls: mu_muon_step and mu_muon_orthogonalize key each call on its
 * structure (device, workspace and its size, every buffer pointer, shape,
 * dtype, head count, the step count and coefficients); lr, weight_decay, mu,
 * nesterov, norm_eps and the per-matrix scales are not part of it. A repeated
 * structure skips planning, and from its second call on its kernels are
 * replayed from a HIP graph captured once (the call's descriptor table, which
 * carries those scalars, is still uploaded each call). Results are bit for bit
 * those of launching the kernels one by one, which the library does while
 * profiling is on, for the no-allocation call, and when the environment
 * variable MU_GRAPHS is 0.
 *
 * Large Gram and apply launches (at least 8 tiles per compute unit; not the
 * last apply, which writes the update) run one workgroup per compute unit,
 * each taking tiles from its XCD's queue and then from the other XCDs' queues;
 * results are bit for bit those of one workgroup per tile,
 * which the environment variable MU_PERSIST = 0 selects (read at each call that
 * plans or captures its launches).
 *
 * Gram-side steps: with bf16 Newton-Schulz and three or more cubic steps, a
 * wide block (short side m >= 1024, long side n > m) runs its first steps on
 * the m x m side. Every iterate is X_k = Q_k X_0 for a polynomial Q_k in
 * A_0 = X_0 X_0^T, so A_{k+1} = (B_k B_k) A_k and Q_{k+1} = B_k Q_k are
 * products of commuting symmetric matrices (computed on their upper tiles);
 * X_R = Q_R X_0 is formed before the last step (R = min(steps - 1, 4)), which
 * then runs as usual. This is the same iteration in exact arithmetic, with
 * fewer flops for every n > m, and the result is rounded differently (its
 * error against the float64 iteration stays within the bf16 tolerance). It
 * needs six more m x m buffers per such block in the workspace (the workspace
 * queries include them). The environment variable MU_GRAMSIDE = 0 plans every
 * block with a Gram and an apply per step (read whenever a call or a query plans).
 *
 * Layout rules common to every entry point:
 *   - every tensor is dense, row-major, with no padding between rows;
 *   - parameter, gradient and state buffers of one entry must not overlap each
 *     other or any other entry's buffers;
 *   - bfloat16 buffers are 2-byte aligned, float32 buffers 4-byte aligned (16-
 *     byte alignment and a column count divisible by 4 select the vector path);
 *   - the workspace is 256-byte aligned.
 * Every list is validated as a whole before the first HIP call: any error
 * returns before anything is enqueued, so on error nothing has been modified.
 * A device fault inside a kernel is asynchronous and surfaces at the caller's
 * next synchronisation. Calls that share a workspace must not overlap in time.
 * Streams are passed as void* and must be hipStream_t values (0 = null stream).
 * Calls cannot be captured into a HIP graph: on a capturing stream every
 * entry point returns MU_ERR_INVALID_ARG without enqueuing anything (each
 * call stages its descriptor table through pinned host memory that later
 * calls reuse, so a replayed capture would read another call's table).
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MU_API_VERSION 2

/* element types */
#define MU_F32 0
#define MU_BF16 1

/* arithmetic of the Newton-Schulz products: float32 MFMA on float32 operands,
 * or bfloat16 MFMA operands with float32 accumulation */
#define MU_NS_F32 0
#define MU_NS_BF16 1

/* status codes */
#define MU_OK 0
#define MU_ERR_INVALID_ARG 1 /* null pointer, n < 0, bad size, heads do not divide rows, steps < 0, t < 1 */
#define MU_ERR_DTYPE 2       /* unknown dtype or precision */
#define MU_ERR_LAYOUT 3      /* misaligned buffer, or overlapping buffers */
#define MU_ERR_WORKSPACE 4   /* workspace null, too small, or misaligned */
#define MU_ERR_HIP 5         /* a HIP call failed; detail in mu_last_error() */

/* Largest accepted rows or cols of a matrix (MU_ERR_INVALID_ARG above it): a
 * 256-row strip of the padded long side stays below 2 GiB, the range that the
 * GEMM kernels address with 32-bit offsets. */
#define MU_MAX_DIM (1 << 21)

/*
 * One 2-D weight under the Muon rule.
 *
 * Muon step, four stages (MuonClip Optimizer page, sections "Momentum" and
 * "Newton-Schulz Orthogonalization"; Qwen training-details page, "Confirmed",
 * for per-head orthogonalisation):
 *   M <- mu*M + (1-mu)*G;  U = nesterov ? (1-mu)*G + mu*M : M
 *   for each head h (rows h*rows/num_heads ... (h+1)*rows/num_heads - 1):
 *       X = U_h / (||U_h||_F + norm_eps), transposed when the block is taller
 *       than wide; ns_steps times: X <- a_k X + b_k (X X^T) X + c_k (X X^T)^2 X
 *   W <- W - lr*weight_decay*W - lr*scale*O       (O = X, untransposed)
 *   (with cautious_wd: W <- W - lr*weight_decay*W*[W*u >= 0] - u, u = lr*scale*O)
 *
 * param    [rows, cols] dtype, updated in place (float32 math, bf16 stores
 *          round to nearest even)
 * grad     [rows, cols] same dtype as param, read only
 * momentum [rows, cols] float32, updated in place
 * num_heads >= 1 and divides rows; each head block is its own matrix
 * scale    multiplies the direction in the update (the caller derives it from
 *          the global matrix shape, as the NeMo AutoModel muown_triton page's
 *          _finish contract says); 1.0 is plain Muon
 * norm_out optional float32 [num_heads] device buffer receiving ||U_h||_F
 * ortho_out optional float32 [rows, cols] device buffer receiving O (the
 *          direction before lr and scale), for inspection; NULL to skip
 */
typedef struct mu_matrix {
    void* param;
    const void* grad;
    float* momentum;
    int64_t rows;
    int64_t cols;
    int32_t dtype;
    int32_t num_heads;
    float scale;
    float* norm_out;
    float* ortho_out;
} mu_matrix;

/*
 * Hyper-parameters of one Muon call (one value for every matrix in the list).
 * coeffs: host pointer to ns_steps rows of (a, b, c); NULL means the pages'
 * cubic step (1.5, -0.5, 0) every time. ns_steps = 0 applies the normalised U.
 * norm_eps: any finite value >= 0, 0 included. ||U_h||_F is summed in float64
 * and the normalisation holds at any magnitude of U whose nonzero elements are
 * normal float32 numbers (values below 2^-126 keep the precision their
 * float32 / bfloat16 storage gives them); U_h = 0 gives O_h = 0 for every
 * norm_eps, and NaN or infinity in U_h makes O_h NaN.
 * cautious_wd: 0 or 1. Cautious weight decay, which the nanochat optimizer
 * page ("Muon Step Implementation") names without a formula; the reading used
 * applies the decay only to elements where it moves the weight the same way
 * as the update u = lr*scale*O (W*u >= 0, decided in float32), so O = 0 keeps
 * the plain decay.
 */
typedef struct mu_muon_hparams {
    float lr;
    float weight_decay;
    float mu;
    int32_t nesterov;
    float norm_eps;
    int32_t ns_steps;
    const float* coeffs;
    int32_t ns_precision;
    int32_t cautious_wd;
} mu_muon_hparams;

/*
 * Normalise + Newton-Schulz only, for one 2-D input (no momentum, no update):
 * output = O computed from U = input exactly as in mu_muon_step. input and
 * output share dtype and shape and must not overlap.
 */
typedef struct mu_ortho {
    const void* input;
    void* output;
    int64_t rows;
    int64_t cols;
    int32_t dtype;
    int32_t num_heads;
    float* norm_out;
} mu_ortho;

/*
 * One tensor under the AdamW rule (nanochat optimizer page, "Parameter
 * Grouping Strategy" and "AdamW Step Implementation"; bias corrections are
 * runtime scalars as on the NeMo AutoModel muown_triton page):
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
 *   p <- p - lr*wd*p - lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps)
 * param [numel] dtype, updated in place; grad [numel] same dtype, read only;
 * exp_avg, exp_avg_sq [numel] float32, updated in place. lr and weight_decay
 * are per tensor so parameter groups with different rates share one launch.
 */
typedef struct mu_tensor {
    void* param;
    const void* grad;
    float* exp_avg;
    float* exp_avg_sq;
    int64_t numel;
    int32_t dtype;
    float lr;
    float weight_decay;
} mu_tensor;

/* step is t >= 1, the number of this AdamW step */
typedef struct mu_adamw_hparams {
    float beta1;
    float beta2;
    float eps;
    int64_t step;
} mu_adamw_hparams;

/*
 * QK-Clip after the update (MuonClip Optimizer page, section "QK-Clip"): each
 * attention head whose largest logit magnitude exceeds tau has its query and
 * key weight rows multiplied by gamma = tau / max_logit (gamma formed in
 * float32; each weight becomes the float32 product rounded to nearest even to
 * its dtype). One pair per attention layer.
 *
 * wq         [q_rows, cols] row-major, q_heads equal contiguous row blocks;
 *            scaled in place
 * wk         [k_rows, cols] row-major, k_heads row blocks; scaled in place.
 *            With grouped-query attention (k_heads dividing q_heads) key head
 *            g serves query heads g*G .. g*G+G-1 (G = q_heads / k_heads) and
 *            takes the smallest gamma among them; k_heads == q_heads is the
 *            page's per-head rule.
 * dtype      MU_F32 | MU_BF16, both matrices
 * max_logit  device float32 [q_heads], read only: max |q.k| of each query head
 *            from the forward pass. NaN never exceeds tau (no clip); +inf
 *            gives gamma = 0.
 * gamma_out  optional device float32 [q_heads] receiving the factor applied
 *            to each query head (1 when not clipped); may be NULL.
 * Heads at or below tau are not written at all.
 */
typedef struct mu_qk_pair {
    void* wq;
    void* wk;
    int64_t q_rows;
    int64_t k_rows;
    int64_t cols;
    int32_t q_heads;
    int32_t k_heads;
    int32_t dtype;
    int32_t pad0;
    const float* max_logit;
    float* gamma_out;
} mu_qk_pair;

/* Workspace bytes mu_qk_clip needs for this list (its segment table). */
int mu_qk_clip_workspace_size(const mu_qk_pair* pairs, int32_t n, size_t* bytes);

/* QK-Clip over the whole list in one launch (tau > 0 and finite). Buffers
 * must not overlap; errors as for the other calls (nothing is enqueued). */
int mu_qk_clip(const mu_qk_pair* pairs, int32_t n, float tau, void* workspace, size_t workspace_bytes,
               void* stream);

/* Workspace bytes mu_muon_step needs for this list (n == 0 gives 0). */
int mu_muon_workspace_size(const mu_matrix* mats, int32_t n, const mu_muon_hparams* hp, size_t* bytes);

/* One Muon step over the whole list, enqueued on `stream`. No host sync. */
int mu_muon_step(const mu_matrix* mats, int32_t n, const mu_muon_hparams* hp,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (serving loops, harnesses
 * that forbid hipMalloc): mu_muon_step with its workspace taken from a static
 * device array of MU_NOALLOC_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends. The call allocates no device or pinned
 * memory. A list whose mu_muon_workspace_size exceeds the array is rejected
 * with MU_ERR_WORKSPACE before anything is enqueued. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race, so
 * serialise them, e.g. on one stream. Nothing in the array needs clearing
 * between calls: every buffer a call reads is written earlier in that call.
 * Otherwise exactly mu_muon_step (same kernels, same results).
 */
#define MU_NOALLOC_SCRATCH_BYTES (64u << 20)
int mu_muon_step_noalloc(const mu_matrix* mats, int32_t n, const mu_muon_hparams* hp, void* stream);

/* Workspace bytes mu_muon_orthogonalize needs for this list. */
int mu_ortho_workspace_size(const mu_ortho* xs, int32_t n, const mu_muon_hparams* hp, size_t* bytes);

/* Normalise + orthogonalise each input into its output (lr, weight_decay, mu
 * and nesterov of hp are ignored). */
int mu_muon_orthogonalize(const mu_ortho* xs, int32_t n, const mu_muon_hparams* hp,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mu_adamw_step needs for n tensors (its descriptor table). */
int mu_adamw_workspace_size(int32_t n, size_t* bytes);

/* One AdamW step over the whole list in a single launch. */
int mu_adamw_step(const mu_tensor* ts, int32_t n, const mu_adamw_hparams* hp,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* mu_status_string(int status);

/* Detail of the last error on this host thread ("" if none). */
const char* mu_last_error(void);

/* MU_API_VERSION of the built library. */
int mu_version(void);

/*
 * Kernel timing with HIP events recorded around every launch on the launch
 * stream. mu_profile_enable(1) clears the counters and starts recording;
 * mu_profile_enable(0) stops. mu_profile_read synchronises on the recorded
 * events and reports, for kernel class `kernel` (MU_K_*), the summed duration
 * in milliseconds, the number of launches, and the algorithmic floating-point
 * operations and bytes those launches were given.
 */
#define MU_K_PREP 0      /* momentum + Nesterov + U write + norm partials */
#define MU_K_NORM 1      /* per-head norm finalisation */
#define MU_K_GRAM 2      /* A = X X^T (upper tiles, mirrored); writes B = aI + bA on cubic steps */
#define MU_K_GRAM2 3     /* A A^T for the quintic term; writes B = aI + bA + cA^2 */
                         /* (on the first step B also carries the factor 1/||U||); */
                         /* also the m x m products of Gram-side steps */
#define MU_K_APPLY 4     /* B X (last step fuses the update) */
#define MU_K_FINISH 5    /* update when ns_steps == 0 */
#define MU_K_ADAMW 6     /* AdamW */
#define MU_K_QKCLIP 7    /* QK-Clip rescale (bytes assume every head clipped) */
#define MU_K_FUSED 8     /* every step but the last apply of mp == 128 problems (>= 256 in a call) */
#define MU_K_RESCALE 9   /* exact 2^e rescale of X0 where ||U||_F is outside [2^-24, 2^24] */
#define MU_K_TILEMAP 10  /* per call: each GEMM tile's problem and coordinates, resolved once */
#define MU_K_COUNT 11
int mu_profile_enable(int on);
int mu_profile_read(int kernel, double* total_ms, int64_t* launches, double* flops, double* bytes);
const char* mu_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
