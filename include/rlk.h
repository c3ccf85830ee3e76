/*
 * rlk.h — C ABI of the fused, deterministic selected-token log-probability
 * operator ("linear_logp") for AMD Instinct MI355X (gfx950).
 *
 * The operator ("Announcing RL-Kernel for vime", sections "Key Capabilities"
 * and "Why the Fused Path Wins"): from bf16 hidden states h [T,H], the bf16
 * LM-head weight W [V,H] and int32 target ids y [T], compute per row
 *
 *     logp[t] = z[t, y_t] - log(sum_v exp(z[t, v])),   z = h W^T,
 *
 * without ever storing the [T, V] logits, plus the deterministic gradient of
 * sum_t g_t * logp_t with respect to h and W.
 *
 * Numerical contract (version RLK_CONTRACT_VERSION).  The pages require the
 * partitioning, merge order, precision, rounding points and primitives to be
 * fixed ("vLLM RL-Kernel v0.1.0: Bitwise Train-Rollout Consistency on ROCm",
 * section "The Numerical Execution Contract") but publish no constants; the
 * ones below are this library's own:
 *   - logits: bf16 x bf16 products accumulated in fp32 by one
 *     v_mfma_f32_16x16x32_bf16 chain per logit, k ascending in steps of 32
 *     (version 2; version 1, a build with RLK_MFMA=32, used
 *     v_mfma_f32_32x32x16_bf16 in steps of 16, which gives other bits);
 *   - the vocabulary is split into 32 contiguous splits of width
 *     S = ceil(V_global / 32); each split into chunks of 128 columns anchored
 *     at the split start (the last chunk may be short);
 *   - chunk statistics (m, s): m = max of the chunk's logits, s = sum of
 *     exp(z - m) over the columns in four interleaved parts (column c in
 *     part (c / 4) mod 4), each a balanced pairwise tree in ascending
 *     column order, combined as (s0 + s1) + (s2 + s3) (version 1: two
 *     parts, (c / 4) mod 2, s0 + s1); chunks of a split are folded left to
 *     right with the operator  (ma,sa) + (mb,sb) = (m, sa*e(ma-m) + sb*e(mb-m)),
 *     m = max(ma,mb); splits are merged with a balanced binary tree;
 *   - exp(x) = exp2(x * log2(e)) and log(x) = log2(x) * ln(2) on the
 *     hardware exp2/log2, every operation rounded separately (no FMA
 *     contraction);
 *   - logp = (z_t - m) - log(s), lse = m + log(s), both fp32.
 * Consequences: a row's results depend only on that row (batch- and
 * order-invariant), repeated runs are bit-identical, and merging the partials
 * of equal, aligned power-of-two blocks of splits reproduces the unsharded
 * result bit for bit.
 *
 * Conventions for every call below:
 *   - tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *     16-byte aligned; the caller owns every buffer and the library keeps no
 *     pointer after the call returns;
 *   - `stream` is a hipStream_t (NULL = the default stream); calls only
 *     enqueue work on it, never synchronise and never allocate device memory;
 *   - scratch space is the caller's `ws` buffer of at least
 *     rlk_workspace_bytes(...) bytes, used only until the enqueued work ends;
 *   - outputs are overwritten, never accumulated;
 *   - host-detectable errors return a status and enqueue nothing; data errors
 *     the host cannot see (a target outside [0,V) that is not ignore_index,
 *     or no part owning an active target) give NaN in that row's logp, and
 *     in the backward NaN in that row's grad_h and in grad_W (the row's
 *     loss is undefined, so is every gradient it reaches);
 *   - H must be a multiple of 64 (the MFMA tile engine's k-block); the
 *     Qwen3 LM-head shapes (H = 2048, 4096) are;
 *   - T == 0 returns RLK_OK without launching anything (after the shape
 *     checks); row-indexed pointers may then be NULL.
 */
#ifndef RLK_H_
#define RLK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The contract version of the default build; rlk_contract_version() returns
 * the one the library was built with. */
#define RLK_CONTRACT_VERSION 2
#define RLK_NSPLIT 32
#define RLK_CHUNK 128

typedef int32_t rlk_status;
enum {
  RLK_OK = 0,
  RLK_ERR_NULL_ARG = 1,              /* a required pointer is NULL */
  RLK_ERR_BAD_SHAPE = 2,             /* T<0, H<=0 or H%64!=0, V<=0, sizes too large */
  RLK_ERR_BAD_ALIGNMENT = 3,         /* a tensor pointer is not 16-byte aligned */
  RLK_ERR_UNALIGNED_VOCAB_RANGE = 4, /* a vocab range that is not an aligned block of splits */
  RLK_ERR_WORKSPACE_TOO_SMALL = 5,   /* ws_bytes < rlk_workspace_bytes(...) */
  RLK_ERR_HIP = 6,                   /* a HIP runtime call or kernel launch failed */
  RLK_ERR_UNSUPPORTED_DEVICE = 7,    /* the current device is not gfx950 */
  RLK_ERR_BAD_ARG = 8                /* another invalid argument (e.g. n_parts < 1) */
};

/* Per-row statistics of one vocabulary range (16 bytes).
 * m = max logit over the range, s = sum of exp(z - m) over the range,
 * z_target = the target's logit when owned == 1 (target inside the range),
 * else 0.  Rows whose target is ignore_index hold {-inf, 0, 0, 0}.
 * "Why the Fused Path Wins" (third reason): ranks combine only these
 * statistics to obtain the global selected log-probability. */
typedef struct {
  float m;
  float s;
  float z_target;
  uint32_t owned;
} rlk_lse_partial_t;

enum { RLK_OP_FWD = 0, RLK_OP_BWD = 1, RLK_OP_PARTIAL = 2 };

/* Identifier of the numerical contract above; results with equal version
 * and equal inputs are bit-identical. */
int32_t rlk_contract_version(void);

/* Static text for a status code. */
const char* rlk_status_string(rlk_status s);

/* Detail of the last error on the calling thread (e.g. the HIP error text);
 * empty string when none. */
const char* rlk_last_error_message(void);

/* Workspace bytes needed by `op` (RLK_OP_*) for T rows, hidden size H and a
 * vocabulary of V rows (for RLK_OP_PARTIAL: V = V_global, the size of the
 * whole vocabulary).  Returns 0 for invalid arguments.
 *
 * The backward processes the vocabulary in groups of splits whose bf16 dz
 * block (T rounded up to 256, times the group's padded columns) fits a
 * budget of 2.5 GiB; the environment variable RLK_DZ_BUDGET_MB (read at
 * every call, capped at 3584) sets another.  RLK_GRAD_H_PASSES = 0 / 1
 * forces grad_h's whole-tile or row-pass form (chosen by batch size
 * otherwise).  Neither changes a result bit; the budget changes the
 * workspace size, so a caller that sets it must size the workspace under
 * the same setting. */
size_t rlk_workspace_bytes(int32_t op, int64_t T, int64_t H, int64_t V);

/* Forward ("Announcing RL-Kernel for vime", "Key Capabilities": the
 * log-softmax of hidden @ W^T at the target, logits never materialised).
 *   h     bf16 [T,H]    hidden states
 *   W     bf16 [V,H]    LM-head weight, one row per vocabulary entry
 *   y     int32 [T]     target ids; rows equal to ignore_index are inactive
 *   logp  fp32 [T] out  selected log-probability (0 for inactive rows)
 *   lse   fp32 [T] out  log-sum-exp of the row's logits, the state the
 *                       backward needs (0 for inactive rows); may be NULL
 * Requires H % 64 == 0. */
rlk_status rlk_linear_logp_fwd(const void* h, const void* W, const int32_t* y,
                               int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                               float* logp, float* lse,
                               void* ws, size_t ws_bytes, void* stream);

/* Backward of L = sum_t g[t] * logp[t] ("Announcing RL-Kernel for vime",
 * "Key Capabilities": the full-gradient path, gradients reach both the
 * hidden states and the weight).  Recomputes the logits chunk by chunk; no
 * atomics, so results are bit-identical across runs.
 *   lse     fp32 [T]       the forward's lse output (must come from the forward)
 *   g       fp32 [T]       upstream gradient dL/dlogp
 *   grad_h  bf16 [T,H] out fp32-accumulated over the whole vocabulary and
 *                          rounded to bf16 once; zero rows for inactive rows;
 *                          may be NULL (not computed)
 *   grad_W  fp32 [V,H] out written once per element; may be NULL
 * Row ordering: grad_W sums rows in ascending row order.
 * An active row whose target lies outside [0, V) makes its grad_h row NaN
 * and, since every grad_W element sums over all active rows, grad_W NaN. */
rlk_status rlk_linear_logp_bwd(const void* h, const void* W, const int32_t* y,
                               const float* lse, const float* g,
                               int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                               void* grad_h, float* grad_W,
                               void* ws, size_t ws_bytes, void* stream);

/* Save-logits variant of the forward and backward: the pages' published
 * fast path ("Announcing RL-Kernel for vime", section "Validation and
 * Benchmarks": FusedLinearLogpSM90Op in the save-logits fused-tile
 * full-gradient path; section "Why the Fused Path Wins", fourth reason: a
 * controlled workspace traded for backward speed).  The forward also stores
 * the fp32 logits of the active rows into the caller's buffer `zsave`; the
 * backward then forms dz from them instead of recomputing the logit tiles
 * (6 instead of 8 H x V multiply-adds per active token).  The saved logits
 * are the same fp32 values the chunk statistics are taken from, so logp,
 * lse, grad_h and grad_W are bit-identical to rlk_linear_logp_fwd /
 * rlk_linear_logp_bwd.  This materialises a [T, V]-sized fp32 buffer; the
 * default path above never does.
 *   zsave  fp32, row t (original row index) of the logits at zsave + t*ldzs,
 *          split s (of the 32) at column s * S_pad, S_pad = ceil(S/64)*64,
 *          S = ceil(V/32); columns past a split's width and rows of
 *          inactive targets are not written
 *   ldzs   row stride in floats: a multiple of 4, >= rlk_saved_logits_ld(V)
 * The forward's logp, lse and workspace are those of rlk_linear_logp_fwd
 * (lse is required here); the backward takes the workspace of
 * rlk_linear_logp_bwd and zsave must hold the forward's output for the same
 * h, W and y. */
int64_t rlk_saved_logits_ld(int64_t V); /* 32 * S_pad; 0 for invalid V */
rlk_status rlk_linear_logp_fwd_save(const void* h, const void* W, const int32_t* y,
                                    int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                                    float* logp, float* lse, float* zsave, int64_t ldzs,
                                    void* ws, size_t ws_bytes, void* stream);
rlk_status rlk_linear_logp_bwd_saved(const void* h, const void* W, const int32_t* y,
                                     const float* lse, const float* g,
                                     const float* zsave, int64_t ldzs,
                                     int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                                     void* grad_h, float* grad_W,
                                     void* ws, size_t ws_bytes, void* stream);

/* Statistics of one vocabulary range [vocab_start, vocab_start + vocab_len)
 * of a vocabulary of V_global rows, as one tensor-parallel rank would hold it
 * ("Why the Fused Path Wins", third reason; "vLLM RL-Kernel v0.1.0 ...",
 * "Boundary Fixes in the RL-Kernel Strict Path": the rank's real vocabulary
 * rows, which rank owns a target, the reduction inside the rank).
 *   W_shard  bf16 [vocab_len, H]  rows vocab_start .. vocab_start+vocab_len-1
 *   y        int32 [T]            GLOBAL target ids
 *   out      [T]                  per-row statistics (rlk_lse_partial_t)
 * The range must be an aligned block of splits: with S = ceil(V_global/32)
 * and n the smallest power of two with n*S >= vocab_len, vocab_start must be
 * a multiple of n*S and vocab_len == min(vocab_start + n*S, V_global) -
 * vocab_start; otherwise RLK_ERR_UNALIGNED_VOCAB_RANGE. */
rlk_status rlk_lse_partial(const void* h, const void* W_shard, const int32_t* y,
                           int64_t T, int64_t H,
                           int64_t vocab_start, int64_t vocab_len, int64_t V_global,
                           int32_t ignore_index, rlk_lse_partial_t* out,
                           void* ws, size_t ws_bytes, void* stream);

/* Merge of per-range statistics into the selected log-probability ("Why the
 * Fused Path Wins", third reason: cross-rank log-sum-exp merge).
 *   parts  [n_parts][T] range statistics in ascending vocabulary order
 *   logp   fp32 [T] out; lse fp32 [T] out (may be NULL)
 * Parts are merged with the balanced binary tree (left subtree = the largest
 * power of two smaller than the count).  When the parts are the n_parts
 * equal aligned blocks of a power-of-two n_parts <= 32, the result equals
 * rlk_linear_logp_fwd bit for bit.  1 <= n_parts <= 32. */
rlk_status rlk_lse_merge(const rlk_lse_partial_t* parts, int32_t n_parts,
                         const int32_t* y, int64_t T, int32_t ignore_index,
                         float* logp, float* lse, void* stream);

/* Per-token RL objective on the selected log-probability, and its
 * derivative as the upstream gradient of rlk_linear_logp_bwd.  The pages
 * say the selected logp exists for the importance ratio, clipping and KL
 * terms of PPO / GRPO ("vLLM RL-Kernel v0.1.0 ...", opening section;
 * "Announcing RL-Kernel for vime", section "Vision"), and name the k3 KL
 * estimator; they print no formulas, so the standard ones are used:
 *     r = e(logp - logp_old),  c = min(max(r, 1 - eps_low), 1 + eps_high)
 *     loss = scale * ( -min(r*adv, c*adv) + beta * ((e(d) - d) - 1) ),  d = logp_ref - logp
 *     g    = scale * ( (r*adv <= c*adv ? -r*adv : 0) + beta * (1 - e(d)) )
 * fp32, each operation rounded once in the order written, e() the
 * library's exp (the clip written so that a NaN r stays NaN).  Rows with
 * y == ignore_index get loss = g = 0; a NaN logp (a target outside the
 * vocabulary) gives NaN loss and g.
 *   logp, logp_old, adv   fp32 [T]   (logp from rlk_linear_logp_fwd)
 *   logp_ref              fp32 [T]   reference policy; may be NULL if beta == 0
 *   loss, g               fp32 [T] out; either may be NULL
 * Requires 0 <= eps_low < 1, eps_high >= 0, beta >= 0.  Pointers need only
 * the natural 4-byte alignment. */
rlk_status rlk_rl_token_loss(const float* logp, const float* logp_old, const float* adv,
                             const float* logp_ref, const int32_t* y, int64_t T,
                             int32_t ignore_index, float eps_low, float eps_high, float beta,
                             float scale, float* loss, float* g, void* stream);

/* The forward with the per-token RL objective fused into its last kernel
 * (the pages' Roadmap lists RL loss fragments among the operator's next
 * pieces; "Announcing RL-Kernel for vime", section "Roadmap"): logp and
 * lse exactly as rlk_linear_logp_fwd, and loss and g exactly as
 * rlk_rl_token_loss would compute them from that logp (the same function
 * on the same fp32 value, so the same bits), without the extra launch and
 * without reading logp back.  The objective's arguments and their checks
 * are those of rlk_rl_token_loss; rows with y == ignore_index get
 * logp = lse = loss = g = 0.  loss or g may be NULL, not both. */
rlk_status rlk_linear_logp_fwd_rl(const void* h, const void* W, const int32_t* y,
                                  int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                                  const float* logp_old, const float* adv, const float* logp_ref,
                                  float eps_low, float eps_high, float beta, float scale,
                                  float* logp, float* lse, float* loss, float* g,
                                  void* ws, size_t ws_bytes, void* stream);

/* The forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results
 * (bit for bit) as rlk_linear_logp_fwd, but the workspace is a fixed
 * device array inside the library: RLK_NOALLOC_SCRATCH_BYTES per GPU,
 * allocated when the library's code is loaded on that GPU and held until
 * the process ends.  Calls whose workspace (rlk_workspace_bytes(RLK_OP_FWD,
 * T, H, V)) exceeds it return RLK_ERR_WORKSPACE_TOO_SMALL and enqueue
 * nothing -- e.g. up to about 3700 rows at H = 4096, V = 151936.  Every call
 * on one GPU uses the same scratch: calls that may run at the same time on
 * one GPU (different streams, different host threads) race and must be
 * ordered by the caller.  The scratch keeps the last call's contents;
 * nothing in it needs to start at zero.  Allocates nothing, on the host
 * side either. */
#define RLK_NOALLOC_SCRATCH_BYTES (64u << 20)
rlk_status rlk_linear_logp_fwd_noalloc(const void* h, const void* W, const int32_t* y,
                                       int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                                       float* logp, float* lse, void* stream);

/* Output element types of rlk_gemm_bf16_nt. */
enum { RLK_DT_F32 = 0, RLK_DT_BF16 = 1 };

/* Deterministic, batch-invariant dense product ("vLLM RL-Kernel v0.1.0:
 * Bitwise Train-Rollout Consistency on ROCm", section "Implementation on
 * ROCm": deterministic MFMA-based GEMM kernels; section "Boundary Fixes in
 * the RL-Kernel Strict Path": for GEMM, the K-dimension reduction,
 * accumulation precision, epilogue and materialization boundary are fixed):
 *     C[i, j] = sum_k A[i, k] * B[j, k]
 *   A  bf16 [M, K]      row-major (K contiguous), e.g. activations x
 *   B  bf16 [N, K]      row-major (K contiguous), e.g. a weight W for x W^T
 *   C  [M, ldc] out     fp32 (c_dtype RLK_DT_F32) or bf16 (RLK_DT_BF16:
 *                       the fp32 result rounded once to nearest even);
 *                       columns N .. ldc-1 are not written
 * Contract: one fp32 v_mfma_f32_32x32x16_bf16 accumulation chain per
 * element, k ascending in steps of 16, no split-K -- the chain of the
 * logits above.  Hence C[i, :] depends only on A[i, :] and B (bitwise
 * invariant to M, to the other rows of A and to their order), and repeated
 * runs are bit-identical.
 * Requires 0 < K <= 2^20 with K % 64 == 0, 0 <= M, N <= 2^24, ldc >= N with
 * ldc % 4 == 0; M == 0 or N == 0 returns RLK_OK without launching. */
rlk_status rlk_gemm_bf16_nt(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                            void* C, int64_t ldc, int32_t c_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_H_ */
