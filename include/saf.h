/*
 * libsaf: Selective Attention Freezing (SAF) hybrid causal attention for AMD MI355X
 * (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * Citations refer to the web page "When Can Attention Heads Be Statically Defined?:
 * 中文精读笔记" (reading notes on the SAF paper). Positions are 0-indexed: query i, key j,
 * distance d = i - j; the page's 1-indexed sums over k = 1..i become j = 0..i.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors Q, K, V, O, dO, dQ, dK, dV are [B, H, T, D], contiguous, D fastest (K, V, dK
 *    and dV have kv_heads heads instead of H when key/value heads are shared, see
 *    saf_attn_desc). lse is [B, H, T] float32. alpha and rho are [H, tab_stride] float32 (row h is used
 *    only when head h is frozen; entries 0..T-1 are read).
 *  - Device pointers are HIP device (or managed) memory; `frozen_mask` is HOST memory.
 *    The caller owns every buffer. The library allocates no device memory and keeps no
 *    mutable global state apart from a thread-local error string and an optional
 *    per-thread timing log (saf_prof_*).
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream)
 *    and never synchronises. Argument errors return before anything is enqueued.
 *    A failed launch returns SAF_EHIP; faults during execution surface at the
 *    caller's next synchronisation.
 *  - Device pointers must be 16-byte aligned. D must be 64 or 128 for the attention and
 *    calibration entry points.
 *  - Status codes: SAF_EINVAL (bad pointer, size or alignment), SAF_EUNSUPPORTED
 *    (D or a dtype combination the kernels do not implement), SAF_EWORKSPACE
 *    (workspace smaller than the matching *_workspace_size), SAF_EHIP (launch error).
 *    saf_last_error() returns a thread-local description of the last non-OK status.
 */
#ifndef SAF_H
#define SAF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAF_OK = 0,
  SAF_EINVAL = 1,
  SAF_EUNSUPPORTED = 2,
  SAF_EWORKSPACE = 3,
  SAF_EHIP = 4
} saf_status;

typedef enum { SAF_FP32 = 0, SAF_BF16 = 1 } saf_dtype;

/* One hybrid attention layer.
 *  B, H, T, D   batch, heads, sequence length (>= 1), head width (64 or 128).
 *  io_dtype     storage type of Q, K, V, O and dO (SAF_BF16 or SAF_FP32).
 *  grad_dtype   storage type of dQ, dK, dV. Only SAF_FP32 is implemented: the frozen-head
 *               sink column of dV needs it to stay within a 2e-2 absolute error.
 *  scale        multiplier of Q K^T for ordinary heads (1/sqrt(D) in part 一 of the page);
 *               frozen-head logits alpha + rho are not scaled (Eq. (3)).
 *  frozen_mask  HOST array [H]; nonzero marks a frozen (static-pattern) head (the selected
 *               head set of part 二.1 / Algorithm 1).
 *  tab_stride   row stride, in elements, of alpha and rho (>= T).
 *  kv_heads     number of key/value heads H_kv: 0 or H for ordinary multi-head attention,
 *               or a divisor of H for grouped-query attention (the GQA path of part 二.4,
 *               section 3.3 / Appendix D.2): query head h reads K and V of head h / (H/H_kv),
 *               so a frozen head drops only its query and still mixes its group's V.
 *               K, V, dK and dV are then [B, H_kv, T, D]; Q, O, dO, dQ stay [B, H, T, D]. */
typedef struct {
  int32_t B, H, T, D;
  saf_dtype io_dtype;
  saf_dtype grad_dtype;
  float scale;
  const uint8_t* frozen_mask;
  int32_t tab_stride;
  int32_t kv_heads;
} saf_attn_desc;

/* Hybrid forward (part 一; part 二.3 Eq. (3); part 二.4 and Fig. 2).
 * Ordinary head h:  O[b,h] = softmax_causal(scale * Q K^T) V,
 *                   lse[b,h,i] = log sum_{j<=i} exp(scale * q_i . k_j).
 * Frozen head h:    P(i,j) = exp(alpha[h,j] + rho[h,i-j]) / Z(i) for j <= i, 0 for j > i,
 *                   Z(i) = sum_{j<=i} exp(alpha[h,j] + rho[h,i-j]);
 *                   O[b,h] = P V[b,h] with the current V; lse[b,h,i] = log Z(i) for every b.
 * Q and K slices of frozen heads are never read (Q and K may be NULL when every head is
 * frozen); alpha and rho may be NULL when no head is frozen. alpha/rho entries must be
 * finite or -inf, and every row i must keep at least one finite logit alpha(j)+rho(i-j).
 * O and lse are written for every head. The forward needs no workspace. */
saf_status saf_attn_fwd(const saf_attn_desc* desc, const void* q, const void* k,
                        const void* v, const float* alpha, const float* rho, void* o,
                        float* lse, void* stream);

/* Workspace bytes saf_attn_bwd needs for `desc` (0 on a NULL or invalid descriptor). */
size_t saf_attn_workspace_size(const saf_attn_desc* desc);

/* Hybrid backward for the upstream gradient dO = dL/dO.
 * Ordinary heads: dV = A^T dO, dS = A o (dO V^T - rowsum(dO o O)), dQ = scale dS K,
 *                 dK = scale dS^T Q, with A recomputed from Q, K and the forward's lse.
 * Frozen heads:   dV = P^T dO only (part 二.4: alpha, rho are fixed buffers without
 *                 gradient and there is no query or key); lse must hold log Z(i).
 * o and lse are the forward's outputs for the same inputs. dQ/dK slices of frozen heads
 * are never written; dV is written for every head. Gradients are float32. With bf16 inputs
 * the frozen heads' P^T dO is formed with P rounded to fp16 (11 significant bits) and dO
 * scaled per (b, frozen head) by a power of two into fp16's range, which keeps every dO value
 * within 2^28 of its slice's largest exact (the workspace holds that copy); the result is
 * scaled back when stored.
 * With shared key/value heads (kv_heads < H) the gradient of a shared K or V is the sum over
 * the query heads of its group: dK[b, g] sums the group's ordinary heads (and is not written
 * when every head of the group is frozen); dV[b, g] sums all of them.
 * workspace: device memory of at least saf_attn_workspace_size(desc) bytes, caller-owned,
 * contents need not be initialised and are garbage afterwards. */
saf_status saf_attn_bwd(const saf_attn_desc* desc, const void* q, const void* k,
                        const void* v, const void* o, const void* dO, const float* lse,
                        const float* alpha, const float* rho, void* dq, void* dk,
                        void* dv, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the device array that saf_attn_bwd_noalloc takes its workspace from. */
#define SAF_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* saf_attn_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace comes from a device array of SAF_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends. Arguments, results, layouts and errors are
 * those of saf_attn_bwd, whose kernels it runs; it calls no allocation routine. A layer whose
 * saf_attn_workspace_size exceeds SAF_NOALLOC_SCRATCH_BYTES is rejected with SAF_EWORKSPACE
 * before anything is enqueued: the bf16 workspace is 8 B H T bytes plus 2 B T D bytes per
 * frozen head (plus 8 B H T D bytes with shared key/value heads), so a layer of B = 2, H = 16,
 * T = 8192, D = 128 fits with up to 15 of its 16 heads frozen.
 * The first call on a device looks up the array's address there (SAF_EHIP if that fails).
 * All calls on one GPU share the array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be ordered by the caller. */
saf_status saf_attn_bwd_noalloc(const saf_attn_desc* desc, const void* q, const void* k,
                                const void* v, const void* o, const void* dO, const float* lse,
                                const float* alpha, const float* rho, void* dq, void* dk, void* dv,
                                void* stream);

/* Calibration batch of one layer: N sequences (N >= 2), H heads, length T, width D. */
typedef struct {
  int32_t N, H, T, D;
  saf_dtype io_dtype;
  float scale;
} saf_var_desc;

/* Workspace bytes saf_var_score needs for `desc` (0 on a NULL or invalid descriptor). */
size_t saf_var_workspace_size(const saf_var_desc* desc);

/* Variance score of part 二.1, Eq. (1), for every head of one layer.
 * q, k:   [N, H, T, D] (io_dtype), the ordinary-attention queries and keys of the N
 *         calibration sequences.
 * a_hat:  [H, T, T] float32 output, the mean causal attention (1/N) sum_n A^(n); entries
 *         with j > i are written as 0.
 * s_var:  [H] float64 output, sum_n ||A^(n) - A_hat||_F^2 / ((N - 1) T^2).
 * rank:   [H] int32 output, head indices by ascending s_var; equal scores keep the lower
 *         head index first.
 * workspace as for saf_attn_bwd. */
saf_status saf_var_score(const saf_var_desc* desc, const void* q, const void* k,
                         float* a_hat, double* s_var, int32_t* rank, void* workspace,
                         size_t ws_bytes, void* stream);

/* The forward-KL selector s^KL that part 二.1 compares with Eq. (1) (the page prints no
 * formula; read as the mean over sequences n and rows i of KL(A^(n)_i || A_hat_i)):
 *   s_kl[h] = (1/(N T)) sum_n sum_i sum_{j<=i} A^(n)(i,j) log(A^(n)(i,j) / A_hat(i,j)),
 * computed in the same pass as a_hat (sum_n A^(n) = N A_hat turns it into
 * sum_n A log A - N A_hat log A_hat per entry). Arguments, workspace and a_hat as for
 * saf_var_score; rank orders the heads by ascending s_kl. */
saf_status saf_kl_score(const saf_var_desc* desc, const void* q, const void* k, float* a_hat,
                        double* s_kl, int32_t* rank, void* workspace, size_t ws_bytes,
                        void* stream);

/* The "sharp mean" candidate pattern of part 二.2 (the notes compare it with the
 * probability mean a_hat): logits averaged over the N sequences, then the causal softmax,
 *   p_sharp[h] = softmax_causal((1/N) sum_n scale Q_n K_n^T),
 * written as [H, T, T] float32 with zeros above the diagonal. Arguments as for
 * saf_var_score; no workspace. */
saf_status saf_sharp_mean(const saf_var_desc* desc, const void* q, const void* k,
                          float* p_sharp, void* stream);

/* Host-only selection across layers (part 二.1): sorts n_heads scores (all L*H heads of a
 * model) ascending, ties to the lower index, and writes the first k = floor(r*n + 1/2)
 * indices to out[0..k-1] (out holds n_heads entries). Returns k, or -1 on bad arguments. */
int32_t saf_select_heads(const double* s_var_all, int32_t n_heads, double r, int32_t* out);

/* ---- Compact static pattern fit (part 二.3, Eq. (3), Eq. (4), Appendix A.2) ----
 * A candidate head's target pattern A [T, T] (its mean attention, e.g. a_hat of
 * saf_var_score: causal, rows summing to 1) is replaced by
 *   P(i,j) = exp(alpha(j) + rho(i-j)) / Z(i) for j <= i,
 * with alpha, rho fitted by minimising the mean over rows of the cross-entropy
 * -sum_j A(i,j) log P(i,j). That objective depends on A only through two marginals
 * (Eq. (4)); the fit runs Adam on them and reports the mean row KL(A_i || P_i), which the
 * page accepts at <= 0.2 nat. alpha, rho, the marginals and log Z are [H, T] float32,
 * contiguous, one row per fitted pattern. */

/* Eq. (4) statistics of H targets a [H, T, T] float32 (entries above the diagonal are not
 * read): col[h, j] = sum_{i>=j} a(i, j), dist[h, d] = sum_{i>=d} a(i, i-d), and
 * ent[h, j] = -sum_{i>=j} a(i,j) log a(i,j) (0 log 0 = 0), whose sum over j divided by T is
 * the mean row entropy. H, T >= 1. No workspace. */
saf_status saf_pattern_stats(int32_t H, int32_t T, const float* a, float* col, float* dist,
                             float* ent, void* stream);

/* The same marginals of the compact pattern itself, and its normaliser:
 * logz[h, i] = log Z(i); col[h, j] = sum_{i>=j} P(i, j); dist[h, d] = sum_{i>=d} P(i, i-d).
 * alpha, rho follow the value rules of saf_attn_fwd (finite, or -inf with a finite logit
 * left in every row). No workspace. */
saf_status saf_compact_marginals(int32_t H, int32_t T, const float* alpha, const float* rho,
                                 float* logz, float* col, float* dist, void* stream);

/* How saf_compact_fit spreads the work (the results agree to float32 rounding):
 * SAF_FIT_PER_STEP launches two kernels per Adam step over all heads, each head spread over
 * many CUs, its state in the workspace; SAF_FIT_PER_HEAD runs the whole fit in one launch,
 * one workgroup per head with the head's state in LDS (T <= 2048; the workspace is not
 * used); SAF_FIT_AUTO takes SAF_FIT_PER_HEAD when T <= 2048 and there are 16 heads or more
 * or T <= 256, SAF_FIT_PER_STEP otherwise. */
typedef enum { SAF_FIT_AUTO = 0, SAF_FIT_PER_STEP = 1, SAF_FIT_PER_HEAD = 2 } saf_fit_schedule;

/* One fit of H patterns of length T: `steps` Adam steps (the page uses 400) with learning
 * rate lr, moment decays beta1 and beta2 and denominator offset eps (a reading, since the
 * page names only the optimiser: 0.1, 0.9, 0.999, 1e-8). lr > 0, 0 <= beta < 1, eps >= 0,
 * steps >= 0, H in [1, 65535], T >= 1, H * T <= 2^31; schedule a saf_fit_schedule value
 * (SAF_EINVAL otherwise; SAF_EUNSUPPORTED for SAF_FIT_PER_HEAD with T > 2048). */
typedef struct {
  int32_t H, T;
  int32_t steps;
  float lr, beta1, beta2, eps;
  int32_t schedule;
} saf_fit_desc;

/* Workspace bytes saf_compact_fit needs (0 on a NULL or invalid descriptor). */
size_t saf_fit_workspace_size(const saf_fit_desc* desc);

/* Fits alpha, rho [H, T] (in: the starting point, e.g. zeros, the uniform causal pattern;
 * out: the fitted tables) to the targets whose saf_pattern_stats are col, dist, ent, by
 * bias-corrected Adam on the mean row cross-entropy, whose gradient is
 * (colP - col) / T for alpha and (distP - dist) / T for rho. Writes kl[h], the mean row
 * KL of the fitted pattern (float32, [H]). workspace as for saf_attn_bwd. */
saf_status saf_compact_fit(const saf_fit_desc* desc, const float* col, const float* dist,
                           const float* ent, float* alpha, float* rho, float* kl,
                           void* workspace, size_t ws_bytes, void* stream);

/* Host-only selection with the fit's acceptance test (part 二.1 and Appendix A.2): walks the
 * n_heads heads (all L*H of a model) by ascending s_var, ties to the lower index, keeps a
 * head when kl_all[head] <= max_kl and skips it otherwise, and stops once
 * k = floor(r*n + 1/2) heads are kept. Writes the kept indices, in walk order, to out
 * (n_heads entries) and returns their number (less than k when too few fits pass), or -1 on
 * bad arguments. */
int32_t saf_select_fitted(const double* s_var_all, const float* kl_all, int32_t n_heads,
                          double r, float max_kl, int32_t* out);

const char* saf_status_string(saf_status status);
const char* saf_last_error(void);

/* Optional timing of the library's own kernel launches, for profiling. While enabled on
 * the calling thread, each kernel the entry points launch is bracketed by a pair of
 * hipEvents recorded on the launch stream. saf_prof_read synchronises on those events and
 * copies up to `cap` records (kernel name, milliseconds) in launch order, returning the
 * number of records; saf_prof_enable(0) drops the log. The events are created once per
 * thread and reused. */
saf_status saf_prof_enable(int enable);
int32_t saf_prof_read(const char** names, float* ms, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* SAF_H */
