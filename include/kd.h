/*
 * kd.h - C ABI of the fused chunked-KL distillation library (libkd.so).
 *
 * Full-vocabulary logit distillation computed straight from hidden states:
 * the library rebuilds the student and teacher logits z = h W^T one
 * vocabulary tile at a time on the GPU (bf16 MFMA, fp32 accumulation) and
 * reduces them with online log-sum-exp and divergence accumulators, so no
 * [tokens, V] logit tensor is ever written to memory.
 *   Source: ricardokevins notes, "Nitrobrew tweet analysis", section
 *   "Nitrobrew 的两个动作" (rebuild logits per vocabulary block, update online
 *   softmax / log-sum-exp accumulators and KL terms, discard the block) and
 *   the forward_kl / reverse_kl listing under "VeRL PR" (inputs: student and
 *   teacher hidden states, both unembeddings, temperature, chunk size).
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) are device pointers on the current HIP device,
 *     owned by the caller; the library allocates no device memory. Scratch
 *     memory is the caller's `workspace`, sized by kd_workspace_size().
 *   - Layout: row-major and contiguous. h_s [N, d_s], h_t [N, d_t] hold one
 *     token per row ([B, T, D] flattened); W_s [V, d_s], W_t [V, d_t] hold one
 *     vocabulary entry per row (the nn.Linear weight layout). Inputs must be
 *     16-byte aligned and d_s, d_t multiples of 8 with 256 * d * element size
 *     below 2^31 (else KD_ERR_UNSUPPORTED).
 *     V is arbitrary (vocabulary tails are masked, never read as logit 0).
 *   - dtype: KD_BF16 (uint16 bf16 bit patterns) or KD_F32, for all four of
 *     h_s, W_s, h_t, W_t alike.
 *   - Temperature: s = z_s / tau, t = z_t / tau before any softmax; q = softmax(s)
 *     is the student, p = softmax(t) the teacher. No tau^2 factor is applied.
 *     (ars-opd-rebuild "03 · 层 2：White-box OPD 基线", section 2.3.)
 *   - Outputs are per token ("reduction none"); mean/sum over valid tokens is
 *     the caller's (the same section: a per-token mean over non-ignored labels).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous; nothing blocks the host. Argument checks run on the host
 *     before any HIP call and return KD_ERR_INVALID_ARG / KD_ERR_UNSUPPORTED /
 *     KD_ERR_WORKSPACE without touching the GPU; a failed launch returns
 *     KD_ERR_HIP. Calls on different streams with different workspaces may run
 *     concurrently; calls sharing a workspace must be ordered by the caller.
 *   - Results do not depend on chunk_V beyond fp32 rounding.
 */
#ifndef KD_H_
#define KD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KD_OK = 0,
  KD_ERR_INVALID_ARG = 1, /* null required pointer, N <= 0, V < 2, beta outside [0,1], tau <= 0, ... */
  KD_ERR_UNSUPPORTED = 2, /* d not a multiple of 8, misaligned pointer, unknown dtype */
  KD_ERR_WORKSPACE = 3,   /* ws_bytes smaller than kd_workspace_size() */
  KD_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} kd_status;

typedef enum { KD_F32 = 0, KD_BF16 = 1 } kd_dtype;

typedef enum {
  KD_OP_FWD = 0,
  KD_OP_BWD = 1,
  KD_OP_TOPK = 2,
  KD_OP_BWD_W = 3,
  KD_OP_TOPK_BWD = 4,
  KD_OP_TAIL = 5,
  KD_OP_TAIL_BWD = 6
} kd_op;

/* Support bits of the tail-bucket divergence (kd_tail_fwd / kd_tail_bwd). */
#define KD_SUPPORT_TEACHER 1 /* the teacher's top-k */
#define KD_SUPPORT_STUDENT 2 /* the student's top-k */
#define KD_SUPPORT_LABEL 4   /* the label token */

/* Largest k accepted by kd_topk_fwd. */
#define KD_TOPK_MAX 64
/* Largest vocabulary accepted by kd_topk_fwd and kd_tail_fwd (8 splits of
 * 65536 entries). */
#define KD_TOPK_MAX_V 524288

/*
 * kd_workspace_size - device workspace (bytes) that `op` needs for this shape.
 *   Source: ricardokevins notes, "Nitrobrew tweet analysis", the evaluation
 *   table's working-set row (peak memory falls from the full [tokens, V]
 *   logits to one vocabulary chunk, O(tokens * chunk_V)), and the chunk size
 *   argument of the forward_kl / reverse_kl listing under "VeRL PR".
 *   op: KD_OP_FWD (kd_fwd), KD_OP_BWD (kd_bwd without dW_s), KD_OP_BWD_W
 *   (kd_bwd with dW_s), KD_OP_TOPK (kd_topk_fwd), KD_OP_TOPK_BWD
 *   (kd_topk_bwd: KD_OP_BWD's chunk buffers plus O(N k) floats), KD_OP_TAIL
 *   (kd_tail_fwd, any support) or KD_OP_TAIL_BWD (kd_tail_bwd, any support:
 *   KD_OP_BWD's buffers plus O(N k) floats).
 *   beta is read for KD_OP_FWD, chunk_V for the backward ops (0 selects
 *   kd_default_chunk, as in the backward calls), k for the top-k and tail
 *   ops; d_s/d_t/dtype size the backward's per-chunk buffers.
 *   The backward's workspace is O(N * chunk_V) (the gradient tile G of one
 *   vocabulary chunk, in the input dtype) plus O(chunk_V * d_s) for one
 *   transposed chunk of W_s; KD_OP_BWD_W adds a transposed copy of G and of
 *   h_s (O(N * chunk_V + N * d_s)); kd_bwd's also holds O(N * chunk_V / 256)
 *   floats for its dominant-entry correction. The forward's is at most 256
 *   partial records of 5 floats per token (7 for 0 < beta < 1), whatever V:
 *   O(N). Writes the size to *bytes (host pointer). Pure host function.
 */
kd_status kd_workspace_size(kd_op op, int64_t N, int64_t V, int32_t d_s, int32_t d_t, kd_dtype dtype,
                            float beta, int32_t chunk_V, int32_t k, size_t* bytes);

/*
 * kd_default_chunk - the recompute chunk that the backward calls use when
 *   passed chunk_V = 0. The recompute structure (one vocabulary chunk of the
 *   gradient at a time) is the Nitrobrew notes' "仓库实现"; the chunk size is
 *   the caller's memory/speed trade-off. The default keeps the [N, chunk]
 *   gradient tile within 1 GiB (input dtype) and splits the vocabulary, V
 *   rounded up to 256, into the fewest equal chunks (multiples of 256) under
 *   that bound, never below 2048 entries unless the vocabulary is smaller.
 *   Few tokens thus get the whole vocabulary as one chunk; 32768 bf16 tokens
 *   over 151936 entries get ten chunks of 15360.
 *   Returns 0 for N < 0, V < 1 or an unknown dtype. Pure host function.
 */
int32_t kd_default_chunk(int64_t N, int64_t V, kd_dtype dtype);

/*
 * kd_fwd - per-token beta-divergence between student and teacher.
 *   Source: ars-opd-rebuild "03 · 层 2：White-box OPD 基线", section 2.3 (beta
 *   table): beta = 0 gives KL(p || q) (forward, teacher first), beta = 1 gives
 *   KL(q || p) (reverse, student first), 0 < beta < 1 gives
 *   beta KL(p || m) + (1 - beta) KL(q || m) with m = beta p + (1 - beta) q.
 *   Blockwise online reduction per "Nitrobrew 的两个动作" (Nitrobrew notes).
 *
 *   h_s, W_s, h_t, W_t (device, read): inputs as described above.
 *   N tokens, V vocabulary entries, d_s / d_t hidden sizes.
 *   beta in [0, 1]; tau > 0.
 *   loss  (device, [N] fp32, written): the divergence of each token.
 *   lse_s, lse_t (device, [N] fp32, written): natural-log log-sum-exp of the
 *         tempered student / teacher logits (kd_bwd consumes them).
 *   aux   (device, [N] fp32, written; may be NULL when beta == 0): the
 *         gradient's centring scalar: KL(q || m) for 0 < beta < 1, the loss
 *         itself for beta == 1.
 *   workspace (device, >= kd_workspace_size(KD_OP_FWD, ...) bytes): scratch.
 */
kd_status kd_fwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                 int32_t d_s, int32_t d_t, float beta, float tau, kd_dtype dtype, float* loss, float* lse_s,
                 float* lse_t, float* aux, void* workspace, size_t ws_bytes, void* stream);

/*
 * kd_fwd_noalloc - kd_fwd without a workspace argument and without any device
 *   allocation, for callers that cannot allocate: code under HIP graph
 *   capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Same arguments, results and kernels as kd_fwd (bit for bit), minus
 *   workspace / ws_bytes. The forward's partial records go to a fixed
 *   scratch array of kd_fwd_noalloc_max_scratch() bytes (144 MiB) that the
 *   library holds on each GPU it runs on until the process ends; a shape
 *   whose kd_workspace_size(KD_OP_FWD, ...) exceeds it returns
 *   KD_ERR_WORKSPACE (before any HIP call that touches the GPU). The array's
 *   device address is looked up once per device, on the first call with that
 *   device current. Calls on one GPU share the array: calls that overlap on
 *   one GPU (other streams, other host threads) race and must be ordered by
 *   the caller.
 */
kd_status kd_fwd_noalloc(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                         int32_t d_s, int32_t d_t, float beta, float tau, kd_dtype dtype, float* loss, float* lse_s,
                         float* lse_t, float* aux, void* stream);

/* Size in bytes of kd_fwd_noalloc's scratch array. Pure host function. */
size_t kd_fwd_noalloc_max_scratch(void);

/*
 * kd_bwd - gradient of sum_n grad_loss[n] * loss[n] with respect to h_s and,
 *   optionally, W_s.
 *   Source: Nitrobrew notes, "仓库实现": the gradient is recomputed block by
 *   block instead of storing logits; "工程落地：简单 idea，不等于简单集成": the
 *   student hidden state and the student unembedding receive gradients, the
 *   teacher's parameters stay fixed.
 *   With g = dloss/ds (s the tempered student logits):
 *     beta = 0:  g = q - p
 *     beta = 1:  g = q (log q - log p - KL(q || p))
 *     else:      g = (1 - beta) q (log q - log m - KL(q || m))
 *   dh_s[n, :] = grad_loss[n] * sum_v (g[n, v] / tau) W_s[v, :]
 *   dW_s[v, :] = sum_n grad_loss[n] * (g[n, v] / tau) h_s[n, :]
 *   For dh_s, the entry whose student probability exceeds 0.6 (at most one
 *   per token) takes minus the sum of the token's other entries (g sums to
 *   zero over v for every beta): its own formula cancels terms of the size
 *   of the log-sum-exps, which fp32 cannot resolve when q saturates.
 *
 *   lse_s, lse_t, aux (device, [N] fp32, read): as written by kd_fwd with the
 *         same inputs, beta and tau (aux unused when beta == 0, may be NULL).
 *   grad_loss (device, [N] fp32, read; NULL means all ones).
 *   chunk_V: vocabulary entries per recompute chunk (a positive multiple of
 *         256, or 0 for kd_default_chunk(N, V, dtype)); the workspace holds
 *         one [N, chunk_V] gradient chunk.
 *   dh_s  (device, [N, d_s] fp32, overwritten; may be NULL if dW_s is not).
 *   dW_s  (device, [V, d_s] fp32, overwritten; may be NULL). When given, the
 *         workspace must hold kd_workspace_size(KD_OP_BWD_W, ...) bytes and
 *         256 * N (rounded up to 128) * element size must stay below 2^31
 *         (about 4.19M bf16 / 2.09M fp32 tokens; else KD_ERR_UNSUPPORTED).
 *   chunk_V * element size * 256 < 2^31 as well (else KD_ERR_UNSUPPORTED).
 */
kd_status kd_bwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                 int32_t d_s, int32_t d_t, float beta, float tau, kd_dtype dtype, int32_t chunk_V,
                 const float* lse_s, const float* lse_t, const float* aux, const float* grad_loss, float* dh_s,
                 float* dW_s, void* workspace, size_t ws_bytes, void* stream);

/*
 * kd_topk_fwd - top-k three-term decomposition over bf16 logits.
 *   Source: lpnh.cn "Top-K知识蒸馏损失实现详解", section 一.2 (binary KL on the
 *   teacher mass inside vs outside the top-k set; conditional KL on the shape
 *   inside the set after renormalising; CE anchor on the true token) and
 *   sections 二.1 / 二.2 (logits in bf16, fp32 only for the log-sum-exp
 *   accumulators; the top-64 gathered in bf16 and only those upcast).
 *   Both models' logits are rounded to bf16 (nearest, ties to even); the
 *   teacher's top-k is taken by (bf16 logit descending, vocabulary index
 *   ascending); all sums are fp32 over the bf16 values. Only KD_BF16 inputs.
 *   With P = sum_K p, Q = sum_K q (tempered):
 *     binary_kl = P log(P/Q) + (1-P) log((1-P)/(1-Q))
 *     cond_kl   = sum_K (p/P) (log(p/P) - log(q/Q))
 *     ce        = logsumexp(z_s) - z_s[label]   (untempered student, bf16)
 *
 *   k in [1, min(V, KD_TOPK_MAX)]; V <= KD_TOPK_MAX_V (else KD_ERR_UNSUPPORTED).
 *   labels   (device, [N] int32, read; may be NULL): -100 marks an ignored
 *            token (its ce is written as NaN); other values must lie in [0, V).
 *   topk_idx (device, [N, k] int32, written): the selection, in order.
 *   topk_val (device, [N, k] fp32, written; may be NULL): the bf16 teacher
 *            logits (untempered) at topk_idx.
 *   topk_val_s (device, [N, k] fp32, written; may be NULL): the bf16 student
 *            logits (untempered) at topk_idx.
 *   binary_kl, cond_kl, p_mass, q_mass, lse_s, lse_t (device, [N] fp32,
 *            written): lse_* over the tempered bf16 logits.
 *   ce       (device, [N] fp32, written when labels != NULL; may be NULL).
 *   lse_s1   (device, [N] fp32, written; may be NULL): natural-log LSE of the
 *            untempered bf16 student logits (the CE's; kd_topk_bwd reads it).
 */
kd_status kd_topk_fwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                      int32_t d_s, int32_t d_t, int32_t k, float tau, kd_dtype dtype, const int32_t* labels,
                      int32_t* topk_idx, float* topk_val, float* topk_val_s, float* binary_kl, float* cond_kl, float* ce,
                      float* p_mass, float* q_mass, float* lse_s, float* lse_t, float* lse_s1, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * kd_topk_bwd - gradient of sum_n (grad_binary[n] binary_kl[n] + grad_cond[n]
 *   cond_kl[n] + grad_ce[n] ce[n]) with respect to h_s, for the terms of
 *   kd_topk_fwd. Source: lpnh.cn "Top-K知识蒸馏损失实现详解", section 一.2 (the
 *   three terms are the training loss). The pages do not spell the gradient
 *   out; here the selection and the teacher are held fixed and the bf16
 *   rounding of the student logits is passed straight through. With q the
 *   tempered student softmax, r the untempered one, Q / P the student /
 *   teacher mass on the set K and p^ the renormalised teacher on K:
 *     dL/dz_v = [ w_b B q_v (1[v in K] - Q) + w_c 1[v in K] (q_v / Q - p^_v) ] / tau
 *               + w_ce (r_v - 1[v = label]),      B = -P/Q + (1-P)/(1-Q)
 *   (B = 0 when k == V), and dh_s[n] = sum_v dL/dz_v W_s[v].
 *   Only KD_BF16 inputs; d_t and the teacher's arrays are not needed.
 *
 *   h_s, W_s (device, read): the forward's student inputs.
 *   k, tau, labels: as given to kd_topk_fwd (labels may be NULL).
 *   topk_idx, topk_val, topk_val_s, p_mass, q_mass, lse_s (device, read):
 *            kd_topk_fwd's outputs (topk_val / topk_val_s must have been
 *            requested there).
 *   lse_s1   (device, [N] fp32, read): kd_topk_fwd's lse_s1; needed when
 *            grad_ce and labels are given, else may be NULL.
 *   grad_binary, grad_cond, grad_ce (device, [N] fp32, read; each may be NULL
 *            = zero weights).
 *   chunk_V: as for kd_bwd. dh_s (device, [N, d_s] fp32, 16-byte aligned,
 *            overwritten).
 *   workspace (device, >= kd_workspace_size(KD_OP_TOPK_BWD, ...) bytes).
 */
kd_status kd_topk_bwd(const void* h_s, const void* W_s, int64_t N, int64_t V, int32_t d_s, int32_t k, float tau,
                      kd_dtype dtype, const int32_t* labels, const int32_t* topk_idx, const float* topk_val,
                      const float* topk_val_s, const float* p_mass, const float* q_mass, const float* lse_s,
                      const float* lse_s1, const float* grad_binary, const float* grad_cond, const float* grad_ce,
                      int32_t chunk_V, float* dh_s, void* workspace, size_t ws_bytes, void* stream);

/*
 * kd_tail_fwd - beta-divergence over a top-k support plus one tail bucket.
 *   Source: ars-opd-rebuild "03 · 层 2：White-box OPD 基线", section 2.4 (the
 *   divergence is taken on the k kept entries plus a tail bucket that holds
 *   all the probability mass outside them, log(1 - sum of the kept
 *   probabilities); the kept set is the teacher's top-k, the student's top-k
 *   or their union with duplicates removed depending on beta, and with a
 *   single kept entry the sampled token together with the teacher's top-1)
 *   and section 2.3 (the beta family and the temperature).
 *   Logits of both models are rounded to bf16 (nearest, ties to even), as for
 *   kd_topk_fwd. With S the support, p / q the tempered teacher / student
 *   softmax over the whole vocabulary, the buckets are {v} for v in S and
 *   the tail T = V \ S (P_T = 1 - sum_S p, Q_T likewise):
 *     beta = 0:     loss = sum_b p_b log(p_b / q_b)
 *     beta = 1:     loss = sum_b q_b log(q_b / p_b)
 *     0 < beta < 1: loss = beta sum_b p_b log(p_b / m_b)
 *                          + (1 - beta) sum_b q_b log(q_b / m_b),
 *                   m_b = beta p_b + (1 - beta) q_b,
 *   with no tail bucket when S covers the vocabulary. A tail mass below fp32
 *   resolution is held at 2^-24. Only KD_BF16 inputs.
 *
 *   support  KD_SUPPORT_* bits; the teacher's or the student's bit (or both)
 *            must be set. The support lists, in order, the teacher's top-k
 *            (bf16 logit descending, index ascending), the student's top-k
 *            entries not already listed, and the label when KD_SUPPORT_LABEL
 *            is set, the label is in [0, V) and not already listed. The
 *            usual choices: k == 1: TEACHER | LABEL; else beta == 0: TEACHER,
 *            beta == 1: STUDENT, 0 < beta < 1: TEACHER | STUDENT.
 *   k in [1, min(V, KD_TOPK_MAX)]; V <= KD_TOPK_MAX_V (else KD_ERR_UNSUPPORTED).
 *   labels   (device, [N] int32, read): required with KD_SUPPORT_LABEL,
 *            else ignored (may be NULL); -100 (or any value outside [0, V))
 *            adds no entry.
 *   sup_idx  (device, [N, smax] int32, written), smax = k per ranked model
 *            + 1 with KD_SUPPORT_LABEL: the support, -1 in unused slots.
 *   sup_t, sup_s (device, [N, smax] fp32, written): the bf16 teacher /
 *            student logits (untempered) at sup_idx; NaN in unused slots.
 *   loss, lse_s, lse_t (device, [N] fp32, written); lse_* over the tempered
 *            bf16 logits. p_mass, q_mass (device, [N] fp32, written; may be
 *            NULL): sum_S p and sum_S q.
 *   workspace (device, >= kd_workspace_size(KD_OP_TAIL, ...) bytes). One
 *            sweep over the vocabulary ranks one model or both.
 */
kd_status kd_tail_fwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                      int32_t d_s, int32_t d_t, int32_t k, int32_t support, float beta, float tau, kd_dtype dtype,
                      const int32_t* labels, int32_t* sup_idx, float* sup_t, float* sup_s, float* loss, float* p_mass,
                      float* q_mass, float* lse_s, float* lse_t, void* workspace, size_t ws_bytes, void* stream);

/*
 * kd_tail_bwd - gradient of sum_n grad_loss[n] loss[n] of kd_tail_fwd with
 *   respect to h_s. Source: as kd_tail_fwd (the pages do not spell the
 *   gradient out). The support and the teacher are held fixed and the bf16
 *   rounding of the student logits is passed straight through. With b(v) the
 *   bucket of v and a_b = dloss/dq_b (beta = 0: -p_b / q_b; beta = 1:
 *   log(q_b / p_b) + 1; else (1 - beta) log(q_b / m_b)):
 *     dloss/dz_v = q_v (a_b(v) - sum_b q_b a_b) / tau,
 *   and dh_s[n] = grad_loss[n] sum_v dloss/dz_v W_s[v]. Only KD_BF16 inputs;
 *   the teacher's arrays are not needed.
 *
 *   h_s, W_s (device, read): the forward's student inputs.
 *   k, support, beta, tau: as given to kd_tail_fwd (k and support fix smax).
 *   sup_idx, sup_t, sup_s, lse_s, lse_t (device, read): kd_tail_fwd's outputs.
 *   grad_loss (device, [N] fp32, read; may be NULL = all ones).
 *   chunk_V: as for kd_bwd. dh_s (device, [N, d_s] fp32, 16-byte aligned,
 *            overwritten).
 *   workspace (device, >= kd_workspace_size(KD_OP_TAIL_BWD, ...) bytes).
 */
kd_status kd_tail_bwd(const void* h_s, const void* W_s, int64_t N, int64_t V, int32_t d_s, int32_t k, int32_t support,
                      float beta, float tau, kd_dtype dtype, const int32_t* sup_idx, const float* sup_t,
                      const float* sup_s, const float* lse_s, const float* lse_t, const float* grad_loss,
                      int32_t chunk_V, float* dh_s, void* workspace, size_t ws_bytes, void* stream);

/*
 * kd_gather_rows / kd_scatter_rows - row gather and scatter for token masking.
 *   Source: lpnh.cn "Top-K知识蒸馏损失实现详解", section 二.4 (gather the hidden
 *   states at the positions that carry a loss before the unembedding, so the
 *   masked positions cost nothing). Gather the hidden states of the tokens
 *   whose label is not ignored, call kd_fwd / kd_bwd on the gathered rows,
 *   and scatter dL/dh_s back; the work is proportional to the kept tokens.
 *   kd_gather_rows:  dst[i, :] = src[rows[i], :] for i < n_rows; an index
 *                    outside [0, n_src) gives a row of zeros.
 *   kd_scatter_rows: dst[rows[i], :] = src[i, :] for i < n_rows; indices outside
 *                    [0, n_dst) are skipped; other rows of dst are untouched;
 *                    duplicate indices leave one of their rows (unspecified).
 *   src, dst, rows (device): row-major arrays of row_bytes bytes per row
 *   (a positive multiple of 4), 4-byte aligned (16-byte alignment and rows of
 *   16-byte multiples take the wide path); rows is int32 [n_rows]. n_rows = 0
 *   is a no-op.
 */
kd_status kd_gather_rows(const void* src, int64_t n_src, int64_t row_bytes, const int32_t* rows, int64_t n_rows,
                         void* dst, void* stream);
kd_status kd_scatter_rows(const void* src, int64_t n_rows, int64_t row_bytes, const int32_t* rows, void* dst,
                          int64_t n_dst, void* stream);

/* kd_status_string - a static, human-readable name for a status code. */
const char* kd_status_string(kd_status s);

/* kd_last_error - a static description of the most recent failure on the
 * calling thread (argument name or HIP error string); "" if none. */
const char* kd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KD_H_ */
