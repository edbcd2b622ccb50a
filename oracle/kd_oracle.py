"""fp64 CPU oracle for full-vocabulary logit distillation from hidden states.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this directory. The product package never does, and this module imports
nothing from it: the two share no code.

What is computed follows the plain definitions, written out on materialised
full logit rows (the GPU path reaches the same numbers by streaming vocabulary
blocks; chunking and an online log-sum-exp are exact re-associations of these
sums). Sources, cited by page title and section:

* [Nitrobrew notes]  ricardokevins notes, "Nitrobrew tweet analysis":
  section "Nitrobrew 的两个动作" (logits z = h W^T rebuilt per vocabulary block,
  online softmax / log-sum-exp and KL accumulators), "仓库实现" (forward-KL
  gradient "p - q", reverse-KL gradient "p (log p - log q - KL)", with p the
  student there), the ``forward_kl`` / ``reverse_kl`` listing under "VeRL PR"
  (student/teacher hidden states, both unembeddings, temperature; gradients
  reach the student only), and "工程落地：简单 idea，不等于简单集成" (the student
  hidden state and the student unembedding receive gradients, the teacher's
  parameters are frozen).
* [White-box OPD]  ars-opd-rebuild "03 · 层 2：White-box OPD 基线": section 2.3
  (the beta table: beta=0 KL(teacher||student), beta=1 KL(student||teacher),
  0<beta<1 beta*KL(teacher||m) + (1-beta)*KL(student||m) with
  m = (1-beta)*student + beta*teacher; temperature divides logits before the
  softmax; log-domain arithmetic, logsumexp for the mixture; per-token mean),
  section 2.4 (tail bucket log(1 - sum of top-k probabilities); the support
  is the teacher's top-k, the student's or their union depending on beta, and
  with one kept entry the sampled token plus the teacher's top-1), section 6
  (CPU test plan).
* [Top-K KD]  lpnh.cn "Top-K知识蒸馏损失实现详解": section 一.2 (binary KL on the
  mass inside/outside the top-k set, conditional KL on the renormalised shape
  inside it, CE anchor on the true token), section 二.1 (bf16 logits, fp32 only
  for log-sum-exp accumulators), section 二.2 (gather the top-64 in bf16, then
  upcast only those values).

Readings where the pages leave a step open are marked READING in the
docstrings; every function carries its pins in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "as_f64", "bf16_round", "bf16_neighbours", "logits", "lse", "log_softmax", "divergence",
    "kd_fwd", "grad_student_logits", "kd_bwd", "kd_fwd_bwd", "kd_bwd_w", "topk_order", "topk_three_terms", "kd_topk_fwd",
    "fp32_dot_error_bound", "svd_teacher", "log1mexp", "topk_grad_student_logits", "kd_topk_bwd",
    "SUPPORT_TEACHER", "SUPPORT_STUDENT", "SUPPORT_LABEL", "tail_default_support", "tail_support_size",
    "tail_support", "tail_divergence", "kd_tail_fwd", "tail_grad_student_logits", "kd_tail_bwd",
]

_SLAB = 8192  # vocabulary rows converted to fp64 at a time (memory only)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def as_f64(x) -> np.ndarray:
    """Decode an input array to float64 exactly.

    uint16 arrays are bf16 bit patterns (sign, 8 exponent bits, 7 mantissa
    bits: the upper half of an IEEE float32); float32/float64 are widened."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_EXP = -133  # exponent of the smallest bf16 subnormal


def _bf16_quantum_exp(x: np.ndarray) -> np.ndarray:
    # bf16 keeps 8 significant bits: a value in [2^(e-1), 2^e) is a multiple of 2^(e-8).
    _, e = np.frexp(x)
    return np.maximum(e - 8, _BF16_MIN_EXP)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), directly
    from float64 (no intermediate float32 rounding, which could round twice).
    Returns the rounded values as float64. [Top-K KD, 二.1: logits are kept in
    bf16.]"""
    x = np.asarray(x, dtype=np.float64)
    qe = _bf16_quantum_exp(x)
    r = np.ldexp(np.rint(np.ldexp(x, -qe)), qe)  # scaling by 2^k is exact; rint ties to even
    # values that round past the largest finite bf16 become infinities
    limit = _BF16_MAX + 2.0 ** 119  # midpoint between max finite and the next (overflowing) step
    r = np.where(np.abs(x) >= limit, np.copysign(np.inf, x), r)
    return r


def bf16_neighbours(x):
    """For each float64 value: the two bf16 values around it and the midpoint
    between them. Returns (lo, hi, mid) with lo <= x <= hi."""
    x = np.asarray(x, dtype=np.float64)
    qe = _bf16_quantum_exp(x)
    y = np.ldexp(x, -qe)
    lo = np.ldexp(np.floor(y), qe)
    hi = np.ldexp(np.ceil(y), qe)
    hi = np.where(hi == lo, np.ldexp(np.floor(y) + 1.0, qe), hi)
    return lo, hi, 0.5 * (lo + hi)


def fp32_dot_error_bound(h, W, factor: float = 8.0):
    """A statistical bound on |fp32-accumulated dot - exact dot| for every logit
    ([rows, V] float64):

        factor * 2^-24 * sqrt(d) * (|z| + sqrt(sum_i (h_i W_i)^2)).

    READING ([Top-K KD], 二.1-二.2: logits are produced in bf16 from an fp32
    accumulation; the pages fix neither the summation order nor its rounding):
    the products of bf16 inputs are exact in fp32, so the error is the sum of
    the roundings of at most d additions, each at most 2^-24 times the partial
    sum it forms. For terms in an order unrelated to their values, partial sums
    stay within a multiple of |z| (the drift) plus sqrt(sum x_i^2) (the spread
    of a random walk), and the roundings add like independent draws, hence the
    sqrt(d). A logit lying within this distance of a bf16 rounding midpoint may
    round either way on the GPU; only such logits may make a top-k selection
    differ from this oracle's. Pinned against float32 accumulation in the
    orders a kernel takes (sequential, pairwise, per-lane blocks then a tree,
    blocks of 16 exact products with rounded and truncated accumulation), and
    against being vacuous (the share of logits it flags)."""
    h64 = as_f64(h)
    d = h64.shape[1]
    h2 = h64 * h64
    out = np.empty((h64.shape[0], W.shape[0]))
    for v0 in range(0, W.shape[0], _SLAB):
        w = as_f64(W[v0:v0 + _SLAB])
        out[:, v0:v0 + _SLAB] = np.abs(h64 @ w.T) + np.sqrt(h2 @ (w * w).T)
    return factor * np.sqrt(d) * 2.0 ** -24 * out


# ---------------------------------------------------------------------------
# logits and log-softmax
# ---------------------------------------------------------------------------
def logits(h, W) -> np.ndarray:
    """z[n, v] = sum_i h[n, i] W[v, i] in float64, over the whole vocabulary.

    [Nitrobrew notes, "Nitrobrew 的两个动作": the logits are h times the
    unembedding transposed; the method rebuilds them block by block, here all
    of V is one block.] bf16 x bf16 products are exact in float64 and the
    sums of at most a few thousand terms carry ~1e-16 relative error."""
    h64 = as_f64(h)
    V = W.shape[0]
    z = np.empty((h64.shape[0], V))
    for v0 in range(0, V, _SLAB):  # conversion in slabs bounds host memory only
        z[:, v0:v0 + _SLAB] = h64 @ as_f64(W[v0:v0 + _SLAB]).T
    return z


def lse(x) -> np.ndarray:
    """Natural-log log-sum-exp over the last axis: max + log sum exp(x - max)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    return m[..., 0] + np.log(np.sum(np.exp(x - m), axis=-1))


def log_softmax(x) -> np.ndarray:
    """log softmax(x) = x - lse(x) over the last axis. [White-box OPD, 2.3:
    everything stays in the log domain.]"""
    x = np.asarray(x, dtype=np.float64)
    return x - lse(x)[..., None]


def log1mexp(a):
    """log(1 - exp(a)) for a <= 0, in the numerically stable two-branch form
    (expm1 near 0, log1p far from it); -inf at a == 0."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.where(a > -np.log(2.0), np.log(-np.expm1(a)), np.log1p(-np.exp(a)))


# ---------------------------------------------------------------------------
# divergences (forward pass)
# ---------------------------------------------------------------------------
def divergence(s, t, beta: float):
    """Per-row beta-divergence between the student distribution q = softmax(s)
    and the teacher distribution p = softmax(t) (s, t: tempered logits).

    [White-box OPD, 2.3, the beta table]
      beta = 0 : KL(p || q)                       (forward, teacher first)
      beta = 1 : KL(q || p)                       (reverse, student first)
      else     : beta KL(p || m) + (1-beta) KL(q || m),  m = beta p + (1-beta) q,
                 log m taken with logaddexp (log-domain mixture).
    READING: the endpoints are taken piecewise, as the page's table lists them
    (the mixture formula itself tends to 0 at both ends).

    Returns (loss, aux): aux is the centring scalar of the gradient:
    KL(q || m) for 0 < beta < 1, the loss itself otherwise."""
    lq = log_softmax(s)
    lp = log_softmax(t)
    q = np.exp(lq)
    p = np.exp(lp)
    if beta == 0.0:
        loss = np.sum(p * (lp - lq), axis=-1)
        return loss, loss.copy()
    if beta == 1.0:
        loss = np.sum(q * (lq - lp), axis=-1)
        return loss, loss.copy()
    if not (0.0 < beta < 1.0):
        raise ValueError("beta must lie in [0, 1]")
    lm = np.logaddexp(np.log(beta) + lp, np.log1p(-beta) + lq)
    kl_pm = np.sum(p * (lp - lm), axis=-1)
    kl_qm = np.sum(q * (lq - lm), axis=-1)
    return beta * kl_pm + (1.0 - beta) * kl_qm, kl_qm


def kd_fwd(h_s, W_s, h_t, W_t, beta: float, tau: float):
    """Per-token forward outputs for the rows of h_s / h_t.

    s = z_s / tau, t = z_t / tau ([White-box OPD, 2.3]: the temperature divides
    the logits before the softmax). READING: no tau^2 factor is applied.
    Returns dict(loss, lse_s, lse_t, aux) with lse_* = LSE of the tempered
    logits (natural log)."""
    if tau <= 0:
        raise ValueError("tau must be positive")
    s = logits(h_s, W_s) / tau
    t = logits(h_t, W_t) / tau
    loss, aux = divergence(s, t, beta)
    return dict(loss=loss, lse_s=lse(s), lse_t=lse(t), aux=aux)


# ---------------------------------------------------------------------------
# gradient (backward pass)
# ---------------------------------------------------------------------------
def grad_student_logits(s, t, beta: float) -> np.ndarray:
    """dL/ds for each row, s = tempered student logits.

    Derived from the definitions in ``divergence`` (and pinned by finite
    differences in the tests); the first two agree with [Nitrobrew notes,
    "仓库实现"] once its letters are read as p = student, q = teacher:
      beta = 0 : q - p
      beta = 1 : q (log q - log p - KL(q||p))
      else     : (1 - beta) q (log q - log m - KL(q||m))

    Evaluation. Both centred forms are w q (d - sum_u q_u d_u) with
    d = log q - log p (beta = 1) or log q - log m. When one entry a holds
    nearly all of q, its d - sum q d is tiny while both terms are of the size
    of the log-sum-exps, and the fp64 rounding of the sum over V terms swamps
    it. Subtracting d_a from every d first changes nothing algebraically (the
    weighted mean moves by the same d_a) but makes the dominant term of the
    sum exactly zero, so c = d - d_a and g = w q (c - sum_u q_u c_u) keep
    their relative precision. For beta = 0 the dominant entry's q_a - p_a is
    taken as the equal sum over the other entries of p - q (both
    distributions sum to one)."""
    lq = log_softmax(s)
    lp = log_softmax(t)
    q = np.exp(lq)
    a = np.argmax(lq, axis=-1)[..., None]
    if beta == 0.0:
        g = q - np.exp(lp)
        np.put_along_axis(g, a, 0.0, axis=-1)
        np.put_along_axis(g, a, -np.sum(g, axis=-1, keepdims=True), axis=-1)
        return g
    if beta == 1.0:
        d = lq - lp
        w = 1.0
    else:
        lm = np.logaddexp(np.log(beta) + lp, np.log1p(-beta) + lq)
        d = lq - lm
        w = 1.0 - beta
    c = d - np.take_along_axis(d, a, axis=-1)
    return w * q * (c - np.sum(q * c, axis=-1, keepdims=True))


def kd_bwd(h_s, W_s, h_t, W_t, beta: float, tau: float, grad_loss=None) -> np.ndarray:
    """dL/dh_s[n, :] = grad_loss[n] * sum_v (g[n, v] / tau) W_s[v, :].

    The teacher receives no gradient ([Nitrobrew notes, "仓库实现"]). The
    chain rule through s = z_s / tau contributes the 1/tau."""
    s = logits(h_s, W_s) / tau
    t = logits(h_t, W_t) / tau
    g = grad_student_logits(s, t, beta) / tau
    if grad_loss is not None:
        g = g * np.asarray(grad_loss, dtype=np.float64)[:, None]
    out = np.zeros((g.shape[0], W_s.shape[1]))
    for v0 in range(0, W_s.shape[0], _SLAB):
        out += g[:, v0:v0 + _SLAB] @ as_f64(W_s[v0:v0 + _SLAB])
    return out


def kd_fwd_bwd(h_s, W_s, h_t, W_t, beta: float, tau: float, grad_loss=None):
    """``kd_fwd`` and ``kd_bwd`` of the same rows from one evaluation of the
    logits: returns (dict(loss, lse_s, lse_t, aux), dL/dh_s)."""
    if tau <= 0:
        raise ValueError("tau must be positive")
    s = logits(h_s, W_s) / tau
    t = logits(h_t, W_t) / tau
    loss, aux = divergence(s, t, beta)
    fwd = dict(loss=loss, lse_s=lse(s), lse_t=lse(t), aux=aux)
    g = grad_student_logits(s, t, beta) / tau
    if grad_loss is not None:
        g = g * np.asarray(grad_loss, dtype=np.float64)[:, None]
    dh = np.zeros((g.shape[0], W_s.shape[1]))
    for v0 in range(0, W_s.shape[0], _SLAB):
        dh += g[:, v0:v0 + _SLAB] @ as_f64(W_s[v0:v0 + _SLAB])
    return fwd, dh


def kd_bwd_w(h_s, W_s, h_t, W_t, beta: float, tau: float, grad_loss=None) -> np.ndarray:
    """dL/dW_s[v, :] = sum_n grad_loss[n] * (g[n, v] / tau) * h_s[n, :].

    The student unembedding receives a gradient as well as the student hidden
    state; the teacher's parameters stay fixed ([Nitrobrew notes],
    "工程落地：简单 idea，不等于简单集成"). Same g and 1/tau as ``kd_bwd``: the
    two gradients are the two factors' sides of z_s = h_s W_s^T."""
    s = logits(h_s, W_s) / tau
    t = logits(h_t, W_t) / tau
    g = grad_student_logits(s, t, beta) / tau
    if grad_loss is not None:
        g = g * np.asarray(grad_loss, dtype=np.float64)[:, None]
    return g.T @ as_f64(h_s)


# ---------------------------------------------------------------------------
# top-k three-term decomposition
# ---------------------------------------------------------------------------
def topk_order(keys, k: int) -> np.ndarray:
    """Indices of the k largest keys of each row, ordered by (key descending,
    vocabulary index ascending). READING: the pages fix no tie rule; bf16
    keys tie often at the k-th slot, so the lower index wins."""
    keys = np.asarray(keys, dtype=np.float64)
    V = keys.shape[-1]
    idx = np.arange(V)
    out = np.empty((keys.shape[0], k), dtype=np.int64)
    for r in range(keys.shape[0]):
        order = np.lexsort((idx, -keys[r]))  # last key is primary
        out[r] = order[:k]
    return out


def topk_three_terms(zs_b, zt_b, sel, tau: float, labels=None):
    """Three-term decomposition given bf16-rounded logits and the selection.

    [Top-K KD, 一.2] binary KL: how much teacher mass falls inside the top-k
    set versus outside; conditional KL: the shape inside the set after
    renormalising; CE anchor: cross-entropy of the student on the true token.
    READING: both KLs are teacher-first (forward), the terms are returned
    separately, log(1 - P) is taken as log1mexp(LSE_K - LSE_V), and the CE
    uses the untempered student logits (tau = 1).
    ``sel`` [rows, k] holds the selected vocabulary indices."""
    rows = np.arange(zs_b.shape[0])[:, None]
    s = zs_b / tau
    t = zt_b / tau
    L_s = lse(s)
    L_t = lse(t)
    sK = s[rows, sel]
    tK = t[rows, sel]
    LK_s = lse(sK)
    LK_t = lse(tK)
    logP = LK_t - L_t
    logQ = LK_s - L_s
    P = np.exp(logP)
    Q = np.exp(logQ)
    log1P = log1mexp(np.minimum(logP, 0.0))
    log1Q = log1mexp(np.minimum(logQ, 0.0))
    with np.errstate(invalid="ignore"):
        tail = np.where(1.0 - P > 0.0, (1.0 - P) * (log1P - log1Q), 0.0)
    binary = P * (logP - logQ) + tail
    lpK = tK - LK_t[:, None]  # log of the renormalised teacher inside the set
    lqK = sK - LK_s[:, None]
    cond = np.sum(np.exp(lpK) * (lpK - lqK), axis=-1)
    out = dict(binary=binary, cond=cond, p_mass=P, q_mass=Q, lse_s=L_s, lse_t=L_t)
    if labels is not None:
        lab = np.asarray(labels, dtype=np.int64)
        valid = lab != -100
        L_s1 = lse(zs_b)
        ce = np.full(zs_b.shape[0], np.nan)
        ce[valid] = L_s1[valid] - zs_b[np.arange(zs_b.shape[0])[valid], lab[valid]]
        out["ce"] = ce
    return out


def kd_topk_fwd(h_s, W_s, h_t, W_t, k: int, tau: float, labels=None, with_bound: bool = False):
    """Top-k three-term KD for the given rows.

    Steps ([Top-K KD, 二.1 and 二.2]): round both models' logits to bf16
    (straight from the exact value), pick the teacher's top-k by
    (bf16 key desc, index asc), and evaluate the three terms over full-vocab
    log-sum-exps of the bf16 logits. Returns the dict of ``topk_three_terms``
    plus ``idx`` [rows, k], ``val_t`` (the selected bf16 teacher logits) and,
    with ``with_bound``, the exact teacher logits and their fp32 error bound
    (for judging selections at bf16 rounding midpoints)."""
    zs = logits(h_s, W_s)
    zt = logits(h_t, W_t)
    zs_b = bf16_round(zs)
    zt_b = bf16_round(zt)
    sel = topk_order(zt_b, k)
    out = topk_three_terms(zs_b, zt_b, sel, tau, labels)
    rows = np.arange(zt.shape[0])[:, None]
    out["idx"] = sel
    out["val_t"] = zt_b[rows, sel]
    if with_bound:
        out["zt_exact"] = zt
        out["zt_bound"] = fp32_dot_error_bound(h_t, W_t)
    return out


def topk_grad_student_logits(zs, zt, sel, tau: float, labels=None, w_binary=None, w_cond=None, w_ce=None):
    """dL/dz_s for L = sum_n w_binary[n] binary[n] + w_cond[n] cond[n] + w_ce[n] ce[n]
    (the three terms of ``topk_three_terms``), z_s the untempered student
    logits, with the selection and the teacher's logits held fixed; a weight
    left as None counts as zero. Derived from the definitions, with q the
    tempered student softmax, Q its mass on the set, P the teacher's:
      binary: (-P/Q + (1-P)/(1-Q)) q_v (1[v in K] - Q)           (d/ds)
      cond:   1[v in K] (q_v / Q - p_v / P)                       (d/ds)
      ce:     softmax(z_s)_v - 1[v = label]                        (d/dz)
    and d/dz = (d/ds) / tau. With every entry selected (k = V) the binary
    term is identically 0 and so is its gradient. Pinned by central finite
    differences of ``topk_three_terms``."""
    zs = as_f64(zs)
    zt = as_f64(zt)
    n_rows, V = zs.shape
    rows = np.arange(n_rows)[:, None]
    zero = np.zeros(n_rows)
    wb = zero if w_binary is None else np.asarray(w_binary, dtype=np.float64)
    wc = zero if w_cond is None else np.asarray(w_cond, dtype=np.float64)
    we = zero if w_ce is None else np.asarray(w_ce, dtype=np.float64)
    s = zs / tau
    t = zt / tau
    q = np.exp(s - lse(s)[:, None])
    p = np.exp(t - lse(t)[:, None])
    inK = np.zeros((n_rows, V), dtype=bool)
    inK[rows, sel] = True
    Q = np.sum(np.where(inK, q, 0.0), axis=-1)
    P = np.sum(np.where(inK, p, 0.0), axis=-1)
    g = np.zeros((n_rows, V))
    if sel.shape[1] < V:
        B = -P / Q + (1.0 - P) / (1.0 - Q)
        g += (wb * B)[:, None] * q * (inK - Q[:, None])
    g += wc[:, None] * np.where(inK, q / Q[:, None] - p / P[:, None], 0.0)
    g /= tau
    if labels is not None:
        lab = np.asarray(labels, dtype=np.int64)
        valid = lab != -100
        r = np.exp(zs - lse(zs)[:, None])
        ce_g = r.copy()
        ce_g[np.nonzero(valid)[0], lab[valid]] -= 1.0
        g += np.where(valid, we, 0.0)[:, None] * ce_g
    return g


def kd_topk_bwd(h_s, W_s, h_t, W_t, k: int, tau: float, labels=None, w_binary=None, w_cond=None, w_ce=None,
                sel=None):
    """dL/dh_s for the weighted three top-k terms of ``kd_topk_fwd``.

    ``sel`` [rows, k], when given, is the selection to hold fixed (the one a
    forward pass made, e.g. on a bf16 tie); by default the oracle's own.

    READING: the pages train on the three terms ([Top-K KD, 一.2]) without
    spelling out their gradient. Here it reaches the student hidden state
    through the student logits only (the teacher and the selection made from
    it are fixed), and the bf16 rounding of the student logits is passed
    straight through: the derivative formulas are evaluated at the same bf16
    logits the forward terms use."""
    zs = logits(h_s, W_s)
    zt = logits(h_t, W_t)
    zs_b = bf16_round(zs)
    zt_b = bf16_round(zt)
    if sel is None:
        sel = topk_order(zt_b, k)
    g = topk_grad_student_logits(zs_b, zt_b, np.asarray(sel, dtype=np.int64), tau, labels, w_binary, w_cond, w_ce)
    out = np.zeros((g.shape[0], W_s.shape[1]))
    for v0 in range(0, W_s.shape[0], _SLAB):
        out += g[:, v0:v0 + _SLAB] @ as_f64(W_s[v0:v0 + _SLAB])
    return out


# ---------------------------------------------------------------------------
# top-k support with a tail bucket
# ---------------------------------------------------------------------------
SUPPORT_TEACHER, SUPPORT_STUDENT, SUPPORT_LABEL = 1, 2, 4


def tail_default_support(k: int, beta: float, with_labels: bool) -> int:
    """Which entries make up the support of the tail-bucket divergence.

    [White-box OPD, 2.4] With a single kept entry the support is the sampled
    token (here: the label) together with the teacher's top-1; with more, it is
    the teacher's top-k, the student's top-k or the union of the two with
    duplicates removed, depending on beta.
    READING: the page names the three sets without pairing each with a beta
    value; here each follows the distribution that weights the divergence:
    beta = 0 (forward KL, a teacher-weighted sum) takes the teacher's top-k,
    beta = 1 (reverse KL, student-weighted) the student's, and 0 < beta < 1
    (both weight it) the union. Returns a mask of SUPPORT_* bits."""
    if k == 1:
        return SUPPORT_TEACHER | (SUPPORT_LABEL if with_labels else 0)
    if beta == 0.0:
        return SUPPORT_TEACHER
    if beta == 1.0:
        return SUPPORT_STUDENT
    return SUPPORT_TEACHER | SUPPORT_STUDENT


def tail_support_size(k: int, support: int) -> int:
    """Slots per row of a support array: k per selected model, one for the label."""
    return k * bool(support & SUPPORT_TEACHER) + k * bool(support & SUPPORT_STUDENT) + bool(support & SUPPORT_LABEL)


def tail_support(zs_b, zt_b, k: int, support: int, labels=None) -> np.ndarray:
    """Support indices per row, [rows, tail_support_size(k, support)], -1 padded.

    Order: the teacher's top-k (``topk_order`` of its bf16 logits), then those
    of the student's top-k not already present (in the student's order), then
    the label when it is a vocabulary index not already present. An ignored
    label (-100) adds nothing."""
    if not 1 <= support <= 7 or not support & (SUPPORT_TEACHER | SUPPORT_STUDENT):
        raise ValueError("support must select the teacher's or the student's top-k")
    n_rows, V = zs_b.shape
    out = np.full((n_rows, tail_support_size(k, support)), -1, dtype=np.int64)
    selt = topk_order(zt_b, k) if support & SUPPORT_TEACHER else None
    sels = topk_order(zs_b, k) if support & SUPPORT_STUDENT else None
    for r in range(n_rows):
        row = []
        if selt is not None:
            row += selt[r].tolist()
        if sels is not None:
            row += [v for v in sels[r].tolist() if v not in row]
        if support & SUPPORT_LABEL and labels is not None:
            y = int(labels[r])
            if 0 <= y < V and y not in row:
                row.append(y)
        out[r, :len(row)] = row
    return out


def _divergence_logprobs(lp, lq, beta: float):
    """The beta table of [White-box OPD, 2.3] on given log-probabilities
    (entries of zero mass contribute nothing). Returns (loss, aux) as
    ``divergence`` does."""
    p = np.exp(lp)
    q = np.exp(lq)
    with np.errstate(invalid="ignore", divide="ignore"):
        if beta == 0.0:
            loss = np.sum(np.where(p > 0, p * (lp - lq), 0.0))
            return loss, loss
        if beta == 1.0:
            loss = np.sum(np.where(q > 0, q * (lq - lp), 0.0))
            return loss, loss
        lm = np.logaddexp(np.log(beta) + lp, np.log1p(-beta) + lq)
        kl_pm = np.sum(np.where(p > 0, p * (lp - lm), 0.0))
        kl_qm = np.sum(np.where(q > 0, q * (lq - lm), 0.0))
    return beta * kl_pm + (1.0 - beta) * kl_qm, kl_qm


def _tail_buckets(lp_row, lq_row, S):
    """Bucket log-probabilities: one per support entry, then the tail bucket
    log(1 - sum over the support) ([White-box OPD, 2.4]) when the support
    leaves part of the vocabulary out."""
    lpS = lp_row[S]
    lqS = lq_row[S]
    if len(S) == lp_row.shape[0]:
        return lpS, lqS, False
    lp_tail = log1mexp(min(float(lse(lpS)), 0.0))
    lq_tail = log1mexp(min(float(lse(lqS)), 0.0))
    return np.append(lpS, lp_tail), np.append(lqS, lq_tail), True


def tail_divergence(zs_b, zt_b, sup, beta: float, tau: float):
    """Beta-divergence over the support buckets plus a tail bucket.

    [White-box OPD, 2.4] The divergence is taken on |S| + 1 buckets: each
    support entry keeps its own (tempered, full-vocabulary) probability under
    each model, and one more bucket holds the mass outside the support, so
    that neither distribution loses mass; the beta family is that of
    [White-box OPD, 2.3]. ``sup`` [rows, slots] holds vocabulary indices,
    -1 padded. Returns dict(loss, aux, p_mass, q_mass, lse_s, lse_t) with
    p_mass / q_mass the support's mass under teacher / student and aux the
    gradient's centring scalar as in ``divergence``."""
    s = as_f64(zs_b) / tau
    t = as_f64(zt_b) / tau
    L_s, L_t = lse(s), lse(t)
    lq = s - L_s[:, None]
    lp = t - L_t[:, None]
    n_rows = s.shape[0]
    out = {f: np.zeros(n_rows) for f in ("loss", "aux", "p_mass", "q_mass")}
    for r in range(n_rows):
        S = np.asarray(sup[r])
        S = S[S >= 0]
        lpb, lqb, _ = _tail_buckets(lp[r], lq[r], S)
        out["loss"][r], out["aux"][r] = _divergence_logprobs(lpb, lqb, beta)
        out["p_mass"][r] = np.exp(lse(lp[r, S]))
        out["q_mass"][r] = np.exp(lse(lq[r, S]))
    out["lse_s"] = L_s
    out["lse_t"] = L_t
    return out


def kd_tail_fwd(h_s, W_s, h_t, W_t, k: int, beta: float, tau: float, support=None, labels=None,
                with_bound: bool = False):
    """Tail-bucket divergence from hidden states.

    Both models' logits are rounded to bf16 (as for the three-term split,
    [Top-K KD, 二.1]); the support is picked by ``tail_support`` (by default
    with the rule of ``tail_default_support``) and the divergence is
    ``tail_divergence``. Returns its dict plus ``sup`` and the bf16 logits at
    the support, ``val_t`` / ``val_s`` (NaN in padding slots); with
    ``with_bound`` also both models' exact logits and fp32 error bounds."""
    if support is None:
        support = tail_default_support(k, beta, labels is not None)
    zs = logits(h_s, W_s)
    zt = logits(h_t, W_t)
    zs_b = bf16_round(zs)
    zt_b = bf16_round(zt)
    sup = tail_support(zs_b, zt_b, k, support, labels)
    out = tail_divergence(zs_b, zt_b, sup, beta, tau)
    rows = np.arange(sup.shape[0])[:, None]
    safe = np.maximum(sup, 0)
    out["sup"] = sup
    out["val_t"] = np.where(sup >= 0, zt_b[rows, safe], np.nan)
    out["val_s"] = np.where(sup >= 0, zs_b[rows, safe], np.nan)
    if with_bound:
        out["zs_exact"], out["zt_exact"] = zs, zt
        out["zs_bound"] = fp32_dot_error_bound(h_s, W_s)
        out["zt_bound"] = fp32_dot_error_bound(h_t, W_t)
    return out


def tail_grad_student_logits(zs, zt, sup, beta: float, tau: float) -> np.ndarray:
    """dL/dz_s of ``tail_divergence`` (untempered student logits; the support
    and the teacher held fixed).

    Derived by the chain rule through the bucket masses: with q the tempered
    student softmax over the vocabulary, b(v) the bucket of entry v (its own
    for a support entry, the tail otherwise) and a_b = dL/dq_b,
      dL/ds_v = q_v (a_b(v) - sum_b q_b a_b),    dL/dz = (dL/ds) / tau,
    where beta = 0: a_b = -p_b / q_b;  beta = 1: a_b = log q_b - log p_b + 1;
    0 < beta < 1: a_b = (1 - beta)(log q_b - log m_b). Pinned by central
    finite differences of the pure-Python bucket loss."""
    s = as_f64(zs) / tau
    t = as_f64(zt) / tau
    lq = s - lse(s)[:, None]
    lp = t - lse(t)[:, None]
    q = np.exp(lq)
    g = np.zeros_like(s)
    for r in range(s.shape[0]):
        S = np.asarray(sup[r])
        S = S[S >= 0]
        lpb, lqb, has_tail = _tail_buckets(lp[r], lq[r], S)
        pb, qb = np.exp(lpb), np.exp(lqb)
        if beta == 0.0:
            a = -pb / qb
        elif beta == 1.0:
            a = lqb - lpb + 1.0
        else:
            lm = np.logaddexp(np.log(beta) + lpb, np.log1p(-beta) + lqb)
            a = (1.0 - beta) * (lqb - lm)
        c = np.sum(qb * a)
        bucket_a = np.full(s.shape[1], a[-1] if has_tail else 0.0)
        bucket_a[S] = a[:len(S)]
        g[r] = q[r] * (bucket_a - c)
    return g / tau


def kd_tail_bwd(h_s, W_s, h_t, W_t, k: int, beta: float, tau: float, support=None, labels=None, grad_loss=None,
                sup=None) -> np.ndarray:
    """dL/dh_s of the tail-bucket divergence, grad_loss[n] weighting row n.

    ``sup``, when given, is the support to hold fixed (the one a forward pass
    picked); by default the oracle's own. READING: as for the three top-k
    terms, the support and the teacher are held fixed and the bf16 rounding of
    the student logits is passed straight through."""
    zs_b = bf16_round(logits(h_s, W_s))
    zt_b = bf16_round(logits(h_t, W_t))
    if sup is None:
        if support is None:
            support = tail_default_support(k, beta, labels is not None)
        sup = tail_support(zs_b, zt_b, k, support, labels)
    g = tail_grad_student_logits(zs_b, zt_b, sup, beta, tau)
    if grad_loss is not None:
        g = g * np.asarray(grad_loss, dtype=np.float64)[:, None]
    out = np.zeros((g.shape[0], W_s.shape[1]))
    for v0 in range(0, W_s.shape[0], _SLAB):
        out += g[:, v0:v0 + _SLAB] @ as_f64(W_s[v0:v0 + _SLAB])
    return out


# ---------------------------------------------------------------------------
# rank-r teacher (spectral compression of the hidden state)
# ---------------------------------------------------------------------------
def svd_teacher(h_t, W_t, r: int, method: str = "svd"):
    """Rank-r factorisation of the teacher's logit map.

    [Nitrobrew notes, thread part 6/8: spectral compression sends a rank-k
    version of the hidden state instead of d_model floats; not lossless.]
    With W_t = U S V^T (thin SVD), the compressed teacher is
    W~ = U_r [V, r] and h~ = h_t V_r S_r [N, r], so that h~ W~^T = U_r U_r^T z_t
    (the teacher logits projected on the top-r left singular subspace).

    ``method="gram"`` takes the same factors from the eigendecomposition of
    the d x d Gram matrix W^T W = V S^2 V^T and U_r = W V_r S_r^-1 (cheaper for
    V >> d; adequate for the leading singular values).
    Returns (h~, W~, singular values in descending order) in float64."""
    W = as_f64(W_t)
    if method == "svd":
        U, S, Vt = np.linalg.svd(W, full_matrices=False)
        Vr = Vt[:r].T
        W_r = U[:, :r]
    elif method == "gram":
        G = W.T @ W
        evals, evecs = np.linalg.eigh(G)
        order = np.argsort(evals)[::-1]
        S = np.sqrt(np.maximum(evals[order], 0.0))
        Vr = evecs[:, order[:r]]
        W_r = (W @ Vr) / S[:r]
    else:
        raise ValueError(method)
    h_r = as_f64(h_t) @ (Vr * S[:r])
    return h_r, W_r, S
