"""Shared helpers for the GPU parity tests: device upload of the seeded
inputs and the acceptance checks (tolerances written out here)."""
from __future__ import annotations

import functools

import numpy as np

import kdsynth

# Per-token loss / LSE / top-k terms:  |gpu - ref| <= RTOL * |ref| + ATOL
RTOL = 1e-3
ATOL = 1e-5
# dL/dh_s per token row: cosine >= COS_MIN and max|d| / max|ref| <= MAXREL
COS_MIN = 0.9999
MAXREL = 2e-2


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def upload(w):
    return tuple(to_dev(x) for x in (w.h_s, w.W_s, w.h_t, w.W_t))


@functools.lru_cache(maxsize=2)
def workload(cfg: int, **over):
    return kdsynth.make(cfg, **over)


def close(gpu, ref, rtol=RTOL, atol=ATOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    lim = rtol * np.abs(ref) + atol
    bad = ~(err <= lim)
    with np.errstate(invalid="ignore", divide="ignore"):
        worst = float(np.max(err / lim)) if err.size else 0.0
    return (not bad.any()), worst, np.nonzero(bad)[0][:8]


def assert_close(name, gpu, ref, rtol=RTOL, atol=ATOL):
    ok, worst, where = close(gpu, ref, rtol, atol)
    assert ok, f"{name}: worst err/limit {worst:.3g} at rows {where.tolist()} gpu={np.asarray(gpu)[where][:4]} ref={np.asarray(ref)[where][:4]}"


U32 = 2.0 ** -24  # unit roundoff of fp32


def grad_floor(lse_s, lse_t, loss, W_s, tau):
    """Per-row absolute floor below which an fp32 evaluation of dL/dh_s cannot
    be resolved: the gradient term of a saturated entry is a difference of
    O(|L_s| + |L_t| + |KL|) quantities, each carrying fp32 rounding of relative
    size 2^-24, and enters dh_s scaled by a W_s row and 1/tau. Eight roundings
    are allowed for. Rows whose exact gradient is below the floor are compared
    absolutely (|gpu - ref| <= floor)."""
    from oracle import kd_oracle as O
    wmax = 0.0
    for v0 in range(0, W_s.shape[0], 16384):
        w = O.as_f64(W_s[v0:v0 + 16384])
        wmax = max(wmax, float(np.sqrt(np.max(np.sum(w * w, axis=1)))))
    return 8 * U32 * (2 * np.abs(lse_s) + 2 * np.abs(lse_t) + np.abs(loss)) * wmax / tau


def wgrad_floor(h_s, W_s, h_t, W_t, beta, tau, grad=None):
    """Per-row floor of dL/dW_s in fp32 (small cases only: uses full logits).
    Row v gathers sum_n dL/ds[n, v] h_s[n] / tau; the fp32 error of each
    dL/ds[n, v] is bounded like the dh_s floor's (eight roundings of the
    O(|L_s| + |L_t| + |KL|) terms), weighted by that entry's student
    probability, so row v's floor is the sum over tokens of that bound times
    max(q[n, v], the teacher's p[n, v]) times |h_s[n]| |grad[n]|."""
    from oracle import kd_oracle as O
    s = O.logits(h_s, W_s) / tau
    t = O.logits(h_t, W_t) / tau
    q = np.exp(O.log_softmax(s))
    p = np.exp(O.log_softmax(t))
    ref = O.kd_fwd(h_s, W_s, h_t, W_t, beta, tau)
    per_tok = 8 * U32 * (2 * np.abs(ref["lse_s"]) + 2 * np.abs(ref["lse_t"]) + np.abs(ref["loss"])) / tau
    hn = np.linalg.norm(O.as_f64(h_s), axis=1)
    gw = np.ones(h_s.shape[0]) if grad is None else np.abs(np.asarray(grad, dtype=np.float64))
    return (np.maximum(q, p) * (per_tok * hn * gw)[:, None]).sum(axis=0)


def assert_grad_rows(gpu, ref, name="dh_s", floor=None):
    """Per row: cosine >= COS_MIN and max|d|/max|ref| <= MAXREL; rows whose
    reference norm is below ``floor`` (see grad_floor) must instead agree to
    within the floor. The cosine over all rows together must also hold."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    for i in range(ref.shape[0]):
        rn = np.linalg.norm(ref[i])
        f = 1e-12 if floor is None else max(float(floor[i]), 1e-12)
        if rn <= f:
            d = float(np.linalg.norm(gpu[i] - ref[i]))
            assert d <= max(f, 1e-6), f"{name} row {i}: |ref|={rn:.3g} below the fp32 floor {f:.3g}, |d|={d:.3g}"
            continue
        cos = float(gpu[i] @ ref[i] / (np.linalg.norm(gpu[i]) * rn + 1e-300))
        mrel = float(np.max(np.abs(gpu[i] - ref[i])) / np.max(np.abs(ref[i])))
        assert cos >= COS_MIN and mrel <= MAXREL, f"{name} row {i}: cos={cos:.7f} maxrel={mrel:.3g}"
    gcos = float(np.sum(gpu * ref) / (np.linalg.norm(gpu) * np.linalg.norm(ref) + 1e-300))
    assert gcos >= COS_MIN, f"{name}: global cosine {gcos:.7f}"


def check_topk_rows(out, h_s, W_s, h_t, W_t, rows, k, tau, labels=None, factor=8.0):
    """Acceptance of kd_topk_fwd on ``rows`` against the fp64 oracle.

    The kernel rounds fp32-accumulated logits to bf16, the oracle rounds the
    exact logits; a logit within the fp32 accumulation bound of a bf16
    rounding midpoint may round either way (``ambiguous``). Per row:
      * every returned teacher / student value is the oracle's rounding, or the
        other neighbour for an ambiguous logit;
      * the list is ordered by (value desc, index asc) and no other vocabulary
        entry can rank above its last element under any admissible rounding;
      * the list equals the oracle's own top-k unless an ambiguous logit is
        involved (returned as ``flagged``);
      * the three terms and both LSEs match the oracle evaluated on the
        kernel's own roundings of the selected logits (tolerances above).
    Returns (exact_rows, flagged_rows)."""
    from oracle import kd_oracle as O
    idx = out["idx"].cpu().numpy()[rows]
    vt = out["val"].cpu().numpy()[rows].astype(np.float64)
    vs = out["val_s"].cpu().numpy()[rows].astype(np.float64)
    zt = O.logits(h_t[rows], W_t)
    zs = O.logits(h_s[rows], W_s)
    bt = O.fp32_dot_error_bound(h_t[rows], W_t, factor)
    bs = O.fp32_dot_error_bound(h_s[rows], W_s, factor)
    exact = flagged = 0
    for i in range(len(rows)):
        rt, rs = O.bf16_round(zt[i]), O.bf16_round(zs[i])
        lo_t, hi_t, mid_t = O.bf16_neighbours(zt[i])
        lo_s, hi_s, mid_s = O.bf16_neighbours(zs[i])
        amb_t = np.abs(zt[i] - mid_t) <= bt[i]
        amb_s = np.abs(zs[i] - mid_s) <= bs[i]
        alt_t = np.where(rt == lo_t, hi_t, lo_t)
        alt_s = np.where(rs == lo_s, hi_s, lo_s)
        sel = idx[i].astype(np.int64)
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < W_t.shape[0], f"row {i}: bad indices"
        okt = (vt[i] == rt[sel]) | (amb_t[sel] & (vt[i] == alt_t[sel]))
        oks = (vs[i] == rs[sel]) | (amb_s[sel] & (vs[i] == alt_s[sel]))
        assert okt.all(), f"row {i}: teacher values {vt[i][~okt][:4]} vs {rt[sel][~okt][:4]}"
        assert oks.all(), f"row {i}: student values {vs[i][~oks][:4]} vs {rs[sel][~oks][:4]}"
        for j in range(k - 1):
            assert (vt[i][j] > vt[i][j + 1]) or (vt[i][j] == vt[i][j + 1] and sel[j] < sel[j + 1]), f"row {i}: order at {j}"
        rest = np.ones(W_t.shape[0], bool)
        rest[sel] = False
        minkey = np.where(amb_t, np.minimum(rt, alt_t), rt)
        last_v, last_i = vt[i][-1], sel[-1]
        v_idx = np.arange(W_t.shape[0])
        above = rest & ((minkey > last_v) | ((minkey == last_v) & (v_idx < last_i)))
        assert not above.any(), f"row {i}: entries {v_idx[above][:5]} must outrank the last selected"
        ref_sel = O.topk_order(rt[None], k)[0]
        if np.array_equal(ref_sel, sel):
            exact += 1
        else:
            flagged += 1
            assert (amb_t & ((np.abs(rt - last_v) <= 2 * np.abs(hi_t - lo_t)))).any(), f"row {i}: differs without ambiguity"
        zt_b, zs_b = rt.copy(), rs.copy()
        zt_b[sel] = vt[i]
        zs_b[sel] = vs[i]
        ref = O.topk_three_terms(zs_b[None], zt_b[None], sel[None], tau)
        for name, key in (("binary", "binary"), ("cond", "cond"), ("p_mass", "p_mass"), ("q_mass", "q_mass"),
                          ("lse_s", "lse_s"), ("lse_t", "lse_t")):
            g = float(out[name].cpu().numpy()[rows[i]])
            assert_close(f"row {i} {name}", np.array([g]), ref[key])
        if labels is not None:
            y = int(labels[rows[i]])
            g = float(out["ce"].cpu().numpy()[rows[i]])
            if y == -100:
                assert np.isnan(g)
            else:
                cands = [rs[y]] + ([alt_s[y]] if amb_s[y] else [])
                oks_ce = []
                for c in cands:
                    zz = zs_b.copy()
                    zz[y] = c
                    ce_ref = O.lse(zz) - c
                    oks_ce.append(close(np.array([g]), np.array([ce_ref]))[0])
                assert any(oks_ce), f"row {i} ce {g} vs {O.lse(zs_b) - rs[y]}"
    return exact, flagged


def check_tail_rows(out, h_s, W_s, h_t, W_t, rows, k, beta, tau, support, labels=None, factor=8.0):
    """Acceptance of kd_tail_fwd on ``rows`` against the fp64 oracle.

    As for the top-k terms, a logit within the fp32 accumulation bound of a
    bf16 rounding midpoint may round either way (``ambiguous``). Per row:
      * the support holds distinct vocabulary indices in a prefix, -1 / NaN
        after it, and its size is what the support bits allow;
      * every returned teacher / student value is the oracle's rounding, or
        the other neighbour for an ambiguous logit;
      * the ranked model's list (the teacher's when its bit is set, else the
        student's) is ordered by (value desc, index asc) and no other entry
        can outrank its last element under any admissible rounding;
      * the support equals the oracle's own unless an ambiguous logit is
        involved (returned as ``flagged``);
      * loss, masses and LSEs match the oracle's tail divergence evaluated on
        the kernel's support and its own roundings of the support's logits.
    Returns (exact_rows, flagged_rows)."""
    from oracle import kd_oracle as O
    T, S, L = O.SUPPORT_TEACHER, O.SUPPORT_STUDENT, O.SUPPORT_LABEL
    V = W_t.shape[0]
    sup = out["sup_idx"].cpu().numpy()[rows]
    vt = out["sup_t"].cpu().numpy()[rows].astype(np.float64)
    vs = out["sup_s"].cpu().numpy()[rows].astype(np.float64)
    res = {f: out[f].cpu().numpy()[rows] for f in ("loss", "p_mass", "q_mass", "lse_s", "lse_t")}
    zt = O.logits(h_t[rows], W_t)
    zs = O.logits(h_s[rows], W_s)
    bt = O.fp32_dot_error_bound(h_t[rows], W_t, factor)
    bs = O.fp32_dot_error_bound(h_s[rows], W_s, factor)
    exact = flagged = 0
    v_idx = np.arange(V)
    for i in range(len(rows)):
        rt, rs = O.bf16_round(zt[i]), O.bf16_round(zs[i])
        lo_t, hi_t, mid_t = O.bf16_neighbours(zt[i])
        lo_s, hi_s, mid_s = O.bf16_neighbours(zs[i])
        amb_t = np.abs(zt[i] - mid_t) <= bt[i]
        amb_s = np.abs(zs[i] - mid_s) <= bs[i]
        alt_t = np.where(rt == lo_t, hi_t, lo_t)
        alt_s = np.where(rs == lo_s, hi_s, lo_s)
        n = int(np.sum(sup[i] >= 0))
        row = sup[i, :n].astype(np.int64)
        assert np.all(sup[i, n:] == -1) and np.all(np.isnan(vt[i, n:])) and np.all(np.isnan(vs[i, n:])), \
            f"row {i}: padding"
        assert len(set(row.tolist())) == n and (n == 0 or (row.min() >= 0 and row.max() < V)), f"row {i}: indices"
        lab = None if labels is None else int(labels[rows[i]])
        ranked = (support & T) + (support & S) // 2
        assert k <= n <= k * ranked + (1 if support & L else 0), f"row {i}: support size {n}"
        okt = (vt[i, :n] == rt[row]) | (amb_t[row] & (vt[i, :n] == alt_t[row]))
        oks = (vs[i, :n] == rs[row]) | (amb_s[row] & (vs[i, :n] == alt_s[row]))
        assert okt.all(), f"row {i}: teacher values {vt[i, :n][~okt][:4]} vs {rt[row][~okt][:4]}"
        assert oks.all(), f"row {i}: student values {vs[i, :n][~oks][:4]} vs {rs[row][~oks][:4]}"
        if support & L and lab is not None and 0 <= lab < V:
            assert lab in row.tolist(), f"row {i}: label {lab} missing"
        # the first ranked list: ordered, and nothing outranks its last element
        vals, r_, amb, alt = (vt[i], rt, amb_t, alt_t) if support & T else (vs[i], rs, amb_s, alt_s)
        head = row[:k]
        for j in range(k - 1):
            assert (vals[j] > vals[j + 1]) or (vals[j] == vals[j + 1] and head[j] < head[j + 1]), f"row {i}: order {j}"
        rest = np.ones(V, bool)
        rest[head] = False
        minkey = np.where(amb, np.minimum(r_, alt), r_)
        above = rest & ((minkey > vals[k - 1]) | ((minkey == vals[k - 1]) & (v_idx < head[-1])))
        assert not above.any(), f"row {i}: entries {v_idx[above][:5]} must outrank the last ranked entry"
        ref_sup = O.tail_support(rs[None], rt[None], k, support, None if lab is None else np.array([lab]))[0]
        if np.array_equal(ref_sup[ref_sup >= 0], row):
            exact += 1
        else:
            flagged += 1
            assert (amb_t | amb_s).any(), f"row {i}: support differs without ambiguity"
        zt_b, zs_b = rt.copy(), rs.copy()
        zt_b[row] = vt[i, :n]
        zs_b[row] = vs[i, :n]
        ref = O.tail_divergence(zs_b[None], zt_b[None], row[None], beta, tau)
        for f in ("loss", "p_mass", "q_mass", "lse_s", "lse_t"):
            assert_close(f"row {i} {f}", res[f][i:i + 1], ref[f])
    return exact, flagged
