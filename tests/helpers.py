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

# (test, rows, exact, flagged) of every top-k / tail acceptance run in this
# session; tests/conftest.py prints them at the end of the run.
PARITY_COUNTS = []


def record_counts(what, rows, exact, flagged):
    PARITY_COUNTS.append((what, int(rows), int(exact), int(flagged)))
    print(f"{what}: rows {rows} exact {exact} flagged {flagged}", flush=True)


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
    reference norm is below 1e-12 (or below ``floor``, see wgrad_floor) must
    instead agree to within max(that, 1e-6). The cosine over all rows
    together must also hold."""
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


class _Rounding:
    """Oracle roundings of one row's exact logits z (over the whole vocabulary)
    and, on demand for a set of columns, the bf16 values the GPU may return:
    it rounds (nearest even) an fp32 accumulation within the oracle's bound B
    of z, so any bf16 value from round(z - B) to round(z + B) is admissible
    (one value, or the two neighbours of a midpoint, or several steps for
    logits near zero, where B spans more than one bf16 step)."""

    def __init__(self, h_row, W, z, factor):
        from oracle import kd_oracle as O
        self.O, self.h, self.W, self.z, self.factor = O, h_row, W, z, factor
        self.r = O.bf16_round(z)

    def admissible(self, cols):
        """(lo, hi): the smallest and largest admissible bf16 value per column."""
        O = self.O
        cols = np.asarray(cols, dtype=np.int64)
        if cols.size == 0:
            return np.zeros(0), np.zeros(0)
        z = self.z[cols]
        b = O.fp32_dot_error_bound(self.h[None], self.W[cols], self.factor)[0]
        return O.bf16_round(z - b), O.bf16_round(z + b)

    def ambiguous(self, cols):
        lo, hi = self.admissible(cols)
        return lo < hi

    def step(self, cols):
        lo, hi, _ = self.O.bf16_neighbours(self.z[np.asarray(cols, dtype=np.int64)])
        return np.abs(hi - lo)


def _ranked_list_ok(i, rk, vals, head, k, V, what):
    """The ranked list ``head`` (values ``vals``) is ordered by (value desc,
    index asc) and no other entry can outrank its last element under any
    admissible rounding."""
    for j in range(k - 1):
        assert (vals[j] > vals[j + 1]) or (vals[j] == vals[j + 1] and head[j] < head[j + 1]), f"row {i}: {what} order {j}"
    last_v, last_i = vals[k - 1], head[k - 1]
    rest = np.ones(V, bool)
    rest[head] = False
    # entries that can outrank it have an admissible value >= last_v; their own
    # rounding is then within the bound of last_v, so a superset is r >= last_v - 1
    cand = np.flatnonzero(rest & (rk.r >= last_v - 1.0))
    minkey = rk.admissible(cand)[0]
    above = (minkey > last_v) | ((minkey == last_v) & (cand < last_i))
    assert not above.any(), f"row {i}: {what} entries {cand[above][:5]} must outrank the last ranked entry"


def _near_kth(rk, k):
    """Columns whose oracle rounding lies within four bf16 steps of the k-th
    largest one: where a differing rounding can change a top-k selection."""
    kth = np.partition(rk.r, -k)[-k]
    col = np.argpartition(rk.r, -k)[-k]
    return np.flatnonzero(np.abs(rk.r - kth) <= 4 * rk.step([col])[0])


def _values_ok(i, rk, cols, vals, what):
    lo, hi = rk.admissible(cols)
    ok = (vals >= lo) & (vals <= hi)
    assert ok.all(), f"row {i}: {what} values {vals[~ok][:4]} vs oracle {rk.r[cols][~ok][:4]}"


def check_topk_rows(out, h_s, W_s, h_t, W_t, rows, k, tau, labels=None, factor=8.0, block=64):
    """Acceptance of kd_topk_fwd on ``rows`` against the fp64 oracle.

    The kernel rounds fp32-accumulated logits to bf16, the oracle rounds the
    exact logits; a logit within the fp32 accumulation bound of a bf16
    rounding midpoint may round either way (``ambiguous``). Per row:
      * every returned teacher / student value is an admissible rounding: a
        bf16 value within the fp32 accumulation bound of the exact logit;
      * the list is ordered by (value desc, index asc) and no other vocabulary
        entry can rank above its last element under any admissible rounding;
      * the list equals the oracle's own top-k unless an ambiguous logit is
        involved (returned as ``flagged``);
      * the three terms and both LSEs match the oracle evaluated on the
        kernel's own roundings of the selected logits (tolerances above).
    Rows are processed ``block`` at a time. Returns (exact_rows, flagged_rows)."""
    from oracle import kd_oracle as O
    rows = np.asarray(rows)
    idx_all = out["idx"].cpu().numpy()
    vt_all = out["val"].cpu().numpy()
    vs_all = out["val_s"].cpu().numpy()
    res = {f: out[f].cpu().numpy() for f in ("binary", "cond", "p_mass", "q_mass", "lse_s", "lse_t")}
    ce_all = out["ce"].cpu().numpy() if labels is not None else None
    V = W_t.shape[0]
    exact = flagged = 0
    for b0 in range(0, len(rows), block):
        rb = rows[b0:b0 + block]
        zt_blk = O.logits(h_t[rb], W_t)
        zs_blk = O.logits(h_s[rb], W_s)
        for j, n in enumerate(rb):
            i = b0 + j
            rt = _Rounding(h_t[n], W_t, zt_blk[j], factor)
            rs = _Rounding(h_s[n], W_s, zs_blk[j], factor)
            sel = idx_all[n].astype(np.int64)
            vt = vt_all[n].astype(np.float64)
            vs = vs_all[n].astype(np.float64)
            assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < V, f"row {i}: bad indices"
            _values_ok(i, rt, sel, vt, "teacher")
            _values_ok(i, rs, sel, vs, "student")
            _ranked_list_ok(i, rt, vt, sel, k, V, "teacher")
            zt_b, zs_b = rt.r.copy(), rs.r.copy()
            zt_b[sel] = vt
            zs_b[sel] = vs
            if np.array_equal(O.topk_order(rt.r[None], k)[0], sel):
                exact += 1
            else:
                # explained by the kernel's own (admissible) roundings of the listed
                # logits, or else by an ambiguous logit near the k-th key
                flagged += 1
                assert np.array_equal(O.topk_order(zt_b[None], k)[0], sel) or \
                    rt.ambiguous(_near_kth(rt, k)).any(), f"row {i}: differs without ambiguity"
            ref = O.topk_three_terms(zs_b[None], zt_b[None], sel[None], tau)
            for name in ("binary", "cond", "p_mass", "q_mass", "lse_s", "lse_t"):
                assert_close(f"row {i} {name}", res[name][n:n + 1], ref[name])
            if labels is not None:
                y = int(labels[n])
                g = float(ce_all[n])
                if y == -100:
                    assert np.isnan(g)
                else:
                    lo_y, hi_y = rs.admissible([y])
                    cands = sorted({float(rs.r[y]), float(lo_y[0]), float(hi_y[0])})
                    oks_ce = []
                    for c in cands:
                        zz = zs_b.copy()
                        zz[y] = c
                        oks_ce.append(close(np.array([g]), np.array([O.lse(zz) - c]))[0])
                    assert any(oks_ce), f"row {i} ce {g} vs {O.lse(zs_b) - zs_b[y]}"
    record_counts(f"top-k k={k} V={V}", len(rows), exact, flagged)
    return exact, flagged


def check_tail_rows(out, h_s, W_s, h_t, W_t, rows, k, beta, tau, support, labels=None, factor=8.0, block=64):
    """Acceptance of kd_tail_fwd on ``rows`` against the fp64 oracle.

    As for the top-k terms, a logit within the fp32 accumulation bound of a
    bf16 rounding midpoint may round either way (``ambiguous``). Per row:
      * the support holds distinct vocabulary indices in a prefix, -1 / NaN
        after it, and its size is what the support bits allow;
      * every returned teacher / student value is an admissible rounding: a
        bf16 value within the fp32 accumulation bound of the exact logit;
      * the ranked model's list (the teacher's when its bit is set, else the
        student's) is ordered by (value desc, index asc) and no other entry
        can outrank its last element under any admissible rounding;
      * the support equals the oracle's own unless an ambiguous logit is
        involved (returned as ``flagged``);
      * loss, masses and LSEs match the oracle's tail divergence evaluated on
        the kernel's support and its own roundings of the support's logits.
    Rows are processed ``block`` at a time. Returns (exact_rows, flagged_rows)."""
    from oracle import kd_oracle as O
    T, S, L = O.SUPPORT_TEACHER, O.SUPPORT_STUDENT, O.SUPPORT_LABEL
    rows = np.asarray(rows)
    V = W_t.shape[0]
    sup_all = out["sup_idx"].cpu().numpy()
    vt_all = out["sup_t"].cpu().numpy()
    vs_all = out["sup_s"].cpu().numpy()
    res = {f: out[f].cpu().numpy() for f in ("loss", "p_mass", "q_mass", "lse_s", "lse_t")}
    exact = flagged = 0
    for b0 in range(0, len(rows), block):
        rb = rows[b0:b0 + block]
        zt_blk = O.logits(h_t[rb], W_t)
        zs_blk = O.logits(h_s[rb], W_s)
        for j, nn in enumerate(rb):
            i = b0 + j
            rt = _Rounding(h_t[nn], W_t, zt_blk[j], factor)
            rs = _Rounding(h_s[nn], W_s, zs_blk[j], factor)
            vt = vt_all[nn].astype(np.float64)
            vs = vs_all[nn].astype(np.float64)
            n = int(np.sum(sup_all[nn] >= 0))
            row = sup_all[nn, :n].astype(np.int64)
            assert np.all(sup_all[nn, n:] == -1) and np.all(np.isnan(vt[n:])) and np.all(np.isnan(vs[n:])), \
                f"row {i}: padding"
            assert len(set(row.tolist())) == n and (n == 0 or (row.min() >= 0 and row.max() < V)), f"row {i}: indices"
            lab = None if labels is None else int(labels[nn])
            ranked = (support & T) + (support & S) // 2
            assert k <= n <= k * ranked + (1 if support & L else 0), f"row {i}: support size {n}"
            _values_ok(i, rt, row, vt[:n], "teacher")
            _values_ok(i, rs, row, vs[:n], "student")
            if support & L and lab is not None and 0 <= lab < V:
                assert lab in row.tolist(), f"row {i}: label {lab} missing"
            # the first ranked list: ordered, and nothing outranks its last element
            vals, rk = (vt, rt) if support & T else (vs, rs)
            _ranked_list_ok(i, rk, vals, row[:k], k, V, "ranked")
            zt_b, zs_b = rt.r.copy(), rs.r.copy()
            zt_b[row] = vt[:n]
            zs_b[row] = vs[:n]
            labs = None if lab is None else np.array([lab])
            ref_sup = O.tail_support(rs.r[None], rt.r[None], k, support, labs)[0]
            if np.array_equal(ref_sup[ref_sup >= 0], row):
                exact += 1
            else:
                # explained by the kernel's own (admissible) roundings of the support's
                # logits (order or membership), or else by an ambiguous logit near a
                # ranked model's k-th key (a rounding the kernel does not return)
                flagged += 1
                own = O.tail_support(zs_b[None], zt_b[None], k, support, labs)[0]
                amb = np.array_equal(own[own >= 0], row) or \
                    (bool(support & T) and rt.ambiguous(_near_kth(rt, k)).any()) or \
                    (bool(support & S) and rs.ambiguous(_near_kth(rs, k)).any())
                assert amb, f"row {i}: support differs without ambiguity"
            ref = O.tail_divergence(zs_b[None], zt_b[None], row[None], beta, tau)
            for f in ("loss", "p_mass", "q_mass", "lse_s", "lse_t"):
                assert_close(f"row {i} {f}", res[f][nn:nn + 1], ref[f])
    record_counts(f"tail k={k} beta={beta} support={support} V={V}", len(rows), exact, flagged)
    return exact, flagged


def exact_shifted_case(seed, N, V, d, shift=100.0, head=0.0, n_head=8, teacher=False):
    """A case whose logits are exact in bf16 and whose student logits all lie
    past the range of exp in fp32: hidden units in {0, 1}, unembedding entries
    in {0, +-1/2}, and for the student a last hidden unit of ``shift`` against
    an unembedding column of ones (a column of ``shift`` would instead scale
    the bf16 rounding residue of the stored gradient, whose exact entries sum
    to zero, into dL/dh_s). Every logit is then a multiple of 1/2
    summed exactly in fp32; the student's lie near ``shift`` (kept below 128,
    where bf16 still has steps of 1/2), so rounding them to bf16 is exact and
    the softmax is that of the unshifted logits. The spread is small, so a
    top-k of a few thousand entries holds little of either model's mass.
    With a nonzero ``head`` the first ``n_head`` vocabulary rows lead both
    models by ``head`` (a hidden unit of 1 against that column), so a top-k
    of ``n_head`` holds most of both masses and the binary term of the
    top-k decomposition is near zero. With ``teacher`` the teacher's logits
    are raised the same way instead of the student's."""
    g = np.random.default_rng(seed)
    vals = np.array([-0.5, 0.0, 0.5], np.float32)
    h_s = g.integers(0, 2, (N, d)).astype(np.float32)
    W_s = vals[g.integers(0, 3, (V, d))]
    h_t = g.integers(0, 2, (N, d)).astype(np.float32)
    W_t = vals[g.integers(0, 3, (V, d))]
    if head:
        for h, W in ((h_s, W_s), (h_t, W_t)):
            h[:, -2] = 1.0
            W[:, -2] = 0.0
            W[:n_head, -2] = head
    h, W = (h_t, W_t) if teacher else (h_s, W_s)
    h[:, -1] = shift
    W[:, -1] = 1.0
    z = h @ W.T
    assert z.min() > 89.0 and z.max() < 127.5, (z.min(), z.max())
    return tuple(kdsynth.f32_to_bf16_bits(x) for x in (h_s, W_s, h_t, W_t))
