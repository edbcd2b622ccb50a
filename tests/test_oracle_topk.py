"""Pins for the oracle's bf16 rounding, top-k order, three-term decomposition
and rank-r teacher (CPU only).

Sources: Top-K KD (section 一.2 the three terms; section 二.1 bf16 logits with
fp32 accumulators; section 二.2 gather the top-64 in bf16), White-box OPD
(section 2.4 tail bucket), Nitrobrew notes (thread part 6/8, spectral
compression of the hidden state).
"""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import kd_oracle as O


def f32_rne_bits(x32):
    """bf16 rounding of float32 values via the bit pattern (independent route)."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return ((r.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)


# --------------------------------------------------------------------------- bf16 rounding
def test_bf16_round_known_values():
    e = 2.0 ** -8
    cases = {
        1.0: 1.0,
        1.0 + e: 1.0,  # exact midpoint between 1 and 1+2^-7: ties to even (1.0)
        1.0 + 3 * e: 1.0 + 2 * 2.0 ** -7,  # midpoint between odd and even mantissa -> even
        1.0 + e + 2.0 ** -30: 1.0 + 2.0 ** -7,  # just above the midpoint (a float32 detour would lose this)
        -(1.0 + e + 2.0 ** -30): -(1.0 + 2.0 ** -7),
        3.0e38: 3.00405527047391e38,  # below the largest finite bf16 (3.3895e38)
        3.4e38: math.inf,  # past the midpoint above the largest finite bf16
        0.0: 0.0,
    }
    for x, want in cases.items():
        got = float(O.bf16_round(np.array([x]))[0])
        assert got == want, (x, got, want)
    # the float32 detour really differs on the double-rounding case
    assert f32_rne_bits(np.float32(1.0 + e + 2.0 ** -30))[()] == 1.0


def test_bf16_round_agrees_with_bit_route_on_float32_values():
    g = np.random.default_rng(0)
    x = np.concatenate([g.normal(0, 5, 200000), g.normal(0, 1e-3, 1000), g.normal(0, 1e30, 1000)]).astype(np.float32)
    assert np.array_equal(O.bf16_round(x.astype(np.float64)), f32_rne_bits(x))


def test_log1mexp_against_scalar_routes_and_its_branch_point():
    """log(1 - e^a), the log of the mass outside a top-k set from the set's
    log-mass a [Top-K KD, 一.2 binary term]: pinned per element to Python's
    scalar math (log of -expm1 near 0, log1p of -exp far from it, each exact
    to a few ulps where it is used), on both sides of the branch point
    -log 2, at a = 0 (no mass outside: -inf) and at a tiny |a| where the
    naive log(1 - exp(a)) loses every digit."""
    a = np.concatenate([-np.logspace(-300, 3, 400), [-math.log(2.0) * (1 + 1e-15), -math.log(2.0),
                                                       -math.log(2.0) * (1 - 1e-15), -1e-20]])
    got = O.log1mexp(a)
    for x, g in zip(a.tolist(), got.tolist()):
        ref = math.log(-math.expm1(x)) if x > -0.5 else math.log1p(-math.exp(x))
        assert abs(g - ref) <= 4e-16 * abs(ref), (x, g, ref)
    assert O.log1mexp(np.array([0.0]))[0] == -np.inf
    assert abs(O.log1mexp(np.array([-1e-20]))[0] - math.log(1e-20)) < 1e-12
    assert 1.0 - math.exp(-1e-20) == 0.0  # the naive form has nothing left to take the log of


def test_bf16_neighbours_bracket():
    g = np.random.default_rng(1)
    x = g.normal(0, 10, 10000)
    lo, hi, mid = O.bf16_neighbours(x)
    r = O.bf16_round(x)
    assert np.all(lo <= x) and np.all(x <= hi)
    assert np.all((r == lo) | (r == hi))
    assert np.all(np.where(np.abs(x - lo) < np.abs(x - hi), r == lo, True))


# --------------------------------------------------------------------------- top-k order
def test_topk_order_matches_brute_force_with_ties():
    g = np.random.default_rng(2)
    keys = np.round(g.normal(0, 2, size=(20, 300)) * 4) / 4  # heavy ties
    for k in (1, 7, 64, 300):
        got = O.topk_order(keys, k)
        for r in range(keys.shape[0]):
            assert got[r].tolist() == brute.topk_row(keys[r].tolist(), k)


# --------------------------------------------------------------------------- three terms
def _case(seed, V=200, N=4):
    g = np.random.default_rng(seed)
    zs = O.bf16_round(g.normal(0, 3, (N, V)))
    zt = O.bf16_round(g.normal(0, 3, (N, V)))
    return zs, zt


@pytest.mark.parametrize("tau", (1.0, 1.7))
def test_three_terms_match_brute_force(tau):
    zs, zt = _case(3)
    k = 16
    sel = O.topk_order(zt, k)
    out = O.topk_three_terms(zs, zt, sel, tau)
    for r in range(zs.shape[0]):
        b, c, P, Q = brute.three_terms_row(zs[r].tolist(), zt[r].tolist(), sel[r].tolist(), tau)
        assert abs(out["binary"][r] - b) < 1e-12 and abs(out["cond"][r] - c) < 1e-12
        assert abs(out["p_mass"][r] - P) < 1e-13 and abs(out["q_mass"][r] - Q) < 1e-13


def test_full_set_reduces_to_forward_kl():
    zs, zt = _case(4, V=50)
    sel = O.topk_order(zt, 50)
    out = O.topk_three_terms(zs, zt, sel, 1.0)
    fkl, _ = O.divergence(zs, zt, 0.0)
    assert np.allclose(out["binary"], 0.0, atol=1e-14)
    assert np.allclose(out["cond"], fkl, rtol=1e-12)
    assert np.allclose(out["p_mass"], 1.0)


def test_single_entry_has_zero_conditional_kl():
    zs, zt = _case(5)
    sel = O.topk_order(zt, 1)
    out = O.topk_three_terms(zs, zt, sel, 1.0)
    assert np.allclose(out["cond"], 0.0, atol=1e-15)


@pytest.mark.parametrize("tau", (1.0, 2.5))
def test_chain_rule_and_tail_bucket(tau):
    # KL(p||q) = binary + P*cond + (1-P)*cond_tail  (chain rule of KL over the
    # partition {top-k, rest}); the (k+1)-bucket KL (White-box OPD 2.4's tail
    # bucket) equals binary + P*cond.
    zs, zt = _case(6, V=300, N=5)
    k = 20
    sel = O.topk_order(zt, k)
    out = O.topk_three_terms(zs, zt, sel, tau)
    s, t = zs / tau, zt / tau
    lq, lp = O.log_softmax(s), O.log_softmax(t)
    fkl, _ = O.divergence(s, t, 0.0)
    for r in range(zs.shape[0]):
        rest = np.setdiff1d(np.arange(zs.shape[1]), sel[r])
        pt, qt = np.exp(lp[r, rest]), np.exp(lq[r, rest])
        Pt, Qt = pt.sum(), qt.sum()
        cond_tail = float(np.sum((pt / Pt) * (np.log(pt / Pt) - np.log(qt / Qt))))
        P = out["p_mass"][r]
        assert abs(out["binary"][r] + P * out["cond"][r] + (1 - P) * cond_tail - fkl[r]) < 1e-12
        pb = np.append(np.exp(lp[r, sel[r]]), Pt)
        qb = np.append(np.exp(lq[r, sel[r]]), Qt)
        bucket = float(np.sum(pb * np.log(pb / qb)))
        assert abs(bucket - (out["binary"][r] + P * out["cond"][r])) < 1e-12


def test_ce_anchor_is_forward_kl_against_a_one_hot_teacher():
    zs, zt = _case(7, V=64, N=6)
    labels = np.array([0, 5, 63, -100, 17, 17])
    sel = O.topk_order(zt, 8)
    out = O.topk_three_terms(zs, zt, sel, 1.0, labels=labels)
    for r, y in enumerate(labels):
        if y == -100:
            assert math.isnan(out["ce"][r])
            continue
        onehot = np.full(64, -1e9)
        onehot[y] = 0.0
        f, _ = O.divergence(zs[r:r + 1], onehot[None], 0.0)
        assert abs(out["ce"][r] - f[0]) < 1e-9


def test_kd_topk_fwd_end_to_end_small():
    g = np.random.default_rng(8)
    N, V, ds, dt = 3, 97, 8, 16
    h_s, h_t = g.normal(size=(N, ds)), g.normal(size=(N, dt))
    W_s, W_t = g.normal(0, 1, (V, ds)), g.normal(0, 1, (V, dt))
    out = O.kd_topk_fwd(h_s, W_s, h_t, W_t, 10, 1.0, labels=np.array([1, 2, 3]), with_bound=True)
    zt = h_t @ W_t.T
    for r in range(N):
        keys = [float(O.bf16_round(np.array([v]))[0]) for v in zt[r]]
        assert out["idx"][r].tolist() == brute.topk_row(keys, 10)
    assert out["zt_bound"].shape == (N, V) and np.all(out["zt_bound"] > 0)


# --------------------------------------------------------------------------- rank-r teacher
@pytest.mark.parametrize("method", ("svd", "gram"))
def test_svd_teacher_pins(method):
    g = np.random.default_rng(9)
    V, d, N, r = 300, 24, 5, 8
    W = g.normal(0, 1, (V, d)) * (1.0 + np.arange(d))  # distinct singular values
    h = g.normal(0, 1, (N, d))
    h_r, W_r, S = O.svd_teacher(h, W, r, method=method)
    assert np.allclose(W_r.T @ W_r, np.eye(r), atol=1e-9)  # orthonormal columns
    approx = W_r @ (W_r.T @ W)  # best rank-r approximation of W
    assert abs(np.linalg.norm(W - approx) ** 2 - np.sum(S[r:] ** 2)) < 1e-6 * np.sum(S ** 2)  # Eckart-Young
    z = h @ W.T
    assert np.allclose(h_r @ W_r.T, z @ W_r @ W_r.T, atol=1e-8)  # projected teacher logits
    h_f, W_f, _ = O.svd_teacher(h, W, d, method=method)
    assert np.allclose(h_f @ W_f.T, z, atol=1e-8)  # full rank reproduces the logits


# --------------------------------------------------------------------------- top-k gradient
@pytest.mark.parametrize("tau", (1.0, 1.7))
def test_topk_gradient_matches_finite_differences(tau):
    g = np.random.default_rng(21)
    N, V, k = 4, 60, 8
    zs, zt = g.normal(0, 2, (N, V)), g.normal(0, 2, (N, V))
    sel = O.topk_order(zt, k)
    labels = np.array([3, -100, 59, 17])
    wb, wc, we = g.uniform(-1, 2, N), g.uniform(-1, 2, N), g.uniform(-1, 2, N)
    an = O.topk_grad_student_logits(zs, zt, sel, tau, labels, wb, wc, we)
    for r in range(N):
        fd = brute.fd_grad_topk_row(zs[r].tolist(), zt[r].tolist(), sel[r].tolist(), tau, int(labels[r]),
                                    wb[r], wc[r], we[r])
        assert np.allclose(an[r], fd, atol=1e-8, rtol=1e-6), np.abs(an[r] - np.array(fd)).max()
    # each term alone, and no labels: the CE part drops out
    only_b = O.topk_grad_student_logits(zs, zt, sel, tau, None, wb, None, None)
    only_c = O.topk_grad_student_logits(zs, zt, sel, tau, None, None, wc, None)
    only_e = O.topk_grad_student_logits(zs, zt, sel, tau, labels, None, None, we)
    assert np.allclose(only_b + only_c + only_e, an, rtol=1e-12, atol=1e-15)
    # every term is a function of a softmax (or of log-masses): each row of the gradient sums to zero
    assert np.all(np.abs(an.sum(-1)) < 1e-12)


def test_topk_gradient_full_set_has_no_binary_part():
    zs, zt = _case(5, V=40)
    sel = O.topk_order(zt, 40)
    wb = np.ones(zs.shape[0])
    assert np.all(O.topk_grad_student_logits(zs, zt, sel, 1.3, None, wb, None, None) == 0.0)
    # with the full set the conditional KL is forward KL, whose gradient is q - p
    wc = np.ones(zs.shape[0])
    gc = O.topk_grad_student_logits(zs, zt, sel, 1.0, None, None, wc, None)
    assert np.allclose(gc, O.grad_student_logits(zs, zt, 0.0), atol=1e-14)


def test_kd_topk_bwd_is_logit_gradient_times_unembedding():
    g = np.random.default_rng(22)
    N, V, ds, dt, k = 3, 300, 16, 12, 8
    h_s, h_t = g.normal(size=(N, ds)), g.normal(size=(N, dt))
    W_s, W_t = g.normal(0, 0.5, (V, ds)), g.normal(0, 0.5, (V, dt))
    wb, wc, we = g.uniform(0, 1, N), g.uniform(0, 1, N), g.uniform(0, 1, N)
    labels = np.array([5, 299, -100])
    dh = O.kd_topk_bwd(h_s, W_s, h_t, W_t, k, 1.5, labels, wb, wc, we)
    # straight-through reading: the gradient of the terms at the bf16-rounded
    # logits, mapped back through z_s = h_s W_s^T; compared on rows one by one
    for r in range(N):
        zs = O.bf16_round(h_s[r] @ W_s.T)
        zt = O.bf16_round(h_t[r] @ W_t.T)
        sel = O.topk_order(zt[None], k)
        fd = np.array(brute.fd_grad_topk_row(zs.tolist(), zt.tolist(), sel[0].tolist(), 1.5, int(labels[r]),
                                             wb[r], wc[r], we[r]))
        assert np.allclose(dh[r], fd @ W_s, rtol=1e-5, atol=1e-8)
