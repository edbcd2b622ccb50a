"""Pins for the fp64 oracle's divergences and gradients (CPU only).

Each test pins the oracle to something other than itself: hand closed forms,
limits, invariants of the definitions, an independent pure-Python brute force
and central finite differences. Sources: White-box OPD (section 2.3 beta table,
temperature, log domain; section 4.1 gradient blow-up; section 6 test plan),
Nitrobrew notes ("仓库实现" gradient forms), and the study card on adaptive KL
(forward and reverse KL share the optimum p = q).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from oracle import kd_oracle as O

HERE = os.path.dirname(__file__)
BETAS = (0.0, 0.25, 0.5, 0.9, 1.0)


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- log-softmax
def test_log_softmax_normalises_and_is_shift_invariant():
    x = rng(0).normal(0, 5, size=(7, 301))
    ls = O.log_softmax(x)
    assert np.allclose(np.exp(ls).sum(-1), 1.0, atol=1e-14)
    assert np.allclose(O.log_softmax(x + 123.25), ls, atol=1e-12)
    # large logits do not overflow (max subtraction)
    big = O.lse(np.array([[1000.0, 1000.0]]))
    assert abs(big[0] - (1000.0 + math.log(2.0))) < 1e-12


# --------------------------------------------------------------------------- hand cases
def _frac_list(xs):
    return np.array([float(Fraction(x)) for x in xs])


def test_v5_hand_cases():
    with open(os.path.join(HERE, "golden", "v5_hand_cases.json")) as f:
        spec = json.load(f)
    env = {"log": math.log}
    for case in spec["cases"]:
        p = _frac_list(case["p"])
        q = _frac_list(case["q"])
        t = np.log(p)[None] + 0.37  # any shift: logits are log-probabilities up to a constant
        s = np.log(q)[None] - 1.91
        for beta, expr in case["expected"].items():
            want = eval(expr, {"__builtins__": {}}, env)  # noqa: S307 - fixture expressions in ln2/ln3/ln5
            got, _ = O.divergence(s, t, float(beta))
            assert abs(got[0] - want) < 1e-13, (case["name"], beta, got[0], want)


def test_swapped_dyadic_general_beta_closed_form():
    # p = (1/2, 1/4, r), q = (1/4, 1/2, r): only the first two entries differ, so
    # m1 = (1+b)/4, m2 = (2-b)/4 and the divergence reduces by hand to
    #   b [1/2 ln(2/(1+b)) + 1/4 ln(1/(2-b))] + (1-b) [1/4 ln(1/(1+b)) + 1/2 ln(2/(2-b))]
    p = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
    q = np.array([0.25, 0.5, 0.125, 0.0625, 0.0625])
    for b in (0.1, 0.3, 0.5, 0.77):
        want = b * (0.5 * math.log(2 / (1 + b)) + 0.25 * math.log(1 / (2 - b))) + \
            (1 - b) * (0.25 * math.log(1 / (1 + b)) + 0.5 * math.log(2 / (2 - b)))
        got, _ = O.divergence(np.log(q)[None], np.log(p)[None], b)
        assert abs(got[0] - want) < 1e-14


# --------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("tau", (1.0, 2.0))
def test_vectorised_matches_pure_python(beta, tau):
    g = rng(11)
    N, V, ds, dt = 3, 13, 6, 5
    h_s, h_t = g.normal(size=(N, ds)), g.normal(size=(N, dt))
    W_s, W_t = g.normal(size=(V, ds)), g.normal(size=(V, dt))
    want = brute.loss_rows(h_s.tolist(), W_s.tolist(), h_t.tolist(), W_t.tolist(), beta, tau)
    got = O.kd_fwd(h_s, W_s, h_t, W_t, beta, tau)["loss"]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("beta", BETAS)
def test_zero_at_equal_distributions(beta):
    # forward and reverse KL (and the mixture) share the optimum p = q
    s = rng(2).normal(0, 3, size=(5, 1000))
    loss, _ = O.divergence(s, s + 4.0, beta)  # shift: same distribution
    assert np.all(np.abs(loss) < 1e-12)


@pytest.mark.parametrize("beta", BETAS)
def test_nonnegative(beta):
    g = rng(3)
    s = g.normal(0, 3, size=(64, 200))
    t = g.normal(0, 3, size=(64, 200))
    loss, _ = O.divergence(s, t, beta)
    assert np.all(loss > 0)


def test_uniform_student_vs_one_raised_teacher_closed_form():
    # student logits all equal (uniform q); teacher logit 0 raised by D, others 0.
    # p0 = e^(D/tau) / (e^(D/tau) + V - 1).  FKL = log V + sum p log p;
    # RKL = -log V - (1/V) sum log p = -log V - D/(tau V) + log Z.
    V = 50
    for D, tau in ((3.0, 1.0), (3.0, 2.0), (10.0, 0.5)):
        zt = np.zeros((1, V))
        zt[0, 0] = D
        zs = np.zeros((1, V))
        Z = math.exp(D / tau) + V - 1
        p0, pr = math.exp(D / tau) / Z, 1.0 / Z
        fkl = math.log(V) + p0 * math.log(p0) + (V - 1) * pr * math.log(pr)
        rkl = -math.log(V) - D / (tau * V) + math.log(Z)
        got_f, _ = O.divergence(zs / tau, zt / tau, 0.0)
        got_r, _ = O.divergence(zs / tau, zt / tau, 1.0)
        assert abs(got_f[0] - fkl) < 1e-13 and abs(got_r[0] - rkl) < 1e-13
        # dividing after the softmax would not even normalise: softmax(z)/tau sums to 1/tau
        assert abs(np.exp(O.log_softmax(zt / tau)).sum() - 1.0) < 1e-14


def test_one_raised_teacher_limits():
    V = 20
    zs = np.zeros((1, V))
    for D, expect_f in ((60.0, math.log(V)),):
        zt = np.zeros((1, V))
        zt[0, 0] = D
        f, _ = O.divergence(zs, zt, 0.0)
        r, _ = O.divergence(zs, zt, 1.0)
        assert abs(f[0] - expect_f) < 1e-9  # FKL -> log V
        assert r[0] > 0.9 * D  # RKL grows without bound (~ D (V-1)/V)


def test_high_temperature_sends_losses_to_zero():
    g = rng(4)
    zs, zt = g.normal(0, 3, (4, 300)), g.normal(0, 3, (4, 300))
    for beta in BETAS:
        prev = None
        for tau in (1.0, 10.0, 100.0, 1e4):
            loss, _ = O.divergence(zs / tau, zt / tau, beta)
            m = float(np.max(loss))
            if prev is not None:
                assert m < prev
            prev = m
        assert prev < 1e-6


def test_beta_endpoint_limits():
    # JSD_b / b -> KL(p||q) as b -> 0+;  JSD_b / (1-b) -> KL(q||p) as b -> 1-
    g = rng(5)
    s, t = g.normal(0, 2, (3, 100)), g.normal(0, 2, (3, 100))
    fkl, _ = O.divergence(s, t, 0.0)
    rkl, _ = O.divergence(s, t, 1.0)
    b = 1e-6
    lo, _ = O.divergence(s, t, b)
    hi, _ = O.divergence(s, t, 1.0 - b)
    assert np.allclose(lo / b, fkl, rtol=1e-4)
    assert np.allclose(hi / b, rkl, rtol=1e-4)


def test_beta_swap_symmetry():
    g = rng(6)
    s, t = g.normal(0, 2, (4, 77)), g.normal(0, 2, (4, 77))
    for b in (0.0, 0.2, 0.5, 0.8, 1.0):
        a, _ = O.divergence(s, t, b)
        c, _ = O.divergence(t, s, 1.0 - b)
        assert np.allclose(a, c, rtol=1e-12, atol=1e-14)


def test_mixture_entropy_bound():
    # JSD_b <= h(b) = -b log b - (1-b) log(1-b), approached for disjoint one-hots
    g = rng(7)
    s, t = g.normal(0, 3, (16, 40)), g.normal(0, 3, (16, 40))
    for b in (0.1, 0.5, 0.9):
        hb = -b * math.log(b) - (1 - b) * math.log(1 - b)
        loss, _ = O.divergence(s, t, b)
        assert np.all(loss <= hb)
        zs = np.full((1, 8), -200.0)
        zt = np.full((1, 8), -200.0)
        zs[0, 0] = 200.0
        zt[0, 1] = 200.0
        near, _ = O.divergence(zs, zt, b)
        assert abs(near[0] - hb) < 1e-9


def test_direction_confident_vs_diffuse():
    # White-box OPD section 6: the ordering of FKL/RKL flips between a
    # confident teacher with a diffuse student and the converse.
    V = 100
    peaked = np.zeros((1, V))
    peaked[0, 0] = 8.0
    flat = np.zeros((1, V))
    f1, _ = O.divergence(flat, peaked, 0.0)  # teacher confident, student diffuse
    r1, _ = O.divergence(flat, peaked, 1.0)
    f2, _ = O.divergence(peaked, flat, 0.0)  # teacher diffuse, student confident
    r2, _ = O.divergence(peaked, flat, 1.0)
    # confident teacher, diffuse student: forward KL (mode-covering) is the larger,
    # it charges the student for the teacher's peak it fails to cover
    assert f1[0] > r1[0]
    # diffuse teacher, confident student: reverse KL is the larger, it charges the
    # student's peak where the teacher has little mass
    assert r2[0] > f2[0]
    assert abs(f1[0] - r2[0]) < 1e-12 and abs(r1[0] - f2[0]) < 1e-12


# --------------------------------------------------------------------------- gradients
@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("tau", (1.0, 2.0))
def test_gradient_matches_finite_differences(beta, tau):
    g = rng(8)
    N, V, ds, dt = 2, 16, 8, 6
    h_s, h_t = g.normal(size=(N, ds)), g.normal(size=(N, dt))
    W_s, W_t = g.normal(0, 0.7, size=(V, ds)), g.normal(0, 0.7, size=(V, dt))
    fd = np.array(brute.fd_grad_h(h_s.tolist(), W_s.tolist(), h_t.tolist(), W_t.tolist(), beta, tau))
    an = O.kd_bwd(h_s, W_s, h_t, W_t, beta, tau)
    assert np.allclose(an, fd, atol=2e-9, rtol=1e-7), np.abs(an - fd).max()
    # grad_loss scales rows
    gl = np.array([0.5, -2.0])
    an2 = O.kd_bwd(h_s, W_s, h_t, W_t, beta, tau, grad_loss=gl)
    assert np.allclose(an2, an * gl[:, None], rtol=1e-13, atol=1e-15)
    # the one-pass forward + backward: the same gradient against finite
    # differences and the same loss against the pure-Python loop
    fwd, dh = O.kd_fwd_bwd(h_s, W_s, h_t, W_t, beta, tau, grad_loss=gl)
    assert np.allclose(dh, fd * gl[:, None], atol=4e-9, rtol=1e-7)
    want = brute.loss_rows(h_s.tolist(), W_s.tolist(), h_t.tolist(), W_t.tolist(), beta, tau)
    assert np.allclose(fwd["loss"], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("tau", (1.0, 2.0))
def test_weight_gradient_matches_finite_differences(beta, tau):
    g = rng(18)
    N, V, ds, dt = 3, 7, 5, 4
    h_s, h_t = g.normal(size=(N, ds)), g.normal(size=(N, dt))
    W_s, W_t = g.normal(0, 0.7, size=(V, ds)), g.normal(0, 0.7, size=(V, dt))
    fd = np.array(brute.fd_grad_W(h_s.tolist(), W_s.tolist(), h_t.tolist(), W_t.tolist(), beta, tau))
    an = O.kd_bwd_w(h_s, W_s, h_t, W_t, beta, tau)
    assert an.shape == (V, ds)
    assert np.allclose(an, fd, atol=2e-9, rtol=1e-7), np.abs(an - fd).max()
    # grad_loss weights the tokens' contributions
    gl = np.array([0.5, -2.0, 1.5])
    an2 = O.kd_bwd_w(h_s, W_s, h_t, W_t, beta, tau, grad_loss=gl)
    parts = [O.kd_bwd_w(h_s[i:i + 1], W_s, h_t[i:i + 1], W_t, beta, tau) for i in range(N)]
    assert np.allclose(an2, sum(w * p for w, p in zip(gl, parts)), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("beta", BETAS)
def test_weight_and_hidden_gradients_agree(beta):
    # both are the two sides of z_s = h_s W_s^T: sum_v W_s[v].dW_s[v] equals
    # sum_n h_s[n].dh_s[n] (each is sum_{n,v} dL/dz_s[n,v] z_s[n,v]), and the
    # rows of dW_s sum to zero because each token's dL/ds sums to zero
    g = rng(19)
    N, V, ds, dt = 5, 40, 6, 9
    h_s, h_t = g.normal(size=(N, ds)), g.normal(size=(N, dt))
    W_s, W_t = g.normal(0, 0.8, size=(V, ds)), g.normal(0, 0.8, size=(V, dt))
    dW = O.kd_bwd_w(h_s, W_s, h_t, W_t, beta, 1.5)
    dh = O.kd_bwd(h_s, W_s, h_t, W_t, beta, 1.5)
    assert abs(np.sum(W_s * dW) - np.sum(h_s * dh)) < 1e-12 * (1 + np.abs(W_s * dW).sum())
    assert np.all(np.abs(dW.sum(0)) < 1e-13)


@pytest.mark.parametrize("beta", BETAS)
def test_gradient_sums_to_zero(beta):
    g = rng(9)
    s, t = g.normal(0, 3, (6, 500)), g.normal(0, 3, (6, 500))
    gr = O.grad_student_logits(s, t, beta)
    assert np.all(np.abs(gr.sum(-1)) < 1e-14)


def test_forward_kl_gradient_is_student_minus_teacher():
    g = rng(10)
    s, t = g.normal(0, 3, (3, 64)), g.normal(0, 3, (3, 64))
    gr = O.grad_student_logits(s, t, 0.0)
    q = np.exp(s - O.lse(s)[:, None])
    p = np.exp(t - O.lse(t)[:, None])
    assert np.allclose(gr, q - p, atol=1e-15)


def test_reverse_kl_gradient_blows_up_as_teacher_prob_vanishes():
    # White-box OPD 4.1 / 6: fix the student; drive the teacher's probability of
    # the student's favourite token from 1e-1 to 1e-6; the reverse-KL gradient
    # norm grows monotonically (the log-ratio term).
    V = 32
    s = np.zeros((1, V))
    s[0, 0] = 3.0
    norms = []
    for pt in (1e-1, 1e-2, 1e-3, 1e-4, 1e-5, 1e-6):
        t = np.zeros((1, V))
        # choose teacher logit 0 so that p_0 = pt given the other 31 logits are 0
        t[0, 0] = math.log(pt * (V - 1) / (1 - pt))
        assert abs(math.exp(O.log_softmax(t)[0, 0]) - pt) < 1e-12
        norms.append(float(np.linalg.norm(O.grad_student_logits(s, t, 1.0))))
    assert all(b > a for a, b in zip(norms, norms[1:]))
    assert norms[-1] > 5 * norms[0]
    # forward KL's gradient stays bounded (|q - p| <= 1 elementwise)
    fk = [float(np.linalg.norm(O.grad_student_logits(s, np.log([[pt] + [(1 - pt) / (V - 1)] * (V - 1)]), 0.0)))
          for pt in (1e-1, 1e-6)]
    assert max(fk) < math.sqrt(2)


def test_plain_dtype_decoding():
    # bf16 bit patterns decode exactly: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E20 = 0.15625
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x0000, 0x8000], dtype=np.uint16)
    assert O.as_f64(bits).tolist() == [1.0, -2.0, 0.15625, 0.0, -0.0]
