"""Pins for the oracle's tail-bucket divergence (CPU only).

Source: White-box OPD, section 2.4 (divergence on the top-k support plus one
tail bucket holding the rest of the mass; the support is the teacher's top-k,
the student's or their union depending on beta; with one kept entry, the
sampled token plus the teacher's top-1) and section 2.3 (the beta table).
"""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import kd_oracle as O

T, S, L = O.SUPPORT_TEACHER, O.SUPPORT_STUDENT, O.SUPPORT_LABEL
BETAS = (0.0, 0.3, 0.5, 1.0)


def _case(seed, V=40, N=4, scale=2.0):
    g = np.random.default_rng(seed)
    zs = O.bf16_round(g.normal(0, scale, (N, V)))
    zt = O.bf16_round(0.6 * zs + g.normal(0, scale, (N, V)))
    return zs, zt


def test_default_support_rule():
    assert O.tail_default_support(1, 0.5, True) == T | L
    assert O.tail_default_support(1, 1.0, False) == T
    assert O.tail_default_support(8, 0.0, True) == T
    assert O.tail_default_support(8, 1.0, True) == S
    assert O.tail_default_support(8, 0.25, False) == T | S
    assert O.tail_support_size(8, T | S) == 16
    assert O.tail_support_size(1, T | L) == 2
    assert O.tail_support_size(5, S) == 5


def test_support_order_dedup_and_label():
    zs, zt = _case(1, V=30, N=6)
    zs = np.round(zs)  # ties, so the index rule matters
    labels = np.array([0, 3, -100, 29, 7, 7])
    k = 6
    for sup in (T, S, T | S, T | L, S | L, T | S | L):
        got = O.tail_support(zs, zt, k, sup, labels)
        assert got.shape == (6, O.tail_support_size(k, sup))
        for r in range(6):
            want = []
            if sup & T:
                want += brute.topk_row(zt[r].tolist(), k)
            if sup & S:
                want += [v for v in brute.topk_row(zs[r].tolist(), k) if v not in want]
            if sup & L and labels[r] != -100 and labels[r] not in want:
                want.append(int(labels[r]))
            row = got[r].tolist()
            assert row[:len(want)] == want
            assert all(v == -1 for v in row[len(want):])
    with pytest.raises(ValueError):
        O.tail_support(zs, zt, k, L, labels)


@pytest.mark.parametrize("tau", (1.0, 2.0))
@pytest.mark.parametrize("beta", BETAS)
def test_tail_loss_matches_brute_force(beta, tau):
    zs, zt = _case(2)
    labels = np.array([5, -100, 39, 0])
    for k, sup in ((1, T | L), (5, T), (5, S), (5, T | S), (3, T | S | L)):
        idx = O.tail_support(zs, zt, k, sup, labels)
        out = O.tail_divergence(zs, zt, idx, beta, tau)
        for r in range(zs.shape[0]):
            row = [v for v in idx[r].tolist() if v >= 0]
            want = brute.tail_loss_row(zs[r].tolist(), zt[r].tolist(), row, beta, tau)
            assert abs(out["loss"][r] - want) < 1e-12 * max(1.0, abs(want)), (k, sup, r)


def test_hand_case_closed_forms():
    # teacher p = (1/2, 1/4, 1/8, 1/8), student uniform; both top-1 supports
    # are entry 0 (the student's by the index rule), so the buckets are
    # p = (1/2, 1/2) and q = (1/4, 3/4).
    zt = np.log(np.array([[0.5, 0.25, 0.125, 0.125]]))
    zs = np.zeros((1, 4))
    ln2, ln3, ln5 = math.log(2), math.log(3), math.log(5)
    want = {
        0.0: 0.5 * (2 * ln2 - ln3),                       # 1/2 ln 2 + 1/2 ln(2/3)
        1.0: 0.75 * ln3 - ln2,                            # 1/4 ln(1/2) + 3/4 ln(3/2)
        # m = (3/8, 5/8): 1/2 [1/2 ln(4/3) + 1/2 ln(4/5)] + 1/2 [1/4 ln(2/3) + 3/4 ln(6/5)]
        0.5: 0.25 * (4 * ln2 - ln3 - ln5) + 0.125 * (ln2 - ln3) + 0.375 * (ln2 + ln3 - ln5),
    }
    for beta, w in want.items():
        sup = O.tail_support(zs, zt, 1, O.tail_default_support(2, beta, False), None)
        assert sup[0, 0] == 0
        got = O.tail_divergence(zs, zt, sup[:, :1], beta, 1.0)["loss"][0]
        assert abs(got - w) < 1e-14, (beta, got, w)


@pytest.mark.parametrize("beta", BETAS)
def test_whole_vocabulary_support_is_the_full_divergence(beta):
    zs, zt = _case(3, V=25)
    for sup in (T, S):
        idx = O.tail_support(zs, zt, 25, sup)
        out = O.tail_divergence(zs, zt, idx, beta, 1.5)
        full, aux = O.divergence(zs / 1.5, zt / 1.5, beta)
        assert np.allclose(out["loss"], full, rtol=1e-12, atol=1e-15)
        assert np.allclose(out["aux"], aux, rtol=1e-12, atol=1e-15)
        assert np.allclose(out["p_mass"], 1.0) and np.allclose(out["q_mass"], 1.0)


@pytest.mark.parametrize("beta", BETAS)
def test_refining_the_support_never_lowers_the_divergence(beta):
    # merging outcomes into one bucket can only lose information (data
    # processing inequality of f-divergences, the beta-JSD included)
    zs, zt = _case(4, V=60, N=5)
    full, _ = O.divergence(zs, zt, beta)
    prev = np.zeros(zs.shape[0])
    for k in (1, 2, 4, 8, 16, 32, 59):
        out = O.tail_divergence(zs, zt, O.tail_support(zs, zt, k, T), beta, 1.0)["loss"]
        assert np.all(out >= prev - 1e-13) and np.all(out <= full + 1e-13)
        prev = out
    union = O.tail_divergence(zs, zt, O.tail_support(zs, zt, 8, T | S), beta, 1.0)["loss"]
    teach = O.tail_divergence(zs, zt, O.tail_support(zs, zt, 8, T), beta, 1.0)["loss"]
    assert np.all(union >= teach - 1e-13)


@pytest.mark.parametrize("tau", (1.0, 2.5))
def test_forward_kl_on_teacher_buckets_is_binary_plus_weighted_cond(tau):
    # chain rule of KL over {top-k, rest}: the (k+1)-bucket forward KL equals
    # the three-term split's binary KL + P * conditional KL
    zs, zt = _case(5, V=80, N=5)
    for k in (1, 7, 30):
        sel = O.topk_order(zt, k)
        three = O.topk_three_terms(zs, zt, sel, tau)
        tail = O.tail_divergence(zs, zt, O.tail_support(zs, zt, k, T), 0.0, tau)
        assert np.allclose(tail["loss"], three["binary"] + three["p_mass"] * three["cond"], rtol=1e-11, atol=1e-14)
        assert np.allclose(tail["p_mass"], three["p_mass"]) and np.allclose(tail["q_mass"], three["q_mass"])


@pytest.mark.parametrize("tau", (1.0, 1.8))
@pytest.mark.parametrize("beta", BETAS)
def test_tail_gradient_matches_finite_differences(beta, tau):
    zs, zt = _case(6, V=12, N=3, scale=1.5)
    labels = np.array([11, 2, -100])
    for k, sup in ((1, T | L), (3, T), (3, S), (3, T | S), (12, T)):
        idx = O.tail_support(zs, zt, k, sup, labels)
        g = O.tail_grad_student_logits(zs, zt, idx, beta, tau)
        for r in range(zs.shape[0]):
            row = [v for v in idx[r].tolist() if v >= 0]
            fd = brute.fd_grad_tail_row(zs[r].tolist(), zt[r].tolist(), row, beta, tau)
            assert np.allclose(g[r], fd, rtol=1e-6, atol=1e-8), (k, sup, r)
        assert np.allclose(g.sum(axis=1), 0.0, atol=1e-13)


@pytest.mark.parametrize("beta", BETAS)
def test_whole_vocabulary_gradient_is_the_full_gradient(beta):
    zs, zt = _case(7, V=30)
    idx = O.tail_support(zs, zt, 30, S)
    g = O.tail_grad_student_logits(zs, zt, idx, beta, 2.0)
    assert np.allclose(g, O.grad_student_logits(zs / 2.0, zt / 2.0, beta) / 2.0, rtol=1e-10, atol=1e-14)


def test_forward_kl_gradient_inside_the_support_is_q_minus_p():
    zs, zt = _case(8, V=50)
    idx = O.tail_support(zs, zt, 6, T)
    g = O.tail_grad_student_logits(zs, zt, idx, 0.0, 1.0)
    q = np.exp(O.log_softmax(zs))
    p = np.exp(O.log_softmax(zt))
    for r in range(zs.shape[0]):
        inside = idx[r]
        assert np.allclose(g[r, inside], q[r, inside] - p[r, inside], rtol=1e-12, atol=1e-15)


def test_kd_tail_fwd_and_bwd_from_hidden_states():
    g = np.random.default_rng(9)
    N, V, d = 3, 20, 8
    h_s = g.normal(0, 1, (N, d))
    h_t = g.normal(0, 1, (N, d))
    W_s = g.normal(0, 0.7, (V, d))
    W_t = g.normal(0, 0.7, (V, d))
    labels = np.array([4, -100, 19])
    for k, beta in ((1, 0.5), (4, 0.0), (4, 1.0), (4, 0.5)):
        out = O.kd_tail_fwd(h_s, W_s, h_t, W_t, k, beta, 1.3, labels=labels)
        zs = [[O.bf16_round(np.array([brute.dot(h_s[n], w)]))[0] for w in W_s] for n in range(N)]
        zt = [[O.bf16_round(np.array([brute.dot(h_t[n], w)]))[0] for w in W_t] for n in range(N)]
        dh = O.kd_tail_bwd(h_s, W_s, h_t, W_t, k, beta, 1.3, labels=labels, grad_loss=np.array([1.0, 0.5, 2.0]))
        for n in range(N):
            row = [v for v in out["sup"][n].tolist() if v >= 0]
            assert out["loss"][n] == pytest.approx(brute.tail_loss_row(zs[n], zt[n], row, beta, 1.3), rel=1e-12)
            assert np.array_equal(out["val_s"][n, :len(row)], np.array(zs[n])[row])
            assert np.array_equal(out["val_t"][n, :len(row)], np.array(zt[n])[row])
            gz = brute.fd_grad_tail_row(zs[n], zt[n], row, beta, 1.3)
            want = [math.fsum(gz[v] * W_s[v][i] for v in range(V)) * [1.0, 0.5, 2.0][n] for i in range(d)]
            assert np.allclose(dh[n], want, rtol=1e-6, atol=1e-8)


def test_gpu_acceptance_check_accepts_the_oracle_and_rejects_planted_mistakes():
    # the parity helper used by the GPU tests, fed the oracle's own output
    torch = pytest.importorskip("torch")
    import kdsynth
    from tests.helpers import check_tail_rows
    N, V = 12, 300
    arrays = kdsynth.small_case(41, N, V, 16, 16)
    labels = kdsynth.uniform_labels(8, N, V, ignore_frac=0.2)
    for k, beta, sup in ((1, 0.5, T | L), (8, 0.5, T | S), (8, 1.0, S), (6, 0.0, T | S | L)):
        ref = O.kd_tail_fwd(*arrays, k, beta, 1.5, support=sup, labels=labels)
        out = dict(sup_idx=torch.from_numpy(ref["sup"].astype(np.int32)),
                   sup_t=torch.from_numpy(ref["val_t"].astype(np.float32)),
                   sup_s=torch.from_numpy(ref["val_s"].astype(np.float32)),
                   **{f: torch.from_numpy(ref[f].astype(np.float32))
                      for f in ("loss", "p_mass", "q_mass", "lse_s", "lse_t")})
        exact, flagged = check_tail_rows(out, *arrays, np.arange(N), k, beta, 1.5, sup, labels)
        assert exact == N and flagged == 0
        bad = dict(out, loss=out["loss"] * 1.01)
        with pytest.raises(AssertionError):
            check_tail_rows(bad, *arrays, np.arange(N), k, beta, 1.5, sup, labels)
        if k > 1:  # two ranked entries exchanged
            swapped = out["sup_idx"].clone()
            swapped[:, [0, 1]] = swapped[:, [1, 0]]
            with pytest.raises(AssertionError):
                check_tail_rows(dict(out, sup_idx=swapped), *arrays, np.arange(N), k, beta, 1.5, sup, labels)
    # a loss without its tail bucket is rejected
    ref = O.kd_tail_fwd(*arrays, 8, 0.0, 1.0, support=T)
    s = O.bf16_round(O.logits(arrays[0], arrays[1]))
    t = O.bf16_round(O.logits(arrays[2], arrays[3]))
    lq, lp = O.log_softmax(s), O.log_softmax(t)
    rows = np.arange(N)[:, None]
    no_tail = np.sum(np.exp(lp[rows, ref["sup"]]) * (lp[rows, ref["sup"]] - lq[rows, ref["sup"]]), axis=1)
    out = dict(sup_idx=torch.from_numpy(ref["sup"].astype(np.int32)),
               sup_t=torch.from_numpy(ref["val_t"].astype(np.float32)),
               sup_s=torch.from_numpy(ref["val_s"].astype(np.float32)),
               loss=torch.from_numpy(no_tail.astype(np.float32)),
               **{f: torch.from_numpy(ref[f].astype(np.float32)) for f in ("p_mass", "q_mass", "lse_s", "lse_t")})
    with pytest.raises(AssertionError):
        check_tail_rows(out, *arrays, np.arange(N), 8, 0.0, 1.0, T)
