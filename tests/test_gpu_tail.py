"""GPU parity of kd_tail_fwd / kd_tail_bwd (beta-divergence over a top-k
support plus a tail bucket, bf16 logits) against the fp64 oracle, through the
C ABI. The support is compared entry for entry; logits within the fp32
accumulation bound of a bf16 rounding midpoint may round either way
(tests/helpers.check_tail_rows). The gradient is compared with the oracle's
gradient for the support the GPU picked (per row cosine >= 0.9999,
max|d| / max|ref| <= 2e-2)."""
import numpy as np
import pytest

import kdsynth
from oracle import kd_oracle as O
from tests.helpers import assert_close, assert_grad_rows, check_tail_rows, exact_shifted_case, to_dev, workload

pytestmark = pytest.mark.gpu

T, S, L = O.SUPPORT_TEACHER, O.SUPPORT_STUDENT, O.SUPPORT_LABEL


def _kd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_chunked_kl_amd as kd
    kd.load_library()
    return kd, torch


def _case(kd, torch, arrays, k, beta, tau, support, labels, rows, grad_seed=None, chunk_V=256):
    """Forward on every token; acceptance on ``rows``; with ``grad_seed`` the
    backward too, weighted by seeded per-token factors."""
    h_s, W_s, h_t, W_t = arrays
    N = h_s.shape[0]
    dev = [to_dev(x) for x in arrays]
    lab = None if labels is None else torch.from_numpy(labels.astype(np.int32)).cuda()
    out = kd.kd_tail_fwd(*dev, k, beta, tau, support, labels=lab)
    torch.cuda.synchronize()
    exact, flagged = check_tail_rows(out, h_s, W_s, h_t, W_t, rows, k, beta, tau, support, labels)
    print(f"  exact {exact} flagged {flagged}", flush=True)
    if grad_seed is not None:
        w = np.random.default_rng(grad_seed).uniform(-0.5, 1.5, N)
        dh = kd.kd_tail_bwd(dev[0], dev[1], out, k, beta, tau, support,
                            grad_loss=torch.from_numpy(w.astype(np.float32)).cuda(), chunk_V=chunk_V)
        torch.cuda.synchronize()
        sup = out["sup_idx"].cpu().numpy()
        ref = []
        for b0 in range(0, len(rows), 256):  # host memory: 256 rows of full-vocabulary logits at a time
            rb = rows[b0:b0 + 256]
            ref.append(O.kd_tail_bwd(h_s[rb], W_s, h_t[rb], W_t, k, beta, tau, grad_loss=w[rb], sup=sup[rb]))
        assert_grad_rows(dh.cpu().numpy()[rows], np.concatenate(ref), name="tail dh_s")
    return out, exact


CASES = [(1, 0.5, T | L), (8, 0.0, T), (8, 1.0, S), (8, 0.5, T | S), (64, 0.3, T | S | L), (5, 1.0, S | L)]


@pytest.mark.parametrize("beta,support", [(0.5, T | S), (1.0, S)])
def test_tail_bwd_logits_past_exp_range(beta, support):
    """Student logits near 100 (every logit raised by the same amount: the
    divergence is unchanged, exp of a logit overflows fp32): forward and
    backward against the oracle on every row."""
    kd, torch = _kd()
    N, V = 64, 3000
    arrays = exact_shifted_case(29, N, V, 16)
    print(f"tail shifted student logits N={N} V={V} beta={beta} support={support}", flush=True)
    _case(kd, torch, arrays, 8, beta, 1.5, support, None, np.arange(N), grad_seed=36)


@pytest.mark.parametrize("teacher", [False, True])
@pytest.mark.parametrize("head", [0.0, 14.0])
@pytest.mark.parametrize("beta,support", [(0.5, T | S), (1.0, T)])
def test_tail_keeps_precision_under_a_common_offset(beta, support, head, teacher):
    """One model's logits raised by 100 (an offset the softmax ignores): loss
    and masses against the oracle to an absolute 4e-6, the precision of
    unshifted logits. With ``head`` the support holds all but a few percent
    of both masses. A bucket log-probability formed as a logit minus an fp32
    log-sum-exp near 67 (tau = 1.5) is good to only about 1e-5."""
    kd, torch = _kd()
    N, V, k, tau = 64, 3000, 8, 1.5
    arrays = exact_shifted_case(33, N, V, 16, head=head, teacher=teacher)
    who = "teacher" if teacher else "student"
    print(f"tail shifted {who} logits head={head} beta={beta} support={support} N={N} V={V}", flush=True)
    dev = [to_dev(x) for x in arrays]
    out = kd.kd_tail_fwd(*dev, k, beta, tau, support)
    torch.cuda.synchronize()
    ref = O.kd_tail_fwd(*arrays, k, beta, tau, support)
    sup = out["sup_idx"].cpu().numpy()
    for n in range(N):  # exact logits: no rounding ties, the same support
        assert sorted(sup[n][sup[n] >= 0].tolist()) == sorted(ref["sup"][n][ref["sup"][n] >= 0].tolist()), n
    for name in ("loss", "p_mass", "q_mass"):
        got = out[name].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[name]).max()
        assert err <= 4e-6, f"{name}: max abs err {err:.3g}"


@pytest.mark.parametrize("k,beta,support", CASES)
@pytest.mark.parametrize("tau", [1.0, 1.5])
def test_tail_ragged_small(k, beta, support, tau):
    kd, torch = _kd()
    N, V, ds, dt = 150, 5000, 64, 128  # 2 token tiles (ragged), 20 vocabulary tiles (ragged)
    arrays = kdsynth.small_case(41, N, V, ds, dt)
    labels = kdsynth.uniform_labels(8, N, V, ignore_frac=0.2)
    print(f"tail ragged N={N} V={V} k={k} beta={beta} support={support} tau={tau}", flush=True)
    _, exact = _case(kd, torch, arrays, k, beta, tau, support, labels, np.arange(N), grad_seed=51)
    assert exact >= 0.9 * N


def test_tail_multi_split_and_ties():
    kd, torch = _kd()
    N, V, ds, dt = 64, 150001, 32, 32  # three vocabulary splits, many bf16 ties
    arrays = kdsynth.small_case(42, N, V, ds, dt, logit_std=0.5)
    print(f"tail splits N={N} V={V}", flush=True)
    _, exact = _case(kd, torch, arrays, 64, 0.5, 1.0, T | S, None, np.arange(N), grad_seed=52, chunk_V=16384)
    assert exact >= 0.8 * N


@pytest.mark.parametrize("support", [T, S, T | S])
def test_tail_whole_vocabulary_is_the_full_divergence(support):
    kd, torch = _kd()
    N, V = 40, 64
    arrays = kdsynth.small_case(43, N, V, 16, 16)
    print(f"tail k == V support={support}", flush=True)
    for beta in (0.0, 0.5, 1.0):
        out, _ = _case(kd, torch, arrays, 64, beta, 1.2, support, None, np.arange(N), grad_seed=53)
        zs = O.bf16_round(O.logits(arrays[0], arrays[1])) / 1.2
        zt = O.bf16_round(O.logits(arrays[2], arrays[3])) / 1.2
        full, _ = O.divergence(zs, zt, beta)
        assert_close(f"beta={beta} full", out["loss"].cpu().numpy(), full)
        assert np.allclose(out["p_mass"].cpu().numpy(), 1.0) and np.allclose(out["q_mass"].cpu().numpy(), 1.0)


@pytest.mark.parametrize("beta,support", [(0.5, T | S), (1.0, S)])
def test_tail_workload_v248k_1024_rows(beta, support):
    kd, torch = _kd()
    w = workload(5)
    rows = kdsynth.sample_rows(w.N, 1024, seed=13)
    print(f"tail {w.name} N={w.N} V={w.V} k={w.k} beta={beta} support={support} rows={len(rows)}", flush=True)
    _, exact = _case(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), w.k, beta, w.tau, support, None, rows,
                     grad_seed=54, chunk_V=0)
    assert exact >= 0.95 * len(rows)


def test_tail_kd_autograd_matches_direct_call():
    """tail_kd (kept rows gathered, per-token mean, autograd) against direct
    calls on every row with the mean's weights; ignored rows get a zero
    gradient and their own values do not enter the loss."""
    kd, torch = _kd()
    N, V, ds, dt = 96, 3000, 64, 64
    arrays = kdsynth.small_case(44, N, V, ds, dt)
    labels = kdsynth.uniform_labels(9, N, V, ignore_frac=0.1)
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int64)).cuda()
    lab32 = lab.to(torch.int32)
    valid = (lab != -100).float()
    assert 0 < int(valid.sum()) < N
    for k, beta in ((1, 0.5), (16, 0.5), (16, 1.0)):
        xs = dev[0].clone().requires_grad_(True)
        loss, fwd = kd.tail_kd(xs, dev[2], dev[1], dev[3], k=k, beta=beta, labels=lab, temperature=1.3,
                               chunk_V=1024, return_dict=True)
        loss.backward()
        assert fwd["loss"].numel() == int(valid.sum())  # only the kept rows were computed
        support = kd.tail_default_support(k, beta, True)
        full = kd.kd_tail_fwd(*dev, k, beta, 1.3, support, labels=lab32)
        direct = kd.kd_tail_bwd(dev[0], dev[1], full, k, beta, 1.3, support,
                                grad_loss=(valid / valid.sum()).contiguous(), chunk_V=1024)
        torch.cuda.synchronize()
        kept = valid.bool()
        assert torch.equal(fwd["loss"], full["loss"][kept])  # the same arithmetic per kept row
        lv = float(loss.detach())
        assert abs(lv - float((full["loss"] * valid).sum() / valid.sum())) <= 1e-5 * max(1.0, abs(lv))
        assert torch.all(xs.grad[~kept] == 0)
        assert torch.allclose(xs.grad.float(), direct.to(torch.bfloat16).float(), rtol=1e-2, atol=1e-4)
        none = kd.tail_kd(dev[0], dev[2], dev[1], dev[3], k=k, beta=beta, labels=lab, temperature=1.3,
                          reduction="none")
        assert torch.equal(none[kept], full["loss"][kept]) and torch.all(none[~kept] == 0)


@pytest.mark.parametrize("k,beta,support", [(1, 0.5, T | L), (8, 0.5, T | S | L), (8, 1.0, S | L)])
def test_tail_label_already_in_the_support(k, beta, support):
    """Labels set to the teacher's or the student's top-1 on some rows: the
    support lists them once (no extra label slot used)."""
    kd, torch = _kd()
    N, V, ds, dt = 64, 2000, 64, 64
    arrays = kdsynth.small_case(45, N, V, ds, dt)
    zs = O.bf16_round(O.logits(arrays[0], arrays[1]))
    zt = O.bf16_round(O.logits(arrays[2], arrays[3]))
    labels = kdsynth.uniform_labels(10, N, V, ignore_frac=0.1)
    labels[::2] = O.topk_order(zt, 1)[::2, 0]
    labels[1::4] = O.topk_order(zs, 1)[1::4, 0]
    print(f"tail label in support k={k} beta={beta} support={support}", flush=True)
    out, exact = _case(kd, torch, arrays, k, beta, 1.0, support, labels, np.arange(N), grad_seed=55)
    assert exact >= 0.9 * N
    sup = out["sup_idx"].cpu().numpy()
    ranked = (k if support & T else 0) + (k if support & S else 0)
    inside = list(range(0, N, 2)) if support & T else list(range(1, N, 4))  # label = a ranked top-1
    for r in inside:  # listed once, by its model's list; the label slot stays free
        assert np.sum(sup[r] == labels[r]) == 1
        assert sup[r, ranked] == -1 or sup[r, ranked] != labels[r]
    for r in range(N):
        if labels[r] >= 0:
            assert np.sum(sup[r] == labels[r]) == 1
