"""GPU parity of kd_topk_fwd (top-k three-term KD over bf16 logits) and
kd_topk_bwd against the fp64 oracle, through the C ABI. Selection is compared
index for index; logits that sit within the fp32 accumulation bound of a bf16
rounding midpoint may round either way (tests/helpers.check_topk_rows). The
gradient is compared with the oracle's gradient for the selection the GPU
made (per row cosine >= 0.9999, max|d| / max|ref| <= 2e-2)."""
import sys

import numpy as np
import pytest

import kdsynth
from oracle import kd_oracle as O
from tests.helpers import assert_grad_rows, check_topk_rows, exact_shifted_case, to_dev, workload

pytestmark = pytest.mark.gpu


def _kd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_chunked_kl_amd as kd
    kd.load_library()
    return kd, torch


def _run(kd, torch, arrays, k, tau, labels=None):
    dev = [to_dev(x) for x in arrays]
    lab = None if labels is None else torch.from_numpy(labels.astype(np.int32)).cuda()
    out = kd.kd_topk_fwd(*dev, k, tau, labels=lab)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("k", [1, 8, 64])
@pytest.mark.parametrize("tau", [1.0, 1.5])
def test_topk_ragged_small(k, tau):
    kd, torch = _kd()
    N, V, ds, dt = 150, 5000, 64, 128  # 2 token tiles (ragged), 20 vocabulary tiles (ragged)
    arrays = kdsynth.small_case(21, N, V, ds, dt)
    labels = kdsynth.uniform_labels(5, N, V, ignore_frac=0.2)
    print(f"topk ragged N={N} V={V} k={k} tau={tau}", flush=True)
    out = _run(kd, torch, arrays, k, tau, labels)
    exact, flagged = check_topk_rows(out, *arrays, np.arange(N), k, tau, labels)
    print(f"exact {exact} flagged {flagged}", flush=True)
    assert exact >= 0.9 * N


def test_topk_multi_split_and_ties():
    kd, torch = _kd()
    # three vocabulary splits; small logits -> many bf16 ties at the k-th slot
    N, V, ds, dt = 64, 150001, 32, 32
    arrays = kdsynth.small_case(22, N, V, ds, dt, logit_std=0.5)
    labels = kdsynth.uniform_labels(6, N, V)
    print(f"topk splits N={N} V={V}", flush=True)
    out = _run(kd, torch, arrays, 64, 1.0, labels)
    exact, flagged = check_topk_rows(out, *arrays, np.arange(N), 64, 1.0, labels)
    print(f"exact {exact} flagged {flagged}", flush=True)
    assert exact >= 0.8 * N


def test_topk_k_equals_v():
    kd, torch = _kd()
    N, V = 40, 64
    arrays = kdsynth.small_case(23, N, V, 16, 16)
    out = _run(kd, torch, arrays, 64, 1.0)
    exact, _ = check_topk_rows(out, *arrays, np.arange(N), 64, 1.0)
    assert np.allclose(out["binary"].cpu().numpy(), 0.0, atol=1e-5)


def test_topk_workload_v248k_1024_rows():
    kd, torch = _kd()
    w = workload(5)
    rows = kdsynth.sample_rows(w.N, 1024)
    print(f"{w.name} N={w.N} V={w.V} rows={len(rows)}", flush=True)
    out = _run(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), w.k, w.tau, w.labels)
    exact, flagged = check_topk_rows(out, w.h_s, w.W_s, w.h_t, w.W_t, rows, w.k, w.tau, w.labels)
    print(f"exact {exact} flagged {flagged}", flush=True)
    assert exact >= 0.95 * len(rows)


def test_topk_workload_svd256_teacher_1024_rows():
    """The same workload with the teacher compressed to rank 256 (its hidden
    state projected on the top-256 right singular vectors of W_t, and W_t
    replaced by the matching left singular vectors), both rounded to bf16 and
    fed to the kernel as an ordinary d_t = 256 teacher."""
    kd, torch = _kd()
    w = workload(5)
    r = kdsynth.SVD_RANK
    print(f"{w.name} rank-{r} teacher: factorising W_t {w.W_t.shape}", flush=True)
    h_r, W_r, S = O.svd_teacher(w.h_t, w.W_t, r, method="gram")
    assert np.allclose(W_r.T @ W_r, np.eye(r), atol=1e-6)
    h_rb = kdsynth.f32_to_bf16_bits(h_r.astype(np.float32))
    W_rb = kdsynth.f32_to_bf16_bits(W_r.astype(np.float32))
    rows = kdsynth.sample_rows(w.N, 1024, seed=11)
    out = _run(kd, torch, (w.h_s, w.W_s, h_rb, W_rb), w.k, w.tau, w.labels)
    exact, flagged = check_topk_rows(out, w.h_s, w.W_s, h_rb, W_rb, rows, w.k, w.tau, w.labels)
    print(f"rank-{r} teacher rows={len(rows)}: exact {exact} flagged {flagged}", flush=True)
    assert exact >= 0.95 * len(rows)


# --------------------------------------------------------------------------- kd_topk_bwd
def _bwd_case(kd, torch, arrays, k, tau, labels, rows, seed, chunk_V=256):
    h_s, W_s, h_t, W_t = arrays
    N = h_s.shape[0]
    rng = np.random.default_rng(seed)
    wb, wc, we = rng.uniform(-0.5, 1.5, N), rng.uniform(-0.5, 1.5, N), rng.uniform(0.0, 1.0, N)
    dev = [to_dev(x) for x in arrays]
    lab = None if labels is None else torch.from_numpy(labels.astype(np.int32)).cuda()
    out = kd.kd_topk_fwd(*dev, k, tau, labels=lab)
    f32 = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()  # noqa: E731
    dh = kd.kd_topk_bwd(dev[0], dev[1], out, k, tau, labels=lab, grad_binary=f32(wb), grad_cond=f32(wc),
                        grad_ce=f32(we) if labels is not None else None, chunk_V=chunk_V)
    torch.cuda.synchronize()
    sel_all = out["idx"].cpu().numpy()
    ref = []
    for b0 in range(0, len(rows), 256):  # host memory: 256 rows of full-vocabulary logits at a time
        rb = rows[b0:b0 + 256]
        ref.append(O.kd_topk_bwd(h_s[rb], W_s, h_t[rb], W_t, k, tau, None if labels is None else labels[rb],
                                 wb[rb], wc[rb], we[rb] if labels is not None else None, sel=sel_all[rb]))
    assert_grad_rows(dh.cpu().numpy()[rows], np.concatenate(ref), name="topk dh_s")
    return out, dh


@pytest.mark.parametrize("k", [1, 8, 64])
@pytest.mark.parametrize("tau", [1.0, 1.5])
def test_topk_bwd_ragged_small(k, tau):
    kd, torch = _kd()
    N, V, ds, dt = 150, 5000, 64, 128
    arrays = kdsynth.small_case(21, N, V, ds, dt)
    labels = kdsynth.uniform_labels(5, N, V, ignore_frac=0.2)
    print(f"topk bwd ragged N={N} V={V} k={k} tau={tau}", flush=True)
    _bwd_case(kd, torch, arrays, k, tau, labels, np.arange(N), seed=31)


def test_topk_bwd_without_labels_and_k_equals_v():
    kd, torch = _kd()
    N, V = 40, 64
    arrays = kdsynth.small_case(23, N, V, 16, 16)
    print("topk bwd k == V, no labels", flush=True)
    _bwd_case(kd, torch, arrays, 64, 1.0, None, np.arange(N), seed=32)


@pytest.mark.parametrize("tau", [1.0, 1.5])
def test_topk_bwd_logits_past_exp_range_without_ce(tau):
    """Student logits near 100 and no CE term: the dense part of the gradient
    (A q) must not evaluate exp of an unnormalised logit (which overflows and
    turned 0 * inf into NaN); every row against the oracle."""
    kd, torch = _kd()
    N, V = 64, 3000
    arrays = exact_shifted_case(27, N, V, 16)
    print(f"topk bwd shifted student logits N={N} V={V} tau={tau}", flush=True)
    _bwd_case(kd, torch, arrays, 8, tau, None, np.arange(N), seed=35)


@pytest.mark.parametrize("teacher", [False, True])
@pytest.mark.parametrize("head", [0.0, 14.0])
def test_topk_terms_keep_precision_under_a_common_offset(head, teacher):
    """One model's logits raised by 100 (an offset the softmax ignores): the
    terms, the masses and the CE against the oracle to an absolute 4e-6, the
    precision of unshifted logits. With ``head`` the teacher's top-8 holds
    all but a few percent of both masses, so the binary term is near zero.
    A set mass formed as the exp of a difference of two fp32 log-sum-exps
    near 67 (tau = 1.5) is good to only about 1e-5 and fails this bound."""
    kd, torch = _kd()
    N, V, k, tau = 64, 3000, 8, 1.5
    arrays = exact_shifted_case(31, N, V, 16, head=head, teacher=teacher)
    labels = kdsynth.uniform_labels(9, N, V)
    who = "teacher" if teacher else "student"
    print(f"topk fwd shifted {who} logits head={head} N={N} V={V} k={k} tau={tau}", flush=True)
    out = _run(kd, torch, arrays, k, tau, labels)
    ref = O.kd_topk_fwd(*arrays, k, tau, labels=labels)
    assert np.array_equal(out["idx"].cpu().numpy(), ref["idx"])  # exact logits: no rounding ties
    for name in ("binary", "cond", "p_mass", "q_mass", "ce"):
        got = out[name].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[name]).max()
        assert err <= 4e-6, f"{name}: max abs err {err:.3g}"
    if head:
        assert (1.0 - ref["q_mass"]).max() < 0.05 and np.abs(ref["binary"]).min() < 1e-5


def test_topk_bwd_workload_v248k_1024_rows():
    kd, torch = _kd()
    w = workload(5)
    rows = kdsynth.sample_rows(w.N, 1024)
    print(f"topk bwd {w.name} N={w.N} V={w.V} rows={len(rows)} default chunk", flush=True)
    _bwd_case(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), w.k, w.tau, w.labels, rows, seed=33, chunk_V=0)


def test_topk_kd_autograd_matches_direct_call():
    kd, torch = _kd()
    N, V, ds, dt = 96, 3000, 64, 64
    arrays = kdsynth.small_case(24, N, V, ds, dt)
    labels = kdsynth.uniform_labels(7, N, V, ignore_frac=0.1)
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int64)).cuda()
    xs = dev[0].clone().requires_grad_(True)
    terms = kd.topk_kd(xs, dev[2], dev[1], dev[3], k=16, labels=lab, temperature=1.3, chunk_V=1024)
    valid = (lab != -100).float()
    loss = (0.7 * terms["binary"] + 1.1 * terms["cond"] + 0.3 * torch.nan_to_num(terms["ce"]) * valid).sum()
    loss.backward()
    out = kd.kd_topk_fwd(*dev, 16, 1.3, labels=lab.to(torch.int32))
    g = lambda c: torch.full((N,), c, dtype=torch.float32, device="cuda")  # noqa: E731
    # ignored rows are gathered out: no term and no gradient there
    direct = kd.kd_topk_bwd(dev[0], dev[1], out, 16, 1.3, labels=lab.to(torch.int32), grad_binary=0.7 * valid,
                            grad_cond=1.1 * valid, grad_ce=0.3 * valid, chunk_V=1024)
    torch.cuda.synchronize()
    kept = valid.bool()
    assert torch.all(terms["binary"][~kept] == 0) and torch.all(terms["ce"][~kept] == 0)
    assert torch.equal(terms["binary"][kept], out["binary"][kept])
    assert torch.all(xs.grad[~kept] == 0)
    assert torch.allclose(xs.grad.float(), direct.to(torch.bfloat16).float(), rtol=1e-2, atol=1e-3)


def test_topk_kd_masked_against_oracle():
    """topk_kd with 40 % of the labels ignored: the kept rows' terms against
    the oracle (three-term acceptance on the kept rows) and the gradient of
    the summed terms against the oracle's top-k gradient for the kernel's
    selection, zero on ignored rows."""
    kd, torch = _kd()
    N, V, ds, dt = 200, 4000, 64, 96
    arrays = kdsynth.small_case(25, N, V, ds, dt)
    labels = kdsynth.uniform_labels(12, N, V, ignore_frac=0.4)
    kept = np.flatnonzero(labels != -100)
    print(f"topk_kd masked N={N} kept={len(kept)}", flush=True)
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int64)).cuda()
    xs = dev[0].clone().requires_grad_(True)
    terms = kd.topk_kd(xs, dev[2], dev[1], dev[3], k=8, labels=lab, temperature=1.2, chunk_V=1024)
    (terms["binary"] + terms["cond"] + 0.5 * terms["ce"]).sum().backward()
    torch.cuda.synchronize()
    assert np.array_equal(terms["rows"].cpu().numpy(), kept)
    sub = tuple(x[kept] if i in (0, 2) else x for i, x in enumerate(arrays))
    out = {f: terms[f].detach() for f in ("idx", "val", "val_s", "p_mass", "q_mass", "lse_s", "lse_t")}
    for f in ("binary", "cond", "ce"):
        out[f] = terms[f].detach()[torch.from_numpy(kept).cuda()]
    exact, flagged = check_topk_rows(out, *sub, np.arange(len(kept)), 8, 1.2, labels[kept])
    print(f"exact {exact} flagged {flagged}", flush=True)
    assert exact >= 0.9 * len(kept)
    one = np.ones(len(kept))
    ref = O.kd_topk_bwd(*sub, 8, 1.2, labels[kept], one, one, 0.5 * one, sel=terms["idx"].cpu().numpy())
    gx = xs.grad.float().cpu().numpy()
    assert np.all(np.delete(gx, kept, axis=0) == 0.0)
    assert_grad_rows(gx[kept], ref, name="masked topk dL/dh_s (bf16)")
