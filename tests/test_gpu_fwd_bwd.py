"""GPU parity of kd_fwd / kd_bwd against the fp64 oracle (through the C ABI).

Small cases compare every row and span several tiles with ragged tails
(tokens, vocabulary and hidden sizes that are not tile multiples). The
full-size workloads compare a seeded subset of rows (always the first and
last) computed one by one by the oracle, in the launch configuration the
benchmark uses. Tolerances (tests/helpers.py): per-token loss and LSEs
|d| <= 1e-3 |ref| + 1e-5; dL/dh_s and dL/dW_s per row cosine >= 0.9999 and
max|d| / max|ref| <= 2e-2 (dL/dh_s rows with |ref| < 1e-12 compared
absolutely to 1e-6; dL/dW_s rows below their fp32 floor compared absolutely).
dL/dW_s at full size needs a full [N, V] gradient on the CPU, so it is
checked there through identities that hold at any size: its rows sum to
zero, and sum W_s . dW_s equals sum h_s . dh_s (both are the sum of
dL/dz_s * z_s).
"""
import sys

import numpy as np
import pytest

import kdsynth
from oracle import kd_oracle as O
from tests.helpers import assert_close, assert_grad_rows, exact_shifted_case, to_dev, upload, wgrad_floor, workload

pytestmark = pytest.mark.gpu


def _kd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_chunked_kl_amd as kd
    kd.load_library()
    return kd, torch


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_rows(arrays, beta, tau, rows, grad=None, block=256):
    """The oracle's forward outputs and dL/dh_s for ``rows``, ``block`` rows
    at a time (host memory only)."""
    h_s, W_s, h_t, W_t = arrays
    fwd, dh = [], []
    for b0 in range(0, len(rows), block):
        rb = rows[b0:b0 + block]
        f, d = O.kd_fwd_bwd(h_s[rb], W_s, h_t[rb], W_t, beta, tau, grad_loss=None if grad is None else grad[rb])
        fwd.append(f)
        dh.append(d)
    return {k: np.concatenate([f[k] for f in fwd]) for k in fwd[0]}, np.concatenate(dh)


def run_case(kd, torch, arrays, beta, tau, rows=None, grad=None, chunk_V=2048, check_bwd=True):
    h_s, W_s, h_t, W_t = arrays
    dev = [to_dev(x) for x in arrays]
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, tau)
    g = None if grad is None else torch.from_numpy(grad.astype(np.float32)).cuda()
    dh = kd.kd_bwd(*dev, beta, tau, lse_s, lse_t, aux, grad_loss=g, chunk_V=chunk_V) if check_bwd else None
    torch.cuda.synchronize()
    sel = np.arange(h_s.shape[0]) if rows is None else np.asarray(rows)
    ref, dref = oracle_rows(arrays, beta, tau, sel, grad)
    assert_close("loss", loss.cpu().numpy()[sel], ref["loss"])
    assert_close("lse_s", lse_s.cpu().numpy()[sel], ref["lse_s"])
    assert_close("lse_t", lse_t.cpu().numpy()[sel], ref["lse_t"])
    if beta > 0:
        assert_close("aux", aux.cpu().numpy()[sel], ref["aux"])
    if check_bwd:
        assert_grad_rows(dh.cpu().numpy()[sel], dref)
    return loss, dh


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_tiny_fp32_workload(beta):
    kd, torch = _kd()
    w = workload(1)
    _say(f"tiny fp32 N={w.N} V={w.V} d={w.d_s} beta={beta}")
    run_case(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), beta, w.tau)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("beta,tau", [(0.0, 1.0), (1.0, 1.0), (1.0, 2.0), (0.3, 1.5), (0.5, 2.0)])
def test_ragged_small(dtype, beta, tau):
    kd, torch = _kd()
    # 3 token tiles (last ragged), 8 vocabulary tiles (last ragged), d_t not a multiple of 64
    N, V, ds, dt = 300, 1000, 64, 200
    arrays = kdsynth.small_case(11, N, V, ds, dt, dtype=dtype)
    grad = np.random.default_rng(3).uniform(-1, 2, size=N)
    grad[::7] = 0.0
    _say(f"ragged {dtype} N={N} V={V} d_s={ds} d_t={dt} beta={beta} tau={tau}")
    run_case(kd, torch, arrays, beta, tau, grad=grad, chunk_V=256)


@pytest.mark.parametrize("N,V", [(1, 2), (1, 300), (129, 2), (65, 257)])
def test_degenerate_shapes(N, V):
    kd, torch = _kd()
    arrays = kdsynth.small_case(5, N, V, 32, 48)
    for beta in (0.0, 0.5, 1.0):
        _say(f"degenerate N={N} V={V} beta={beta}")
        run_case(kd, torch, arrays, beta, 1.0, chunk_V=256)


@pytest.mark.parametrize("V", [257, 320, 321])
def test_dominant_entry_on_the_last_vocabulary_row(V):
    """The student's dominant entry (q near 1, the zero-sum path of the
    backward) on the vocabulary's last row, inside the last 256-row tile, whose
    rows past V the gradient sweep neutralises (each wave holds a 64-row
    slice): V = 257 puts it alone at the start of the first slice, V = 320 at
    the end of a full slice with every later slice past V, V = 321 alone at
    the start of the second slice. Every row against the oracle, each beta."""
    kd, torch = _kd()
    h_s, W_s, h_t, W_t = kdsynth.small_case(23, 130, V, 32, 48, dtype="f32")
    h_s[:, 0] = 4.0           # a hidden unit shared by every token
    W_s[V - 1, :] = 0.0
    W_s[V - 1, 0] = 5.0       # z_s = 20 on the last row for every token
    arrays = tuple(kdsynth.f32_to_bf16_bits(x) for x in (h_s, W_s, h_t, W_t))
    for beta in (0.0, 0.5, 1.0):
        _say(f"dominant last row N=130 V={V} beta={beta}")
        run_case(kd, torch, arrays, beta, 1.0, chunk_V=256)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_student_logits_offset_by_100(beta):
    """Student logits exact in bf16 and all near 100 (a hidden unit of 100
    against a column of ones; the softmax is that of the unshifted logits):
    the log-sum-exps near 100 cancel against each other in the loss and in
    the gradient's centring; every row against the oracle."""
    kd, torch = _kd()
    arrays = exact_shifted_case(41, 150, 3000, 16)
    _say(f"student logits offset by 100 N=150 V=3000 beta={beta}")
    run_case(kd, torch, arrays, beta, 1.5, chunk_V=1024)


def test_identical_distributions_give_zero():
    kd, torch = _kd()
    # teacher == student (same hidden state and unembedding): every divergence is 0
    h, W, _, _ = kdsynth.small_case(6, 200, 3000, 128, 128)
    dev = [to_dev(x) for x in (h, W, h, W)]
    for beta in (0.0, 0.5, 1.0):
        loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, 1.0)
        torch.cuda.synchronize()
        assert np.max(np.abs(loss.cpu().numpy())) < 2e-5
        assert np.array_equal(lse_s.cpu().numpy(), lse_t.cpu().numpy())


def test_beta_swap_symmetry_gpu():
    kd, torch = _kd()
    h_s, W_s, h_t, W_t = (to_dev(x) for x in kdsynth.small_case(7, 256, 2048, 128, 128))
    for b in (0.0, 0.25, 0.5):
        a = kd.kd_fwd(h_s, W_s, h_t, W_t, b, 1.0)[0]
        c = kd.kd_fwd(h_t, W_t, h_s, W_s, 1.0 - b, 1.0)[0]
        torch.cuda.synchronize()
        assert np.allclose(a.cpu().numpy(), c.cpu().numpy(), rtol=2e-4, atol=2e-5)


def test_backward_chunk_invariance():
    kd, torch = _kd()
    arrays = kdsynth.small_case(8, 384, 5000, 256, 128)
    dev = [to_dev(x) for x in arrays]
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, 1.0, 1.0)
    outs = [kd.kd_bwd(*dev, 1.0, 1.0, lse_s, lse_t, aux, chunk_V=c).cpu().numpy() for c in (256, 1024, 8192)]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-4, atol=1e-7)


def test_workload_rkl_v152k_n4k_all_rows():
    """Every row of the 4k-token workload, at the default recompute chunk."""
    kd, torch = _kd()
    w = workload(2)
    _say(f"{w.name} N={w.N} V={w.V} all rows, default chunk")
    run_case(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), 1.0, w.tau, chunk_V=0)


@pytest.mark.parametrize("n,beta", [(192, 1.0), (256, 1.0), (256, 0.5), (512, 1.0)])
def test_small_n_sweep_shapes_all_rows(n, beta):
    """The small-N sweep's shapes (the 4k-token workload's vocabulary and
    hidden sizes at a few hundred tokens), every row, forward and dL/dh_s at
    the default (whole-vocabulary) chunk. These forward grids (token tiles x
    vocabulary splits: 238 blocks at 256 tokens, 476 at 512) are not
    multiples of 8, so they run rounded up with idle padding blocks."""
    kd, torch = _kd()
    w = workload(2)
    _say(f"{w.name} shapes N={n} V={w.V} beta={beta} all rows, default chunk")
    run_case(kd, torch, (w.h_s[:n], w.W_s, w.h_t[:n], w.W_t), beta, w.tau, chunk_V=0)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_workload_jsd_sweep_v152k_n32k_1024_rows(beta):
    """1024 seeded rows (first and last included) of the benchmarked workload,
    in the benchmark's launch configuration (the default recompute chunk)."""
    kd, torch = _kd()
    w = workload(3)
    rows = kdsynth.sample_rows(w.N, 1024)
    _say(f"{w.name} N={w.N} V={w.V} beta={beta} rows={len(rows)} default chunk")
    run_case(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), beta, w.tau, rows=rows, chunk_V=0)


def test_workload_heavy_head_v248k_1024_rows():
    """1024 seeded rows of the heavy-head workload, among them the 32 rows whose
    largest logit on a heavy vocabulary entry is highest (the hardest for the
    log-sum-exp range) and rows with a saturated student (q_max = 1 - 1e-7 and
    beyond, where dL/dh_s is 1e-6 .. 1e-14 and a direct fp32 evaluation of the
    dominant entry's gradient loses it)."""
    kd, torch = _kd()
    w = workload(4)
    heavy = kdsynth.bf16_bits_to_f32(w.W_s[w.meta["heavy_rows"]]).astype(np.float64)
    zmax = np.concatenate([(kdsynth.bf16_bits_to_f32(w.h_s[i:i + 2048]).astype(np.float64) @ heavy.T).max(axis=1)
                           for i in range(0, w.N, 2048)])
    must = np.concatenate([np.argsort(zmax)[-32:], [22, 238, 300, 8005]])
    rows = kdsynth.sample_rows(w.N, 1024, must=must)
    _say(f"{w.name} N={w.N} V={w.V} rows={len(rows)} default chunk")
    run_case(kd, torch, (w.h_s, w.W_s, w.h_t, w.W_t), 1.0, w.tau, rows=rows, chunk_V=0)


def test_heavy_head_chunk_sizes():
    """The heavy-head workload's three recompute chunk sizes give dL/dh_s
    within fp32 noise of the default chunk (and the oracle on sampled rows)."""
    kd, torch = _kd()
    w = workload(4)
    dev = upload(w)
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, 1.0, w.tau)
    base = kd.kd_bwd(*dev, 1.0, w.tau, lse_s, lse_t, aux, chunk_V=0)
    rows = kdsynth.sample_rows(w.N, 64, seed=17)
    _, dref = oracle_rows((w.h_s, w.W_s, w.h_t, w.W_t), 1.0, w.tau, rows)
    for c in (4096, 8192, 16384):
        _say(f"{w.name} chunk_V={c}")
        dh = kd.kd_bwd(*dev, 1.0, w.tau, lse_s, lse_t, aux, chunk_V=c)
        torch.cuda.synchronize()
        assert_grad_rows(dh.cpu().numpy()[rows], dref, name=f"dh_s chunk {c}")
        d = (dh - base).abs().max().item()
        assert d <= 1e-3 * base.abs().max().item(), d
        del dh
    del dev, base
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- dL/dW_s
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("beta,tau", [(0.0, 1.0), (1.0, 1.0), (1.0, 2.0), (0.5, 1.5)])
def test_weight_gradient_ragged_small(dtype, beta, tau):
    kd, torch = _kd()
    N, V, ds, dt = 300, 1000, 64, 200
    arrays = kdsynth.small_case(11, N, V, ds, dt, dtype=dtype)
    h_s, W_s, h_t, W_t = arrays
    grad = np.random.default_rng(4).uniform(-1, 2, size=N)
    grad[::5] = 0.0
    _say(f"dW ragged {dtype} N={N} V={V} d_s={ds} d_t={dt} beta={beta} tau={tau}")
    dev = [to_dev(x) for x in arrays]
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, tau)
    g = torch.from_numpy(grad.astype(np.float32)).cuda()
    dh, dW = kd.kd_bwd(*dev, beta, tau, lse_s, lse_t, aux, grad_loss=g, chunk_V=256, want_dW=True)
    dh_only = kd.kd_bwd(*dev, beta, tau, lse_s, lse_t, aux, grad_loss=g, chunk_V=256)
    _, dW_only = kd.kd_bwd(*dev, beta, tau, lse_s, lse_t, aux, grad_loss=g, chunk_V=256, want_dh=False,
                           want_dW=True)
    torch.cuda.synchronize()
    ref = O.kd_bwd_w(h_s, W_s, h_t, W_t, beta, tau, grad_loss=grad)
    assert_grad_rows(dW.cpu().numpy(), ref, name="dW_s", floor=wgrad_floor(h_s, W_s, h_t, W_t, beta, tau, grad))
    # the dh_s path is unchanged by also asking for dW_s, and dW_s alone is the same
    assert np.array_equal(dh.cpu().numpy(), dh_only.cpu().numpy())
    assert np.array_equal(dW.cpu().numpy(), dW_only.cpu().numpy())


@pytest.mark.parametrize("N,V", [(1, 2), (1, 300), (129, 2), (65, 257)])
def test_weight_gradient_degenerate(N, V):
    kd, torch = _kd()
    arrays = kdsynth.small_case(5, N, V, 32, 48)
    dev = [to_dev(x) for x in arrays]
    for beta in (0.0, 0.5, 1.0):
        _say(f"dW degenerate N={N} V={V} beta={beta}")
        loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, 1.0)
        _, dW = kd.kd_bwd(*dev, beta, 1.0, lse_s, lse_t, aux, chunk_V=256, want_dW=True)
        torch.cuda.synchronize()
        ref = O.kd_bwd_w(*arrays, beta, 1.0)
        assert_grad_rows(dW.cpu().numpy(), ref, name="dW_s", floor=wgrad_floor(*arrays, beta, 1.0))


def test_weight_gradient_chunk_invariance():
    kd, torch = _kd()
    arrays = kdsynth.small_case(8, 384, 5000, 256, 128)
    dev = [to_dev(x) for x in arrays]
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, 1.0, 1.0)
    outs = [kd.kd_bwd(*dev, 1.0, 1.0, lse_s, lse_t, aux, chunk_V=c, want_dh=False, want_dW=True)[1].cpu().numpy()
            for c in (256, 1024, 8192)]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-4, atol=1e-7)


def _identity_check(kd, torch, w, beta, chunk_V):
    dev = upload(w)
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, w.tau)
    dh, dW = kd.kd_bwd(*dev, beta, w.tau, lse_s, lse_t, aux, chunk_V=chunk_V, want_dW=True)
    torch.cuda.synchronize()
    W_s = dev[1].float()
    h_s = dev[0].float()
    a = float((W_s.double() * dW.double()).sum())
    b = float((h_s.double() * dh.double()).sum())
    scale = float((W_s.double() * dW.double()).abs().sum())
    assert abs(a - b) <= 1e-3 * scale, (a, b, scale)
    col = dW.double().sum(0)
    assert float(col.abs().max()) <= 1e-3 * float(dW.double().abs().sum(0).max()), float(col.abs().max())
    assert torch.isfinite(dW).all()
    del dev, dh, dW
    torch.cuda.empty_cache()


def test_weight_gradient_identities_v152k_n4k():
    kd, torch = _kd()
    w = workload(2)
    _say(f"dW identities {w.name} N={w.N} V={w.V}")
    _identity_check(kd, torch, w, 1.0, 8192)


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_weight_gradient_identities_v152k_n32k(beta):
    kd, torch = _kd()
    w = workload(3)
    _say(f"dW identities {w.name} N={w.N} V={w.V} beta={beta}")
    _identity_check(kd, torch, w, beta, 16384)


@pytest.mark.parametrize("beta", [1.0, 0.5])
def test_weight_gradient_mid_size_all_rows(beta):
    """dL/dW_s against the oracle on every vocabulary row at a size where the
    wide gradient-tile path runs (2048 tokens over 65536 entries at the
    default chunk: one chunk of 256 tiles, two per workgroup) and the
    weight-gradient GEMM spans 256 x 2 output tiles."""
    kd, torch = _kd()
    N, V, ds, dt = 2048, 65536, 512, 1024
    arrays = kdsynth.small_case(82, N, V, ds, dt)
    grad = np.random.default_rng(83).uniform(-1, 2, size=N)
    _say(f"dW mid size N={N} V={V} d_s={ds} d_t={dt} beta={beta}")
    dev = [to_dev(x) for x in arrays]
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, 1.2)
    g = torch.from_numpy(grad.astype(np.float32)).cuda()
    _, dW = kd.kd_bwd(*dev, beta, 1.2, lse_s, lse_t, aux, grad_loss=g, chunk_V=0, want_dh=False, want_dW=True)
    torch.cuda.synchronize()
    ref = O.kd_bwd_w(*arrays, beta, 1.2, grad_loss=grad)
    assert_grad_rows(dW.cpu().numpy(), ref, name="dW_s", floor=wgrad_floor(*arrays, beta, 1.2, grad))


# --------------------------------------------------------------------------- token masking
def test_gather_scatter_rows_exact():
    kd, torch = _kd()
    g = np.random.default_rng(41)
    N, d = 300, 200  # bf16 rows of 400 bytes: the 16-byte path
    x = torch.from_numpy(g.integers(0, 1 << 16, size=(N, d), dtype=np.uint16).view(np.int16)).cuda()
    rows_np = np.array([5, 0, 299, 17, 300, -1, 150], dtype=np.int32)  # two indices out of range
    rows = torch.from_numpy(rows_np).cuda()
    y = kd.kd_gather_rows(x, rows)
    want = np.zeros((len(rows_np), d), dtype=np.int16)
    ok = (rows_np >= 0) & (rows_np < N)
    want[ok] = x.cpu().numpy()[rows_np[ok]]
    assert np.array_equal(y.cpu().numpy(), want)
    z = kd.kd_scatter_rows(y, rows, N)
    back = np.zeros((N, d), dtype=np.int16)
    back[rows_np[ok]] = want[ok]
    assert np.array_equal(z.cpu().numpy(), back)
    # 4-byte path (fp32 rows of one value)
    v = torch.arange(7, dtype=torch.float32, device="cuda").reshape(7, 1)
    w = kd.kd_scatter_rows(v, rows, N)
    exp = np.zeros((N, 1), dtype=np.float32)
    exp[rows_np[ok], 0] = np.arange(7, dtype=np.float32)[ok]
    assert np.array_equal(w.cpu().numpy(), exp)
    torch.cuda.synchronize()


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_masked_tokens_are_skipped_not_changed(beta):
    kd, torch = _kd()
    N, V, ds, dt = 300, 1000, 64, 200
    arrays = kdsynth.small_case(11, N, V, ds, dt)
    labels = kdsynth.uniform_labels(9, N, V, ignore_frac=0.4)
    valid = labels != -100
    _say(f"masked N={N} kept={int(valid.sum())} beta={beta}")
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int64)).cuda()
    # full computation of every row, as the reference for the kept rows
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, 1.5)
    gl = torch.from_numpy((valid / valid.sum()).astype(np.float32)).cuda()
    dh_full = kd.kd_bwd(*dev, beta, 1.5, lse_s, lse_t, aux, grad_loss=gl, chunk_V=512)
    # the loss on the kept rows only
    xs = dev[0].clone().requires_grad_(True)
    per_tok = kd.jsd(xs, dev[2], dev[1], dev[3], beta=beta, temperature=1.5, reduction="none", chunk_V=512,
                     labels=lab)
    mean = kd.jsd(xs, dev[2], dev[1], dev[3], beta=beta, temperature=1.5, reduction="mean", chunk_V=512, labels=lab)
    mean.backward()
    torch.cuda.synchronize()
    pt = per_tok.detach().cpu().numpy()
    assert np.array_equal(pt[valid], loss.cpu().numpy()[valid])  # same arithmetic per kept row
    assert np.all(pt[~valid] == 0.0)
    m = float(mean.detach())
    assert abs(m - float(loss.cpu().numpy()[valid].mean())) <= 1e-6 * (1 + abs(m))
    gx = xs.grad.float().cpu().numpy()
    assert np.all(gx[~valid] == 0.0)
    assert np.allclose(gx[valid], dh_full.to(torch.bfloat16).float().cpu().numpy()[valid], rtol=1e-6, atol=0)


@pytest.mark.parametrize("fn,beta", [("forward_kl", 0.0), ("reverse_kl", 1.0), ("jsd", 0.5), ("jsd", 0.3)])
def test_masked_losses_against_oracle(fn, beta):
    """The losses with 40 % of the labels ignored against the oracle on the
    kept rows: per-token values (0 at ignored positions), the mean over kept
    tokens, and the gradient of that mean (the oracle's dL/dh_s with weight
    1 / kept on each kept row; zero on ignored rows)."""
    kd, torch = _kd()
    N, V, ds, dt = 300, 5000, 64, 136
    arrays = kdsynth.small_case(61, N, V, ds, dt)
    labels = kdsynth.uniform_labels(19, N, V, ignore_frac=0.4)
    kept = np.flatnonzero(labels != -100)
    _say(f"masked {fn} beta={beta} N={N} kept={len(kept)}")
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int64)).cuda()
    f = getattr(kd, fn)
    kw = dict(temperature=1.5, chunk_V=1024, labels=lab)
    if fn == "jsd":
        kw["beta"] = beta
    xs = dev[0].clone().requires_grad_(True)
    mean = f(xs, dev[2], dev[1], dev[3], **kw)
    mean.backward()
    per_tok = f(dev[0], dev[2], dev[1], dev[3], reduction="none", **kw)
    total = f(dev[0], dev[2], dev[1], dev[3], reduction="sum", **kw)
    torch.cuda.synchronize()
    ref, dref = oracle_rows(arrays, beta, 1.5, kept, grad=np.full(N, 1.0 / len(kept)))
    pt = per_tok.cpu().numpy()
    assert_close("kept loss", pt[kept], ref["loss"])
    assert np.all(np.delete(pt, kept) == 0.0)
    assert_close("mean", np.array([float(mean.detach())]), np.array([ref["loss"].mean()]))
    assert_close("sum", np.array([float(total)]), np.array([ref["loss"].sum()]))
    gx = xs.grad.float().cpu().numpy()
    assert np.all(np.delete(gx, kept, axis=0) == 0.0)
    assert_grad_rows(gx[kept], dref, name="masked dL/dh_s (bf16)")


def test_all_tokens_masked():
    kd, torch = _kd()
    arrays = kdsynth.small_case(12, 64, 500, 32, 32)
    dev = [to_dev(x) for x in arrays]
    lab = torch.full((64,), -100, dtype=torch.int64, device="cuda")
    xs = dev[0].clone().requires_grad_(True)
    m = kd.reverse_kl(xs, dev[2], dev[1], dev[3], labels=lab)
    m.backward()
    assert float(m.detach()) == 0.0 and float(xs.grad.float().abs().sum()) == 0.0
    n = kd.reverse_kl(dev[0], dev[2], dev[1], dev[3], labels=lab, reduction="none")
    assert n.shape == (64,) and float(n.abs().sum()) == 0.0


@pytest.mark.parametrize("beta", [1.0, 0.5])
def test_split_contraction_backward(beta):
    """Few tokens: the dh GEMM splits its contraction over the chunk into up to
    32 partial tiles summed in a fixed order (chunk_V = 16384 -> 32 splits of
    512 entries; 4096 -> 8; 256 -> none). Every split count matches the oracle."""
    kd, torch = _kd()
    N, V, ds, dt = 200, 20000, 96, 64
    arrays = kdsynth.small_case(71, N, V, ds, dt)
    grad = np.random.default_rng(8).uniform(-1, 2, size=N)
    for chunk in (16384, 4096, 256):
        _say(f"split dh N={N} V={V} chunk={chunk} beta={beta}")
        run_case(kd, torch, arrays, beta, 1.3, grad=grad, chunk_V=chunk)


def test_split_contraction_topk_backward():
    kd, torch = _kd()
    N, V, ds, dt = 150, 30000, 64, 64
    arrays = kdsynth.small_case(72, N, V, ds, dt)
    labels = kdsynth.uniform_labels(13, N, V, ignore_frac=0.2)
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int32)).cuda()
    rng = np.random.default_rng(14)
    wb, wc, we = (rng.uniform(0, 1.5, N) for _ in range(3))
    f32 = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()  # noqa: E731
    out = kd.kd_topk_fwd(*dev, 16, 1.2, labels=lab)
    dh = kd.kd_topk_bwd(dev[0], dev[1], out, 16, 1.2, labels=lab, grad_binary=f32(wb), grad_cond=f32(wc),
                        grad_ce=f32(we), chunk_V=16384)
    torch.cuda.synchronize()
    ref = O.kd_topk_bwd(*arrays, 16, 1.2, labels, wb, wc, we, sel=out["idx"].cpu().numpy())
    assert_grad_rows(dh.cpu().numpy(), ref, name="topk dh_s (split)")


def test_default_chunk_backward():
    """chunk_V = 0 runs the library's default chunk (here the whole vocabulary,
    one chunk, with the dh contraction split): the same bits as passing that
    chunk explicitly, and the oracle's gradient, for all three backward calls."""
    kd, torch = _kd()
    N, V, ds, dt = 200, 20000, 96, 64
    c = kd.default_chunk(N, V)
    assert c == 20224
    arrays = kdsynth.small_case(73, N, V, ds, dt)
    grad = np.random.default_rng(9).uniform(-1, 2, size=N)
    _say(f"default chunk kd_bwd N={N} V={V} chunk={c}")
    _, dh0 = run_case(kd, torch, arrays, 0.5, 1.1, grad=grad, chunk_V=0)
    _, dhc = run_case(kd, torch, arrays, 0.5, 1.1, grad=grad, chunk_V=c)
    assert torch.equal(dh0, dhc)
    dev = [to_dev(x) for x in arrays]
    _say(f"default chunk kd_topk_bwd / kd_tail_bwd N={N} V={V} chunk={c}")
    one = torch.ones(N, dtype=torch.float32, device="cuda")
    out = kd.kd_topk_fwd(*dev, 8, 1.1)
    t0, tc = (kd.kd_topk_bwd(dev[0], dev[1], out, 8, 1.1, grad_binary=one, grad_cond=one, chunk_V=cv)
              for cv in (0, c))
    tl = kd.kd_tail_fwd(*dev, 8, 0.5, 1.1, kd.KD_SUPPORT_TEACHER | kd.KD_SUPPORT_STUDENT)
    l0, lc = (kd.kd_tail_bwd(dev[0], dev[1], tl, 8, 0.5, 1.1, kd.KD_SUPPORT_TEACHER | kd.KD_SUPPORT_STUDENT,
                             chunk_V=cv) for cv in (0, c))
    torch.cuda.synchronize()
    assert torch.equal(t0, tc) and torch.equal(l0, lc)
    ref = O.kd_topk_bwd(*arrays, 8, 1.1, None, np.ones(N), np.ones(N), None, sel=out["idx"].cpu().numpy())
    assert_grad_rows(t0.cpu().numpy(), ref, name="topk dh_s (default chunk)")


@pytest.mark.parametrize("N,V,ds,dt,dtype", [
    (300, 5000, 8, 136, "bf16"),   # pair 1 is one stage, pair 2 three with a 16-byte tail; 20 vocabulary tiles
    (130, 1100, 72, 8, "bf16"),    # the reverse, and a ragged last vocabulary tile
    (257, 3000, 8, 8, "f32"),      # one stage per pair: the fetch runs two stages ahead across pairs and tiles
    (64, 600, 264, 40, "f32"),
])
def test_stage_ring_fetch_boundaries(N, V, ds, dt, dtype):
    """The stage ring rebuilds its fetch state when the cursor moves to the
    other operand pair or to the next vocabulary tile, and fetches past a
    block's last tile read nothing. K extents of one to five 128-byte stages
    with ragged tails, several tiles per block, both dtypes; fwd and bwd at
    beta = 1/2 (two forward sweeps) against the oracle."""
    kd, torch = _kd()
    _say(f"ring fetch N={N} V={V} d_s={ds} d_t={dt} {dtype}")
    arrays = kdsynth.small_case(90 + ds + dt, N, V, ds, dt, dtype=dtype)
    grad = np.random.default_rng(ds).uniform(-1, 2, size=N)
    run_case(kd, torch, arrays, 0.5, 1.2, grad=grad, chunk_V=1024)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_small_token_tile_forward(beta):
    """Up to 64 tokens the forward sweep runs a 64-row token tile with a
    four-stage ring: against the oracle at 1, 37 and 64 tokens (several
    vocabulary tiles per workgroup, ragged hidden sizes), and the first 64
    tokens of a 65-token call (the 128-row tile) give the same per-token
    results within fp32 rounding."""
    kd, torch = _kd()
    V, ds, dt = 9000, 136, 264
    arrays = kdsynth.small_case(95, 65, V, ds, dt)
    for n in (1, 37, 64):
        _say(f"small token tile N={n} V={V} beta={beta}")
        sub = tuple(x[:n] if i in (0, 2) else x for i, x in enumerate(arrays))
        run_case(kd, torch, sub, beta, 1.3, chunk_V=2048)
    dev = [to_dev(x) for x in arrays]
    big = kd.kd_fwd(*dev, beta, 1.3)
    small = kd.kd_fwd(dev[0][:64].contiguous(), dev[1], dev[2][:64].contiguous(), dev[3], beta, 1.3)
    torch.cuda.synchronize()
    for name, b, s in zip(("loss", "lse_s", "lse_t", "aux"), big, small):
        if name == "aux" and beta == 0.0:
            continue
        np.testing.assert_allclose(s.cpu().numpy(), b.cpu().numpy()[:64], rtol=2e-6, atol=1e-6, err_msg=name)
