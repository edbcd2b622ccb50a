"""Seeded random-shape parity sweep (GPU): token counts, vocabulary sizes and
hidden sizes that are not tile multiples (hidden sizes down to 8), random
beta, tau and recompute chunk, both dtypes, for kd_fwd / kd_bwd; and random
k and support for the top-k paths. Each case is checked against the fp64
oracle with the tolerances of tests/helpers.py, every row."""
import numpy as np
import pytest

import kdsynth
from oracle import kd_oracle as O
from tests.helpers import assert_grad_rows, check_tail_rows, check_topk_rows, to_dev
from tests.test_gpu_fwd_bwd import run_case

pytestmark = pytest.mark.gpu


def _kd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_chunked_kl_amd as kd
    kd.load_library()
    return kd, torch


def _shape(rng, max_n=300, max_v=4000):
    N = int(rng.integers(1, max_n + 1))
    V = int(rng.integers(2, max_v + 1))
    ds = 8 * int(rng.integers(1, 41))
    dt = 8 * int(rng.integers(1, 41))
    return N, V, ds, dt


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_fwd_bwd(seed):
    kd, torch = _kd()
    rng = np.random.default_rng(1000 + seed)
    N, V, ds, dt = _shape(rng)
    dtype = "f32" if seed % 3 == 0 else "bf16"
    beta = float(rng.choice([0.0, 1.0, rng.uniform(0.05, 0.95)]))
    tau = float(rng.uniform(0.5, 3.0))
    chunk = 256 * int(rng.integers(1, 9))
    print(f"random fwd/bwd seed={seed} N={N} V={V} d_s={ds} d_t={dt} {dtype} beta={beta:.3f} tau={tau:.2f} "
          f"chunk={chunk}", flush=True)
    arrays = kdsynth.small_case(2000 + seed, N, V, ds, dt, dtype=dtype, logit_std=float(rng.uniform(1, 5)))
    grad = rng.uniform(-1, 2, size=N)
    run_case(kd, torch, arrays, beta, tau, grad=grad, chunk_V=chunk)


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_topk_and_tail(seed):
    kd, torch = _kd()
    rng = np.random.default_rng(3000 + seed)
    N, V, ds, dt = _shape(rng, max_n=200, max_v=70000 if seed % 2 else 3000)
    k = int(rng.integers(1, min(V, 64) + 1))
    tau = float(rng.uniform(0.7, 2.0))
    arrays = kdsynth.small_case(4000 + seed, N, V, ds, dt, logit_std=float(rng.uniform(1, 4)))
    labels = kdsynth.uniform_labels(5000 + seed, N, V, ignore_frac=0.2)
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int32)).cuda()
    rows = np.arange(N)
    print(f"random top-k seed={seed} N={N} V={V} d_s={ds} d_t={dt} k={k} tau={tau:.2f}", flush=True)
    out = kd.kd_topk_fwd(*dev, k, tau, labels=lab)
    torch.cuda.synchronize()
    exact, _ = check_topk_rows(out, *arrays, rows, k, tau, labels)
    assert exact >= 0.8 * N
    beta = float(rng.choice([0.0, 1.0, rng.uniform(0.05, 0.95)]))
    support = int(rng.choice([1, 2, 3, 5, 6, 7]))
    print(f"  tail beta={beta:.3f} support={support}", flush=True)
    tl = kd.kd_tail_fwd(*dev, k, beta, tau, support, labels=lab)
    torch.cuda.synchronize()
    exact, _ = check_tail_rows(tl, *arrays, rows, k, beta, tau, support, labels)
    assert exact >= 0.8 * N
    w = rng.uniform(-0.5, 1.5, N)
    dh = kd.kd_tail_bwd(dev[0], dev[1], tl, k, beta, tau, support,
                        grad_loss=torch.from_numpy(w.astype(np.float32)).cuda(), chunk_V=256 * int(rng.integers(1, 5)))
    torch.cuda.synchronize()
    ref = O.kd_tail_bwd(*arrays, k, beta, tau, grad_loss=w, sup=tl["sup_idx"].cpu().numpy())
    assert_grad_rows(dh.cpu().numpy(), ref, name="tail dh_s")
