"""kd_fwd_noalloc (the forward with no workspace and no allocation: its
partial records live in the library's fixed per-GPU scratch array) against
kd_fwd with a caller workspace, through the C ABI: bit for bit on two calls in
a row, the second with a smaller input (the array keeps the first call's
contents), and against the fp64 oracle. A shape whose forward workspace
exceeds the array is refused on the host."""
import numpy as np
import pytest

import kdsynth
from oracle import kd_oracle as O
from tests.helpers import assert_close, to_dev

pytestmark = pytest.mark.gpu


def _kd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_chunked_kl_amd as kd
    kd.load_library()
    return kd, torch


@pytest.mark.parametrize("beta", [1.0, 0.5, 0.0])
def test_noalloc_forward_matches_kd_fwd_twice(beta):
    kd, torch = _kd()
    cases = ((700, 30000, 256, 384, 1.3), (130, 5000, 64, 128, 0.9))  # the second smaller
    for seed, (N, V, ds, dt, tau) in enumerate(cases):
        print(f"noalloc N={N} V={V} d_s={ds} d_t={dt} beta={beta} tau={tau}", flush=True)
        arrays = kdsynth.small_case(300 + seed, N, V, ds, dt)
        dev = [to_dev(x) for x in arrays]
        ref = kd.kd_fwd(*dev, beta, tau)
        got = kd.kd_fwd_noalloc(*dev, beta, tau)
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "lse_s", "lse_t", "aux"), got, ref):
            if name == "aux" and beta == 0.0:
                continue
            assert torch.equal(a, b), name
        want = O.kd_fwd(*arrays, beta, tau)
        assert_close("loss", got[0].cpu().numpy(), want["loss"])
        assert_close("lse_s", got[1].cpu().numpy(), want["lse_s"])


def test_noalloc_forward_refuses_a_shape_above_its_scratch():
    kd, torch = _kd()
    lib = kd.load_library()
    cap = int(lib.kd_fwd_noalloc_max_scratch())
    assert cap == 144 << 20
    # 40000 tokens over 262144 entries: 256 splits of 5 records -> 205 MB of partial records
    N, V = 40000, 262144
    need = kd.workspace_size(kd.KD_OP_FWD, N, V, 64, 64, kd.KD_BF16, beta=1.0)
    assert need > cap
    fake = 1 << 20  # never dereferenced: the size check runs on the host first
    assert lib.kd_fwd_noalloc(fake, fake, fake, fake, N, V, 64, 64, 1.0, 1.0, kd.KD_BF16, fake, fake, fake, fake,
                              None) == kd.KD_ERR_WORKSPACE
    assert b"kd_fwd_noalloc" in lib.kd_last_error()
