"""GPU parity against the fp64 oracle for every start position of the two
contractions in the logit sweeps' stage ring.

A sweep tile is whole turns of its three-stage ring (four for the 64-token
tile). The student's contraction runs its ceil(d_s * size / 128) stages; when
that count is 1 modulo 3 the teacher's starts at ring position 1 and is padded
to the end of a turn; otherwise both are padded to whole turns. The top-k
sweep contracts the teacher first when its stage count is 1 modulo 3. Stages
past a contraction's K extent load nothing and add zeros. These cases take the
stage counts through every remainder (hidden sizes of 1, 2 and 3 stages, and
sizes with a K tail inside a stage), with ragged token and vocabulary tails,
and compare loss, log-sum-exps, aux and dL/dh_s (and the top-k selection and
terms) with the oracle at the usual tolerances (tests/helpers.py)."""
import numpy as np
import pytest

import kdsynth
from oracle import kd_oracle as O
from tests.helpers import assert_close, assert_grad_rows, check_tail_rows, check_topk_rows, to_dev

pytestmark = pytest.mark.gpu


def _kd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_chunked_kl_amd as kd
    kd.load_library()
    return kd, torch


def _fwd_bwd(kd, torch, arrays, beta, tau):
    dev = [to_dev(x) for x in arrays]
    loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, tau)
    dh = kd.kd_bwd(*dev, beta, tau, lse_s, lse_t, aux, chunk_V=1024)
    torch.cuda.synchronize()
    ref, dref = O.kd_fwd_bwd(*arrays, beta, tau)
    assert_close("loss", loss.cpu().numpy(), ref["loss"])
    assert_close("lse_s", lse_s.cpu().numpy(), ref["lse_s"])
    assert_close("lse_t", lse_t.cpu().numpy(), ref["lse_t"])
    assert_close("aux", aux.cpu().numpy(), ref["aux"])
    assert_grad_rows(dh.cpu().numpy(), dref)


# bf16: 64 values per 128-byte stage. (d_s, d_t) -> student stages mod 3 in
# {0, 1, 2} against teacher stages mod 3 in {0, 1, 2}, then K tails.
BF16_DIMS = [(ds, dt) for ds in (64, 128, 192) for dt in (64, 128, 192)] + [(72, 200), (200, 72), (136, 264)]


@pytest.mark.parametrize("ds,dt", BF16_DIMS)
@pytest.mark.parametrize("beta", [1.0, 0.5])
def test_ring_positions_bf16(ds, dt, beta):
    kd, torch = _kd()
    N, V = 200, 3000  # 2 token tiles (ragged), 12 vocabulary tiles (ragged)
    print(f"ring positions bf16 d_s={ds} d_t={dt} beta={beta}", flush=True)
    arrays = kdsynth.small_case(900 + ds + 7 * dt, N, V, ds, dt)
    _fwd_bwd(kd, torch, arrays, beta, 1.5)


@pytest.mark.parametrize("ds,dt", [(32, 96), (64, 32), (40, 72)])
def test_ring_positions_fp32(ds, dt):
    kd, torch = _kd()
    N, V = 130, 1500  # fp32: 32 values per stage
    print(f"ring positions fp32 d_s={ds} d_t={dt}", flush=True)
    arrays = kdsynth.small_case(950 + ds + 7 * dt, N, V, ds, dt, dtype="f32")
    _fwd_bwd(kd, torch, arrays, 1.0, 1.0)


@pytest.mark.parametrize("ds,dt", [(64, 192), (128, 64), (192, 320)])
def test_ring_positions_small_token_tile(ds, dt):
    kd, torch = _kd()
    N, V = 50, 2600  # the 64-token tile and its four-stage ring
    print(f"ring positions 64-token tile d_s={ds} d_t={dt}", flush=True)
    arrays = kdsynth.small_case(970 + ds + 7 * dt, N, V, ds, dt)
    _fwd_bwd(kd, torch, arrays, 0.5, 1.0)


@pytest.mark.parametrize("ds,dt", [(128, 64), (64, 128), (192, 256), (128, 320)])
def test_ring_positions_topk(ds, dt):
    kd, torch = _kd()
    N, V, k = 150, 4000, 8
    print(f"ring positions top-k d_s={ds} d_t={dt}", flush=True)
    arrays = kdsynth.small_case(990 + ds + 7 * dt, N, V, ds, dt)
    labels = kdsynth.uniform_labels(991, N, V, ignore_frac=0.2)
    dev = [to_dev(x) for x in arrays]
    lab = torch.from_numpy(labels.astype(np.int32)).cuda()
    out = kd.kd_topk_fwd(*dev, k, 1.0, labels=lab)
    torch.cuda.synchronize()
    exact, flagged = check_topk_rows(out, *arrays, np.arange(N), k, 1.0, labels)
    assert exact >= 0.9 * N


@pytest.mark.parametrize("ds,dt", [(64, 128), (128, 64)])
def test_ring_positions_tail_student_ranked(ds, dt):
    """The student-ranked sweep exchanges the two operand pairs, so the pair
    contracted first is then the student's."""
    kd, torch = _kd()
    N, V, k = 150, 4000, 8
    print(f"ring positions tail (student ranked) d_s={ds} d_t={dt}", flush=True)
    arrays = kdsynth.small_case(995 + ds + 7 * dt, N, V, ds, dt)
    dev = [to_dev(x) for x in arrays]
    sup = kd.KD_SUPPORT_STUDENT
    out = kd.kd_tail_fwd(*dev, k, 1.0, 1.0, sup)
    torch.cuda.synchronize()
    exact, flagged = check_tail_rows(out, *arrays, np.arange(N), k, 1.0, 1.0, sup)
    assert exact >= 0.9 * N
