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
    return (not bad.any()), float(np.max(err / lim)) if err.size else 0.0, np.nonzero(bad)[0][:8]


def assert_close(name, gpu, ref, rtol=RTOL, atol=ATOL):
    ok, worst, where = close(gpu, ref, rtol, atol)
    assert ok, f"{name}: worst err/limit {worst:.3g} at rows {where.tolist()} gpu={np.asarray(gpu)[where][:4]} ref={np.asarray(ref)[where][:4]}"


U32 = 2.0 ** -24  # unit roundoff of fp32


def grad_floor(lse_s, lse_t, loss, W_s, tau):
    """Per-row absolute floor below which an fp32 evaluation of dL/dh_s cannot
    be resolved: the gradient term of a saturated entry is a difference of
    O(|L_s| + |L_t| + |KL|) quantities, each carrying fp32 rounding of relative
    size 2^-24, and enters dh_s scaled by a W_s row and 1/tau. Eight roundings
    are allowed for. Rows whose exact gradient is below the floor are compared
    absolutely (|gpu - ref| <= floor)."""
    from oracle import kd_oracle as O
    wmax = 0.0
    for v0 in range(0, W_s.shape[0], 16384):
        w = O.as_f64(W_s[v0:v0 + 16384])
        wmax = max(wmax, float(np.sqrt(np.max(np.sum(w * w, axis=1)))))
    return 8 * U32 * (2 * np.abs(lse_s) + 2 * np.abs(lse_t) + np.abs(loss)) * wmax / tau


def assert_grad_rows(gpu, ref, name="dh_s", floor=None):
    """Per row: cosine >= COS_MIN and max|d|/max|ref| <= MAXREL; rows whose
    reference norm is below ``floor`` (see grad_floor) must instead agree to
    within the floor. The cosine over all rows together must also hold."""
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
