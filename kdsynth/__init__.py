"""Seeded synthetic inputs for the chunked-KL distillation workloads.

This module only draws numbers: Gaussian hidden states and unembeddings,
label vectors and row subsets, rounded to bf16 where a workload asks for bf16.
It holds none of the divergence arithmetic, so both the fp64 oracle (through
the tests) and the GPU path (through the tests and the benchmark) can take
their inputs from here without sharing any of the method's code.

Workload shapes follow the distillation settings the source pages discuss
(Qwen-sized student/teacher pairs at a ~152k vocabulary, a 248,320-entry
vocabulary for the top-k variant). Every tensor is drawn from numpy's PCG64
in fixed-size blocks whose seeds are spawned from ``SeedSequence(1000 + cfg)``,
so the bits do not depend on the number of threads used to draw them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_BLOCK = 1 << 22  # elements per independently seeded block


# ---------------------------------------------------------------------------
# bit-level helpers (storage format only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the
    16-bit patterns as uint16. Inputs here are finite Gaussian draws."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: np.random.SeedSequence, shape, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) float32 array of ``shape``, drawn block by block.

    Block b of the flattened array uses the b-th child of ``seed``; the result
    is identical for any thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nblk = (n + _BLOCK - 1) // _BLOCK
    children = seed.spawn(nblk)

    def work(b):
        lo = b * _BLOCK
        hi = min(n, lo + _BLOCK)
        g = np.random.Generator(np.random.PCG64(children[b]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if scale != 1.0:
            out[lo:hi] *= np.float32(scale)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass
class Workload:
    """One synthetic distillation batch.

    ``h_s [N,d_s]``, ``W_s [V,d_s]``, ``h_t [N,d_t]``, ``W_t [V,d_t]`` are
    row-major; for ``dtype == "bf16"`` they hold uint16 bf16 bit patterns,
    for ``"f32"`` float32 values. ``labels`` (int32 [N]) is set for the top-k
    workloads only."""

    name: str
    dtype: str
    N: int
    V: int
    d_s: int
    d_t: int
    tau: float
    betas: tuple
    h_s: np.ndarray
    W_s: np.ndarray
    h_t: np.ndarray
    W_t: np.ndarray
    labels: np.ndarray | None = None
    k: int | None = None
    meta: dict = field(default_factory=dict)


# Shapes of the five workloads (tokens N, vocab V, hidden sizes d_s/d_t).
SHAPES = {
    1: dict(name="tiny_rkl_f32", dtype="f32", N=64, V=1000, d_s=64, d_t=64, tau=1.0, betas=(1.0,)),
    2: dict(name="rkl_v152k_n4k", dtype="bf16", N=4096, V=151936, d_s=1024, d_t=2560, tau=1.0, betas=(1.0,)),
    3: dict(name="jsd_sweep_v152k_n32k", dtype="bf16", N=32768, V=151936, d_s=2560, d_t=4096, tau=2.0,
            betas=(0.0, 0.5, 1.0)),
    4: dict(name="rkl_v248k_heavyhead", dtype="bf16", N=8192, V=248320, d_s=5120, d_t=5120, tau=1.0, betas=(1.0,)),
    5: dict(name="topk64_v248k", dtype="bf16", N=16384, V=248320, d_s=2048, d_t=5120, tau=1.0, betas=(), k=64),
}

HEAVY_ROWS = 10  # vocabulary rows scaled x4 in the heavy-head workload
HEAVY_SCALE = 4.0
SVD_RANK = 256


def _seeds(cfg: int, n: int):
    return np.random.SeedSequence(1000 + cfg).spawn(n)


def _unembed_scale(d: int) -> float:
    # rows ~ N(0, 0.02^2), then rescaled so that with h ~ N(0,1) the logit
    # standard deviation is ~3:  net std = 0.02 * 3 / (0.02 * sqrt(d)).
    return 0.02 * (3.0 / (0.02 * np.sqrt(d)))


def make(cfg: int, N: int | None = None, V: int | None = None, d_s: int | None = None,
         d_t: int | None = None) -> Workload:
    """Build workload ``cfg`` (1..5). ``N``/``V``/``d_s``/``d_t`` override the
    shape (same recipe, fewer tokens or a smaller vocabulary) for tests."""
    sh = dict(SHAPES[cfg])
    for key, val in (("N", N), ("V", V), ("d_s", d_s), ("d_t", d_t)):
        if val is not None:
            sh[key] = int(val)
    n_, v_, ds, dt = sh["N"], sh["V"], sh["d_s"], sh["d_t"]
    seeds = _seeds(cfg, 8)
    meta = {}
    labels = None
    if cfg == 1:
        h_s = normal_f32(seeds[0], (n_, ds))
        W_s = normal_f32(seeds[1], (v_, ds), 1.0 / np.sqrt(ds))
        h_t = normal_f32(seeds[2], (n_, dt))
        W_t = normal_f32(seeds[3], (v_, dt), 1.0 / np.sqrt(dt))
        out = (h_s, W_s, h_t, W_t)
    elif cfg in (2, 4, 5):
        h_s = normal_f32(seeds[0], (n_, ds))
        W_s = normal_f32(seeds[1], (v_, ds), _unembed_scale(ds))
        h_t = normal_f32(seeds[2], (n_, dt))
        W_t = normal_f32(seeds[3], (v_, dt), _unembed_scale(dt))
        if cfg == 4:
            g = np.random.Generator(np.random.PCG64(seeds[4]))
            rows = np.sort(g.choice(v_, size=min(HEAVY_ROWS, v_), replace=False))
            W_s[rows] *= np.float32(HEAVY_SCALE)
            W_t[rows] *= np.float32(HEAVY_SCALE)
            meta["heavy_rows"] = rows
        if cfg == 5:
            g = np.random.Generator(np.random.PCG64(seeds[5]))
            labels = g.integers(0, v_, size=n_, dtype=np.int64).astype(np.int32)
        out = (h_s, W_s, h_t, W_t)
    elif cfg == 3:
        # Teacher overlaps the student: it sees the student's hidden state plus
        # extra features, and its unembedding is the student's padded with
        # zeros plus half-scale independent noise.
        if dt < ds:
            raise ValueError("workload 3 needs d_t >= d_s")
        sig = _unembed_scale(ds)
        h_s = normal_f32(seeds[0], (n_, ds))
        W_s = normal_f32(seeds[1], (v_, ds), sig)
        h_x = normal_f32(seeds[2], (n_, dt - ds))
        h_t = np.concatenate([h_s, h_x], axis=1)
        noise = normal_f32(seeds[3], (v_, dt), 0.5 * sig)
        W_t = noise
        W_t[:, :ds] += W_s
        out = (h_s, W_s, h_t, W_t)
    else:
        raise ValueError(f"unknown workload {cfg}")

    if sh["dtype"] == "bf16":
        out = tuple(f32_to_bf16_bits(x) for x in out)
    return Workload(name=sh["name"], dtype=sh["dtype"], N=n_, V=v_, d_s=ds, d_t=dt, tau=sh["tau"],
                    betas=tuple(sh["betas"]), h_s=out[0], W_s=out[1], h_t=out[2], W_t=out[3],
                    labels=labels, k=sh.get("k"), meta=meta)


def sample_rows(N: int, count: int, seed: int = 7, must=()) -> np.ndarray:
    """A sorted, seeded subset of about ``count`` token rows that always
    contains the first and last row and the rows listed in ``must``."""
    if count >= N:
        return np.arange(N)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    base = {0, N - 1, *[int(m) for m in must if 0 <= int(m) < N]}
    rows = set(base)
    for e in g.permutation(N):
        if len(rows) >= max(count, len(base)):
            break
        rows.add(int(e))
    return np.array(sorted(rows), dtype=np.int64)


def small_case(seed: int, N: int, V: int, d_s: int, d_t: int, dtype: str = "bf16", logit_std: float = 3.0,
               overlap: float = 0.0):
    """A small random case (Gaussian h, unembedding scaled for ``logit_std``).

    ``overlap`` in [0,1) mixes the student's logits into the teacher's when
    ``d_s == d_t``: W_t = overlap * W_s + sqrt(1 - overlap^2) * noise and the
    teacher reuses the student's hidden state. Returns (h_s, W_s, h_t, W_t)."""
    ss = np.random.SeedSequence(seed).spawn(4)
    h_s = normal_f32(ss[0], (N, d_s))
    W_s = normal_f32(ss[1], (V, d_s), logit_std / np.sqrt(d_s))
    if overlap > 0.0:
        if d_s != d_t:
            raise ValueError("overlap needs d_s == d_t")
        h_t = h_s.copy()
        W_t = np.float32(overlap) * W_s + np.float32(np.sqrt(1 - overlap ** 2)) * normal_f32(
            ss[3], (V, d_t), logit_std / np.sqrt(d_t))
    else:
        h_t = normal_f32(ss[2], (N, d_t))
        W_t = normal_f32(ss[3], (V, d_t), logit_std / np.sqrt(d_t))
    out = (h_s, W_s, h_t, W_t)
    if dtype == "bf16":
        out = tuple(f32_to_bf16_bits(x) for x in out)
    return out


def uniform_labels(seed: int, N: int, V: int, ignore_frac: float = 0.0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    lab = g.integers(0, V, size=N, dtype=np.int64).astype(np.int32)
    if ignore_frac > 0:
        lab[g.random(N) < ignore_frac] = -100
    return lab
