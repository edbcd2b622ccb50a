"""Host checks of the seeded input generator (CPU)."""
import numpy as np

import kdsynth


def test_blocks_are_thread_count_independent(monkeypatch):
    ss = np.random.SeedSequence(123)
    a = kdsynth.normal_f32(ss, (3, kdsynth._BLOCK + 77), 0.5)
    monkeypatch.setattr(kdsynth, "_threads", lambda: 1)
    b = kdsynth.normal_f32(np.random.SeedSequence(123), (3, kdsynth._BLOCK + 77), 0.5)
    assert np.array_equal(a, b)


def test_bf16_storage_round_trip():
    x = np.array([1.0, 1.0 + 2 ** -8, -3.5, 1e-3], dtype=np.float32)
    bits = kdsynth.f32_to_bf16_bits(x)
    back = kdsynth.bf16_bits_to_f32(bits)
    assert back.tolist()[0] == 1.0 and back.tolist()[1] == 1.0 and back.tolist()[2] == -3.5
    assert abs(back[3] - 1e-3) < 1e-5


def test_workload_recipes_small():
    w = kdsynth.make(2, N=64, V=512)
    assert w.h_s.dtype == np.uint16 and w.W_s.shape == (512, 1024) and w.W_t.shape == (512, 2560)
    z = kdsynth.bf16_bits_to_f32(w.h_s).astype(np.float64) @ kdsynth.bf16_bits_to_f32(w.W_s).astype(np.float64).T
    assert 2.5 < z.std() < 3.5  # logit std ~3
    w3 = kdsynth.make(3, N=64, V=512)
    hs = kdsynth.bf16_bits_to_f32(w3.h_s)
    ht = kdsynth.bf16_bits_to_f32(w3.h_t)
    assert np.array_equal(ht[:, :2560], hs)
    zs = hs.astype(np.float64) @ kdsynth.bf16_bits_to_f32(w3.W_s).astype(np.float64).T
    zt = ht.astype(np.float64) @ kdsynth.bf16_bits_to_f32(w3.W_t).astype(np.float64).T
    c = np.corrcoef(zs.ravel(), zt.ravel())[0, 1]
    assert 0.75 < c < 0.92  # partial overlap (~0.85)
    w4 = kdsynth.make(4, N=16, V=4096, d_s=256, d_t=256)
    assert len(w4.meta["heavy_rows"]) == 10
    w5 = kdsynth.make(5, N=32, V=1000, d_s=64, d_t=128)
    assert w5.labels.min() >= 0 and w5.labels.max() < 1000 and w5.k == 64
    w1 = kdsynth.make(1)
    assert w1.h_s.dtype == np.float32 and w1.W_s.shape == (1000, 64)


def test_sample_rows_contains_ends():
    r = kdsynth.sample_rows(1000, 50, must=[500])
    assert r[0] == 0 and r[-1] == 999 and 500 in r and len(set(r)) == len(r)
