"""The C-ABI library loads, exports every symbol include/kd.h declares, and
rejects bad arguments on the host before any HIP call (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "vocab_chunked_kl_amd", "libkd.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkd.so not built (run __graft_entry__.build())")


def header_symbols():
    text = open(os.path.join(ROOT, "include", "kd.h")).read()
    return sorted(set(re.findall(r"^(?:kd_status|const char\*|int32_t|size_t)\s+(kd_\w+)\s*\(", text, flags=re.M)))


def _chunk_buffers(kd, n, v, d, cv):
    """The backward's per-chunk buffers (kd_bwd's size without its
    dominant-entry correction), which the top-k and tail backward share."""
    al = lambda x: -(-x // 256) * 256  # noqa: E731
    return kd.workspace_size(kd.KD_OP_BWD, n, v, d, d, kd.KD_BF16, chunk_V=cv) - al((cv // 256) * n * 4) - 2 * al(n * 4)


def test_header_symbols_exported():
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()
    names = header_symbols()
    assert set(names) == set(kd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()
    assert lib.kd_status_string(0) == b"KD_OK"
    assert lib.kd_status_string(3) == b"KD_ERR_WORKSPACE"


def test_workspace_sizes():
    import vocab_chunked_kl_amd as kd
    # backward workspace = one bf16 gradient chunk [N, chunk_V] + one transposed W_s chunk [d_s, chunk_V]
    N, V, ds, dt = 32768, 151936, 2560, 4096
    for cv in (2048, 8192):
        b = kd.workspace_size(kd.KD_OP_BWD, N, V, ds, dt, kd.KD_BF16, chunk_V=cv)
        # G chunk, W_s chunk transposed, then the dominant-entry correction's
        # per-split sums of one chunk, their total and the index, per token
        assert b == N * cv * 2 + ds * cv * 2 + (cv // 256) * N * 4 + 2 * N * 4
        # with dW_s: plus the chunk transposed [chunk_V, Np] and h_s transposed [d_s, Np],
        # Np = N rounded up to the 128-token tile
        for n in (N, 300):
            np_ = -(-n // 128) * 128
            al = lambda x: -(-x // 256) * 256  # noqa: E731
            bw = kd.workspace_size(kd.KD_OP_BWD_W, n, V, ds, dt, kd.KD_BF16, chunk_V=cv)
            b0 = kd.workspace_size(kd.KD_OP_BWD, n, V, ds, dt, kd.KD_BF16, chunk_V=cv)
            assert bw == b0 + al(cv * np_ * 2) + al(ds * np_ * 2)
    f1 = kd.workspace_size(kd.KD_OP_FWD, N, V, ds, dt, kd.KD_BF16, beta=1.0)
    f5 = kd.workspace_size(kd.KD_OP_FWD, N, V, ds, dt, kd.KD_BF16, beta=0.5)
    # forward: one partial record (5 floats; +2 for the JSD sums) per token per
    # 1024-entry vocabulary slice
    S = -(-(-(-V // 256)) // 4)
    al = lambda x: -(-x // 256) * 256  # noqa: E731
    assert f1 == al(5 * S * N * 4) and f5 == f1 + al(2 * S * N * 4)
    # up to 4 token tiles: the slice width minimising (waves of workgroups on 256 CUs) x (tiles + 1.5);
    # from 5 token tiles on, 4 tiles
    tiles = -(-V // 256)
    for n, want_tps in ((64, 3), (256, 5), (512, 5), (640, 4), (1024, 4)):
        T = -(-n // 128)
        if T <= 4:
            cost = {t: (-(-(T * -(-tiles // t)) // 256)) * (t + 1.5) for t in range(1, 9)}
            assert min(cost, key=lambda t: (cost[t], t)) == want_tps
        S_n = -(-tiles // want_tps)
        assert kd.workspace_size(kd.KD_OP_FWD, n, V, ds, dt, kd.KD_BF16, beta=1.0) == al(5 * S_n * n * 4), n
    # few tokens: the dh GEMM splits its contraction into s = min(ceil(256 / output tiles), chunk_V / 512)
    # partial tiles of N x d_s fp32 (output tiles of 256 x 256; none from 128 tiles on)
    for n, d, cv, s in ((64, 1024, 16384, 32), (4096, 1024, 16384, 4), (300, 64, 2048, 4), (64, 1024, 256, 1),
                        (32768, 2560, 16384, 1)):
        base = al(n * cv * 2) + al(d * cv * 2)
        want = base + (al(s * n * d * 4) if s > 1 else 0)
        # kd_bwd's dominant-entry correction: per-split sums of one chunk, their total, the index
        want += al((cv // 256) * n * 4) + 2 * al(n * 4)
        assert kd.workspace_size(kd.KD_OP_BWD, n, V, d, dt, kd.KD_BF16, chunk_V=cv) == want, (n, d, cv)
    # the forward keeps at most 256 partial records of 5 (+2 for 0 < beta < 1) floats per
    # token, whatever the vocabulary: O(N), within the backward's O(N chunk_V)
    for n, v in ((64, 151936), (32768, 151936), (8192, 248320), (4096, 1 << 20), (100, 3 << 20)):
        for beta in (1.0, 0.5):
            got = kd.workspace_size(kd.KD_OP_FWD, n, v, ds, dt, kd.KD_BF16, beta=beta)
            cap = al(5 * 256 * n * 4) + (al(2 * 256 * n * 4) if beta == 0.5 else 0)
            assert got <= cap, (n, v, got, cap)
            assert got <= n * kd.default_chunk(n, v) * 2 + 512, (n, v)
    with pytest.raises(kd.KDError):
        kd.workspace_size(kd.KD_OP_BWD, N, V, ds, dt, kd.KD_BF16, chunk_V=1000)
    with pytest.raises(kd.KDError):
        kd.workspace_size(kd.KD_OP_FWD, N, V, ds, dt, kd.KD_BF16, beta=1.5)
    with pytest.raises(kd.KDError):
        kd.workspace_size(kd.KD_OP_TOPK, N, V, ds, dt, kd.KD_BF16, k=0)


def test_default_chunk():
    import vocab_chunked_kl_amd as kd
    # the [N, chunk] gradient tile stays within 1 GiB; the vocabulary (rounded up to 256) is cut into the
    # fewest equal chunks under that bound, each rounded up to 256, never below 2048 unless V is smaller
    cases = [
        (32768, 151936, kd.KD_BF16, 15360),  # 16384 allowed: 10 chunks of 15207 -> 15360
        (4096, 151936, kd.KD_BF16, 76032),   # 131072 allowed: 2 chunks
        (64, 151936, kd.KD_BF16, 152064),    # the whole (padded) vocabulary
        (8192, 248320, kd.KD_BF16, 62208),   # 65536 allowed: 4 chunks of 62080 -> 62208
        (1 << 22, 151936, kd.KD_BF16, 2048),  # the bound would give 128: the 2048 floor
        (10, 1000, kd.KD_F32, 1024),         # a small vocabulary is one chunk
        (32768, 151936, kd.KD_F32, 8192),    # fp32: 8192 allowed, 19 chunks of 8004 -> 8192
        (0, 151936, kd.KD_BF16, 152064),
    ]
    for n, v, dt, want in cases:
        assert kd.default_chunk(n, v, dt) == want, (n, v, dt)
        assert (n or 1) * want * (2 if dt == kd.KD_BF16 else 4) <= (1 << 30) or want == 2048 or want >= v
    assert kd.default_chunk(-1, 100) == 0 and kd.default_chunk(8, 0) == 0 and kd.default_chunk(8, 100, 7) == 0
    # chunk_V = 0 sizes every backward op's workspace for the default chunk
    for n, v in ((64, 151936), (4096, 151936), (3000, 50000)):
        c = kd.default_chunk(n, v)
        for op in (kd.KD_OP_BWD, kd.KD_OP_BWD_W, kd.KD_OP_TOPK_BWD, kd.KD_OP_TAIL_BWD):
            assert kd.workspace_size(op, n, v, 1024, 2048, kd.KD_BF16, chunk_V=0, k=16) == \
                kd.workspace_size(op, n, v, 1024, 2048, kd.KD_BF16, chunk_V=c, k=16), (n, v, op)
    with pytest.raises(kd.KDError):
        kd.workspace_size(kd.KD_OP_BWD, 64, 1000, 64, 64, kd.KD_BF16, chunk_V=-256)


FAKE = 0x10000  # aligned non-null address: never dereferenced, every call below fails validation first


def call_fwd(lib, **kw):
    a = dict(h_s=FAKE, W_s=FAKE, h_t=FAKE, W_t=FAKE, N=8, V=100, d_s=64, d_t=64, beta=1.0, tau=1.0, dtype=1,
             loss=FAKE, lse_s=FAKE, lse_t=FAKE, aux=FAKE, ws=FAKE, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.kd_fwd(*[a[k] for k in ("h_s", "W_s", "h_t", "W_t", "N", "V", "d_s", "d_t", "beta", "tau", "dtype",
                                       "loss", "lse_s", "lse_t", "aux", "ws", "ws_bytes", "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(h_s=None), 1), (dict(N=0), 1), (dict(V=1), 1), (dict(beta=1.5), 1), (dict(beta=-0.1), 1),
    (dict(tau=0.0), 1), (dict(tau=float("nan")), 1), (dict(d_s=60), 2), (dict(dtype=7), 2),
    (dict(W_t=FAKE + 2), 2), (dict(loss=None), 1), (dict(aux=None, beta=0.5), 1), (dict(ws_bytes=10), 3),
    (dict(ws=None, ws_bytes=1 << 30), 3),
])
def test_fwd_validation(kw, code):
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()
    assert call_fwd(lib, **kw) == code


def test_bwd_and_topk_validation():
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()
    args = [FAKE, FAKE, FAKE, FAKE, 8, 100, 64, 64, 1.0, 1.0, 1]
    # chunk_V not a multiple of 256, or so large that a 256-row tile of it passes 2 GiB
    assert lib.kd_bwd(*args, 300, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40, None) == 1
    assert lib.kd_bwd(*args, 1 << 22, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40, None) == 2
    # workspace too small
    assert lib.kd_bwd(*args, 256, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 16, None) == 3
    # neither dh nor dW
    assert lib.kd_bwd(*args, 256, FAKE, FAKE, FAKE, None, None, None, FAKE, 1 << 40, None) == 1
    # dW with only the dh-sized workspace
    bws = kd.workspace_size(kd.KD_OP_BWD, 8, 100, 64, 64, kd.KD_BF16, chunk_V=256)
    assert lib.kd_bwd(*args, 256, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, bws, None) == 3
    assert lib.kd_bwd(*args, 256, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, bws, None) == 3
    # dW with more tokens than the token-contracted GEMM's 32-bit tile offsets allow
    many = [FAKE, FAKE, FAKE, FAKE, 1 << 23, 100, 64, 64, 1.0, 1.0, 1]
    assert lib.kd_bwd(*many, 256, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == 2
    # misaligned dW
    assert lib.kd_bwd(*args, 256, FAKE, FAKE, FAKE, None, FAKE, FAKE + 2, FAKE, 1 << 40, None) == 2
    targs = [FAKE, FAKE, FAKE, FAKE, 8, 100, 64, 64]
    outs = [FAKE] * 11
    # k out of range, fp32 inputs, labels without ce
    assert lib.kd_topk_fwd(*targs, 0, 1.0, 1, None, *outs, FAKE, 1 << 40, None) == 1
    assert lib.kd_topk_fwd(*targs, 200, 1.0, 1, None, *outs, FAKE, 1 << 40, None) == 1
    # vocabulary above the top-k limit
    big = [FAKE, FAKE, FAKE, FAKE, 8, kd.KD_TOPK_MAX_V + 1, 64, 64]
    assert lib.kd_topk_fwd(*big, 8, 1.0, 1, None, *outs, FAKE, 1 << 40, None) == 2
    assert lib.kd_topk_fwd(*targs, 8, 1.0, 0, None, *outs, FAKE, 1 << 40, None) == 2
    o = list(outs)
    o[5] = None  # ce
    assert lib.kd_topk_fwd(*targs, 8, 1.0, 1, FAKE, *o, FAKE, 1 << 40, None) == 1


def test_topk_bwd_validation():
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()

    def call(**kw):
        a = dict(h_s=FAKE, W_s=FAKE, N=8, V=100, d_s=64, k=8, tau=1.0, dtype=1, labels=None, idx=FAKE, val=FAKE,
                 val_s=FAKE, p_mass=FAKE, q_mass=FAKE, lse_s=FAKE, lse_s1=FAKE, gb=FAKE, gc=FAKE, ge=None,
                 chunk=256, dh=FAKE, ws=FAKE, ws_bytes=1 << 40, stream=None)
        a.update(kw)
        return lib.kd_topk_bwd(*[a[n] for n in ("h_s", "W_s", "N", "V", "d_s", "k", "tau", "dtype", "labels", "idx",
                                                "val", "val_s", "p_mass", "q_mass", "lse_s", "lse_s1", "gb", "gc",
                                                "ge", "chunk", "dh", "ws", "ws_bytes", "stream")])
    assert call(dtype=0) == 2                    # bf16 only
    assert call(k=0) == 1 and call(k=101) == 1   # k outside [1, min(V, 64)]
    assert call(val_s=None) == 1                 # needs the forward's selected logits
    assert call(ge=FAKE, labels=FAKE, lse_s1=None) == 1  # CE gradient needs the untempered LSE
    assert call(dh=FAKE + 4) == 2                # dh_s must be 16-byte aligned
    assert call(chunk=300) == 1
    assert call(tau=0.0) == 1
    need = kd.workspace_size(kd.KD_OP_TOPK_BWD, 8, 100, 64, 64, kd.KD_BF16, chunk_V=256, k=8)
    al = lambda x: -(-x // 256) * 256  # noqa: E731
    # chunk buffers + two per-token coefficients + the (k + 1)-entry list's indices and values
    assert need == _chunk_buffers(kd, 8, 100, 64, 256) + 2 * al(8 * 4) + 2 * al(8 * 9 * 4)
    assert call(ws_bytes=need - 1) == 3


def test_gather_scatter_validation():
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()
    # n_rows = 0 is a no-op even with null pointers; bad sizes / pointers fail before any launch
    assert lib.kd_gather_rows(None, 10, 64, None, 0, None, None) == 0
    assert lib.kd_scatter_rows(None, 0, 64, None, None, 10, None) == 0
    assert lib.kd_gather_rows(FAKE, 10, 64, None, 4, FAKE, None) == 1
    assert lib.kd_gather_rows(FAKE, 10, 62, FAKE, 4, FAKE, None) == 1
    assert lib.kd_gather_rows(FAKE, -1, 64, FAKE, 4, FAKE, None) == 1
    assert lib.kd_scatter_rows(FAKE, 4, 0, FAKE, FAKE, 10, None) == 1
    assert lib.kd_scatter_rows(FAKE + 2, 4, 64, FAKE, FAKE, 10, None) == 2


def test_tail_validation_and_workspace():
    import vocab_chunked_kl_amd as kd
    lib = kd.load_library()
    al = lambda x: -(-x // 256) * 256  # noqa: E731
    N, V = 300, 151936
    S = -(-V // 65536)
    # LSE partials (6 floats per token per 65536-entry split) + one list area per ranked model
    assert kd.workspace_size(kd.KD_OP_TAIL, N, V, 64, 64, kd.KD_BF16, k=16) == \
        al(6 * S * N * 4) + 2 * al(S * N * 16 * 4)
    # chunk buffers + one per-token coefficient + values for the largest support (2k + 1)
    assert kd.workspace_size(kd.KD_OP_TAIL_BWD, N, V, 64, 64, kd.KD_BF16, chunk_V=256, k=16) == \
        _chunk_buffers(kd, N, V, 64, 256) + al(N * 4) + al(N * 33 * 4)

    def fwd(**kw):
        a = dict(h_s=FAKE, W_s=FAKE, h_t=FAKE, W_t=FAKE, N=8, V=100, d_s=64, d_t=64, k=4, support=1, beta=0.0,
                 tau=1.0, dtype=1, labels=None, sup_idx=FAKE, sup_t=FAKE, sup_s=FAKE, loss=FAKE, p_mass=None,
                 q_mass=None, lse_s=FAKE, lse_t=FAKE, ws=FAKE, ws_bytes=1 << 40, stream=None)
        a.update(kw)
        return lib.kd_tail_fwd(*[a[n] for n in ("h_s", "W_s", "h_t", "W_t", "N", "V", "d_s", "d_t", "k", "support",
                                                "beta", "tau", "dtype", "labels", "sup_idx", "sup_t", "sup_s", "loss",
                                                "p_mass", "q_mass", "lse_s", "lse_t", "ws", "ws_bytes", "stream")])
    assert fwd(dtype=0) == 2
    assert fwd(k=0) == 1 and fwd(k=65) == 1 and fwd(k=101, V=100) == 1
    assert fwd(support=0) == 1 and fwd(support=4, labels=FAKE) == 1 and fwd(support=8) == 1
    assert fwd(support=5) == 1                   # the label bit needs labels
    assert fwd(beta=1.5) == 1 and fwd(tau=-1.0) == 1
    assert fwd(V=kd.KD_TOPK_MAX_V + 1) == 2
    assert fwd(sup_s=None) == 1 and fwd(loss=None) == 1
    need = kd.workspace_size(kd.KD_OP_TAIL, 8, 100, 64, 64, kd.KD_BF16, k=4)
    assert fwd(ws_bytes=need - 1) == 3

    def bwd(**kw):
        a = dict(h_s=FAKE, W_s=FAKE, N=8, V=100, d_s=64, k=4, support=2, beta=1.0, tau=1.0, dtype=1, sup_idx=FAKE,
                 sup_t=FAKE, sup_s=FAKE, lse_s=FAKE, lse_t=FAKE, grad=None, chunk=256, dh=FAKE, ws=FAKE,
                 ws_bytes=1 << 40, stream=None)
        a.update(kw)
        return lib.kd_tail_bwd(*[a[n] for n in ("h_s", "W_s", "N", "V", "d_s", "k", "support", "beta", "tau", "dtype",
                                                "sup_idx", "sup_t", "sup_s", "lse_s", "lse_t", "grad", "chunk", "dh",
                                                "ws", "ws_bytes", "stream")])
    assert bwd(dtype=0) == 2
    assert bwd(support=4) == 1 and bwd(k=0) == 1
    assert bwd(lse_t=None) == 1 and bwd(sup_idx=None) == 1
    assert bwd(dh=FAKE + 4) == 2
    assert bwd(chunk=100) == 1 and bwd(chunk=1 << 22) == 2
    need = kd.workspace_size(kd.KD_OP_TAIL_BWD, 8, 100, 64, 64, kd.KD_BF16, chunk_V=256, k=4)
    assert bwd(ws_bytes=need - 1) == 3
