"""Fused chunked-KL logit distillation on MI355X (gfx950).

Full-vocabulary distillation divergences computed straight from the student's
and teacher's final hidden states: the logits z = h W^T are rebuilt one
vocabulary tile at a time inside HIP kernels and reduced on the fly, so no
[tokens, V] tensor is ever materialised (ricardokevins notes, "Nitrobrew
tweet analysis", section "Nitrobrew 的两个动作"; the ``forward_kl`` /
``reverse_kl`` call shape follows the listing under "VeRL PR").

Layers:
  * ``libkd.so`` - the C ABI of ``include/kd.h`` (all arithmetic).
  * ``kd_fwd`` / ``kd_bwd`` / ``kd_topk_fwd`` / ``workspace_size`` below -
    thin ctypes bindings with the same names (argument marshalling only).
  * ``forward_kl`` / ``reverse_kl`` / ``jsd`` / ``topk_kd`` - autograd-aware
    losses with the per-token mean over non-ignored labels of ars-opd-rebuild
    "03 · 层 2：White-box OPD 基线", section 2.3.

PyTorch supplies device memory and the current stream only. There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KDError", "load_library", "workspace_size", "kd_fwd", "kd_fwd_noalloc", "kd_bwd", "kd_topk_fwd", "kd_topk_bwd",
    "kd_tail_fwd", "kd_tail_bwd", "kd_gather_rows", "kd_scatter_rows",
    "forward_kl", "reverse_kl", "jsd", "topk_kd", "tail_kd", "tail_default_support", "KD_TOPK_MAX",
    "KD_SUPPORT_TEACHER", "KD_SUPPORT_STUDENT", "KD_SUPPORT_LABEL",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkd.so")
KD_OK, KD_ERR_INVALID_ARG, KD_ERR_UNSUPPORTED, KD_ERR_WORKSPACE, KD_ERR_HIP = range(5)
KD_F32, KD_BF16 = 0, 1
KD_OP_FWD, KD_OP_BWD, KD_OP_TOPK, KD_OP_BWD_W, KD_OP_TOPK_BWD, KD_OP_TAIL, KD_OP_TAIL_BWD = range(7)
KD_SUPPORT_TEACHER, KD_SUPPORT_STUDENT, KD_SUPPORT_LABEL = 1, 2, 4
KD_TOPK_MAX = 64
KD_TOPK_MAX_V = 524288
EXPORTED = ("kd_workspace_size", "kd_default_chunk", "kd_fwd", "kd_fwd_noalloc", "kd_fwd_noalloc_max_scratch", "kd_bwd",
            "kd_topk_fwd", "kd_topk_bwd", "kd_tail_fwd", "kd_tail_bwd", "kd_gather_rows", "kd_scatter_rows",
            "kd_status_string", "kd_last_error")


class KDError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkd.so once and declare the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python vocab_chunked_kl_amd/build.py` (needs ROCm hipcc)")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kd_workspace_size.argtypes = [ctypes.c_int, i64, i64, i32, i32, ctypes.c_int, f32, i32, i32,
                                      ctypes.POINTER(sz)]
    lib.kd_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, f32, f32, ctypes.c_int, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, f32, f32, ctypes.c_int, i32, vp, vp, vp, vp, vp, vp,
                           vp, sz, vp]
    lib.kd_topk_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_topk_bwd.argtypes = [vp, vp, i64, i64, i32, i32, f32, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, i32, vp, vp, sz, vp]
    lib.kd_tail_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, f32, f32, ctypes.c_int, vp, vp, vp, vp,
                                vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_tail_bwd.argtypes = [vp, vp, i64, i64, i32, i32, i32, f32, f32, ctypes.c_int, vp, vp, vp, vp, vp, vp, i32,
                                vp, vp, sz, vp]
    lib.kd_fwd_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, f32, f32, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.kd_fwd_noalloc_max_scratch.argtypes = []
    lib.kd_fwd_noalloc_max_scratch.restype = sz
    lib.kd_default_chunk.argtypes = [i64, i64, ctypes.c_int]
    lib.kd_default_chunk.restype = i32
    lib.kd_gather_rows.argtypes = [vp, i64, i64, vp, i64, vp, vp]
    lib.kd_scatter_rows.argtypes = [vp, i64, i64, vp, vp, i64, vp]
    for fn in ("kd_workspace_size", "kd_fwd", "kd_fwd_noalloc", "kd_bwd", "kd_topk_fwd", "kd_topk_bwd", "kd_tail_fwd", "kd_tail_bwd",
               "kd_gather_rows", "kd_scatter_rows"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.kd_status_string.argtypes = [ctypes.c_int]
    lib.kd_status_string.restype = ctypes.c_char_p
    lib.kd_last_error.argtypes = []
    lib.kd_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code: int):
    if code != KD_OK:
        lib = load_library()
        raise KDError(code, f"{lib.kd_status_string(code).decode()}: {lib.kd_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KD_BF16
    if t.dtype == torch.float32:
        return KD_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _inputs(h_s, W_s, h_t, W_t):
    for name, t in (("h_s", h_s), ("W_s", W_s), ("h_t", h_t), ("W_t", W_t)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D tensor")
    if h_s.dtype != W_s.dtype or h_s.dtype != h_t.dtype or h_s.dtype != W_t.dtype:
        raise TypeError("h_s, W_s, h_t, W_t must share one dtype")
    N, d_s = h_s.shape
    V, d_t = W_t.shape
    if h_t.shape[0] != N or W_s.shape != (V, d_s) or h_t.shape[1] != d_t:
        raise ValueError(f"shape mismatch: h_s {tuple(h_s.shape)} W_s {tuple(W_s.shape)} "
                         f"h_t {tuple(h_t.shape)} W_t {tuple(W_t.shape)}")
    return N, V, d_s, d_t, _dtype_code(h_s)


def default_chunk(N: int, V: int, dtype: int = KD_BF16) -> int:
    """The recompute chunk the backward calls use for ``chunk_V=0``
    (kd_default_chunk): the fewest equal chunks whose [N, chunk] gradient
    tile fits in 1 GiB."""
    return int(load_library().kd_default_chunk(N, V, dtype))


def workspace_size(op: int, N: int, V: int, d_s: int, d_t: int, dtype: int = KD_BF16, beta: float = 1.0,
                   chunk_V: int = 0, k: int = 64) -> int:
    """Bytes of device workspace ``op`` needs (kd_workspace_size); ``chunk_V=0``
    is the library's default chunk."""
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.kd_workspace_size(op, N, V, d_s, d_t, dtype, float(beta), chunk_V, k, ctypes.byref(out)))
    return int(out.value)


def _workspace(nbytes: int, device, workspace=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def kd_fwd(h_s, W_s, h_t, W_t, beta: float, tau: float, workspace=None, stream=None):
    """Per-token divergence; returns (loss, lse_s, lse_t, aux), each fp32 [N]."""
    lib = load_library()
    N, V, d_s, d_t, dt = _inputs(h_s, W_s, h_t, W_t)
    dev = h_s.device
    loss, lse_s, lse_t, aux = (torch.empty(N, dtype=torch.float32, device=dev) for _ in range(4))
    nbytes = workspace_size(KD_OP_FWD, N, V, d_s, d_t, dt, beta=beta)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.kd_fwd(_ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), N, V, d_s, d_t, float(beta), float(tau), dt,
                      _ptr(loss), _ptr(lse_s), _ptr(lse_t), _ptr(aux), _ptr(ws), ws.numel() * ws.element_size(),
                      _stream(stream)))
    return loss, lse_s, lse_t, aux


def kd_fwd_noalloc(h_s, W_s, h_t, W_t, beta: float, tau: float, out=None, stream=None):
    """kd_fwd without a workspace: the library's fixed per-GPU scratch holds
    the partial records. ``out``: optional (loss, lse_s, lse_t, aux) fp32 [N]
    tensors to write (else new ones). Returns (loss, lse_s, lse_t, aux)."""
    lib = load_library()
    N, V, d_s, d_t, dt = _inputs(h_s, W_s, h_t, W_t)
    if out is None:
        out = tuple(torch.empty(N, dtype=torch.float32, device=h_s.device) for _ in range(4))
    for t in out:
        if t.dtype != torch.float32 or t.numel() != N or not t.is_contiguous():
            raise ValueError(f"outputs must be contiguous fp32 tensors of {N} elements")
    loss, lse_s, lse_t, aux = out
    _check(lib.kd_fwd_noalloc(_ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), N, V, d_s, d_t, float(beta), float(tau), dt,
                              _ptr(loss), _ptr(lse_s), _ptr(lse_t), _ptr(aux), _stream(stream)))
    return loss, lse_s, lse_t, aux


def kd_bwd(h_s, W_s, h_t, W_t, beta: float, tau: float, lse_s, lse_t, aux, grad_loss=None, chunk_V: int = 0,
           workspace=None, stream=None, dh=None, dW=None, want_dh: bool = True, want_dW: bool = False):
    """dL/dh_s (fp32 [N, d_s]) and, with ``want_dW``, dL/dW_s (fp32 [V, d_s])
    for L = sum_n grad_loss[n] * loss[n]. Returns dh, or (dh, dW) when
    ``want_dW`` (dh is None when ``want_dh`` is False)."""
    lib = load_library()
    N, V, d_s, d_t, dt = _inputs(h_s, W_s, h_t, W_t)
    dev = h_s.device
    if not want_dh and not want_dW:
        raise ValueError("nothing to compute: want_dh and want_dW are both False")
    if want_dh and dh is None:
        dh = torch.empty(N, d_s, dtype=torch.float32, device=dev)
    if want_dW and dW is None:
        dW = torch.empty(V, d_s, dtype=torch.float32, device=dev)
    for name, t, shape in (("dh", dh if want_dh else None, (N, d_s)), ("dW", dW if want_dW else None, (V, d_s))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {shape}")
    op = KD_OP_BWD_W if want_dW else KD_OP_BWD
    nbytes = workspace_size(op, N, V, d_s, d_t, dt, beta=beta, chunk_V=chunk_V)
    ws = _workspace(nbytes, dev, workspace)
    for name, t in (("lse_s", lse_s), ("lse_t", lse_t), ("aux", aux), ("grad_loss", grad_loss)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != N or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor of {N} elements")
    _check(lib.kd_bwd(_ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), N, V, d_s, d_t, float(beta), float(tau), dt,
                      int(chunk_V), _ptr(lse_s), _ptr(lse_t), _ptr(aux), _ptr(grad_loss),
                      _ptr(dh if want_dh else None), _ptr(dW if want_dW else None), _ptr(ws),
                      ws.numel() * ws.element_size(), _stream(stream)))
    if want_dW:
        return (dh if want_dh else None), dW
    return dh


def kd_topk_fwd(h_s, W_s, h_t, W_t, k: int, tau: float, labels=None, workspace=None, stream=None, with_values=True):
    """Top-k three-term decomposition; returns a dict of per-token tensors."""
    lib = load_library()
    N, V, d_s, d_t, dt = _inputs(h_s, W_s, h_t, W_t)
    dev = h_s.device
    f = lambda: torch.empty(N, dtype=torch.float32, device=dev)  # noqa: E731
    out = dict(idx=torch.empty(N, k, dtype=torch.int32, device=dev),
               val=torch.empty(N, k, dtype=torch.float32, device=dev) if with_values else None,
               val_s=torch.empty(N, k, dtype=torch.float32, device=dev) if with_values else None,
               binary=f(), cond=f(), ce=f() if labels is not None else None, p_mass=f(), q_mass=f(),
               lse_s=f(), lse_t=f(), lse_s1=f())
    if labels is not None and (labels.dtype != torch.int32 or labels.numel() != N or not labels.is_contiguous()):
        raise ValueError("labels must be a contiguous int32 tensor of N elements")
    nbytes = workspace_size(KD_OP_TOPK, N, V, d_s, d_t, dt, k=k)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.kd_topk_fwd(_ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), N, V, d_s, d_t, int(k), float(tau), dt,
                           _ptr(labels), _ptr(out["idx"]), _ptr(out["val"]), _ptr(out["val_s"]), _ptr(out["binary"]),
                           _ptr(out["cond"]),
                           _ptr(out["ce"]), _ptr(out["p_mass"]), _ptr(out["q_mass"]), _ptr(out["lse_s"]),
                           _ptr(out["lse_t"]), _ptr(out["lse_s1"]), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)))
    return out


def kd_topk_bwd(h_s, W_s, fwd: dict, k: int, tau: float, labels=None, grad_binary=None, grad_cond=None,
                grad_ce=None, chunk_V: int = 0, workspace=None, stream=None, dh=None):
    """dL/dh_s (fp32 [N, d_s]) of sum_n grad_binary[n] binary[n] + grad_cond[n] cond[n]
    + grad_ce[n] ce[n]; ``fwd`` is the dict returned by ``kd_topk_fwd`` for the
    same inputs (called with ``with_values=True``)."""
    lib = load_library()
    N, V, d_s, _, dt = _inputs(h_s, W_s, h_s, W_s)
    dev = h_s.device
    if fwd.get("val") is None or fwd.get("val_s") is None:
        raise ValueError("kd_topk_bwd needs the selected logits: call kd_topk_fwd with with_values=True")
    for name, t in (("grad_binary", grad_binary), ("grad_cond", grad_cond), ("grad_ce", grad_ce)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != N or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor of {N} elements")
    if dh is None:
        dh = torch.empty(N, d_s, dtype=torch.float32, device=dev)
    nbytes = workspace_size(KD_OP_TOPK_BWD, N, V, d_s, d_s, dt, chunk_V=chunk_V, k=k)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.kd_topk_bwd(_ptr(h_s), _ptr(W_s), N, V, d_s, int(k), float(tau), dt, _ptr(labels),
                           _ptr(fwd["idx"]), _ptr(fwd["val"]), _ptr(fwd["val_s"]), _ptr(fwd["p_mass"]),
                           _ptr(fwd["q_mass"]), _ptr(fwd["lse_s"]), _ptr(fwd.get("lse_s1")), _ptr(grad_binary),
                           _ptr(grad_cond), _ptr(grad_ce), int(chunk_V), _ptr(dh), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)))
    return dh


def tail_default_support(k: int, beta: float, with_labels: bool) -> int:
    """Support of the tail-bucket divergence (ars-opd-rebuild "03 · 层 2：White-box
    OPD 基线", section 2.4): one kept entry -> the label plus the teacher's top-1;
    else the teacher's top-k (beta = 0, a teacher-weighted sum), the student's
    (beta = 1) or their union (0 < beta < 1)."""
    if k == 1:
        return KD_SUPPORT_TEACHER | (KD_SUPPORT_LABEL if with_labels else 0)
    if beta == 0.0:
        return KD_SUPPORT_TEACHER
    if beta == 1.0:
        return KD_SUPPORT_STUDENT
    return KD_SUPPORT_TEACHER | KD_SUPPORT_STUDENT


def _support_slots(k: int, support: int) -> int:
    return (k if support & KD_SUPPORT_TEACHER else 0) + (k if support & KD_SUPPORT_STUDENT else 0) + \
        (1 if support & KD_SUPPORT_LABEL else 0)


def kd_tail_fwd(h_s, W_s, h_t, W_t, k: int, beta: float, tau: float, support: int, labels=None, workspace=None,
                stream=None):
    """Tail-bucket divergence over a top-k support; returns a dict of
    per-token tensors (``loss``, ``sup_idx`` / ``sup_t`` / ``sup_s`` [N, smax],
    ``p_mass``, ``q_mass``, ``lse_s``, ``lse_t``)."""
    lib = load_library()
    N, V, d_s, d_t, dt = _inputs(h_s, W_s, h_t, W_t)
    dev = h_s.device
    if labels is not None and (labels.dtype != torch.int32 or labels.numel() != N or not labels.is_contiguous()):
        raise ValueError("labels must be a contiguous int32 tensor of N elements")
    smax = max(_support_slots(int(k), int(support)), 1)
    f = lambda: torch.empty(N, dtype=torch.float32, device=dev)  # noqa: E731
    out = dict(sup_idx=torch.empty(N, smax, dtype=torch.int32, device=dev),
               sup_t=torch.empty(N, smax, dtype=torch.float32, device=dev),
               sup_s=torch.empty(N, smax, dtype=torch.float32, device=dev),
               loss=f(), p_mass=f(), q_mass=f(), lse_s=f(), lse_t=f())
    nbytes = workspace_size(KD_OP_TAIL, N, V, d_s, d_t, dt, k=k)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.kd_tail_fwd(_ptr(h_s), _ptr(W_s), _ptr(h_t), _ptr(W_t), N, V, d_s, d_t, int(k), int(support),
                           float(beta), float(tau), dt, _ptr(labels), _ptr(out["sup_idx"]), _ptr(out["sup_t"]),
                           _ptr(out["sup_s"]), _ptr(out["loss"]), _ptr(out["p_mass"]), _ptr(out["q_mass"]),
                           _ptr(out["lse_s"]), _ptr(out["lse_t"]), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)))
    return out


def kd_tail_bwd(h_s, W_s, fwd: dict, k: int, beta: float, tau: float, support: int, grad_loss=None,
                chunk_V: int = 0, workspace=None, stream=None, dh=None):
    """dL/dh_s (fp32 [N, d_s]) of sum_n grad_loss[n] loss[n] for the dict
    ``fwd`` that ``kd_tail_fwd`` returned for the same inputs."""
    lib = load_library()
    N, V, d_s, _, dt = _inputs(h_s, W_s, h_s, W_s)
    dev = h_s.device
    if grad_loss is not None and (grad_loss.dtype != torch.float32 or grad_loss.numel() != N
                                  or not grad_loss.is_contiguous()):
        raise ValueError(f"grad_loss must be a contiguous fp32 tensor of {N} elements")
    if fwd["sup_idx"].shape != (N, _support_slots(int(k), int(support))):
        raise ValueError("fwd's support arrays do not match k and support")
    if dh is None:
        dh = torch.empty(N, d_s, dtype=torch.float32, device=dev)
    nbytes = workspace_size(KD_OP_TAIL_BWD, N, V, d_s, d_s, dt, chunk_V=chunk_V, k=k)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.kd_tail_bwd(_ptr(h_s), _ptr(W_s), N, V, d_s, int(k), int(support), float(beta), float(tau), dt,
                           _ptr(fwd["sup_idx"]), _ptr(fwd["sup_t"]), _ptr(fwd["sup_s"]), _ptr(fwd["lse_s"]),
                           _ptr(fwd["lse_t"]), _ptr(grad_loss), int(chunk_V), _ptr(dh), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)))
    return dh


def _check_rows(rows):
    if rows.dtype != torch.int32 or rows.dim() != 1 or not rows.is_contiguous() or not rows.is_cuda:
        raise ValueError("rows must be a contiguous 1-D int32 GPU tensor")


def kd_gather_rows(src, rows, stream=None):
    """dst[i] = src[rows[i]] for a contiguous 2-D ``src`` (zeros for indices
    outside [0, len(src)))."""
    lib = load_library()
    _check_rows(rows)
    if src.dim() != 2 or not src.is_contiguous():
        raise ValueError("src must be a contiguous 2-D tensor")
    dst = torch.empty(rows.numel(), src.shape[1], dtype=src.dtype, device=src.device)
    _check(lib.kd_gather_rows(_ptr(src), src.shape[0], src.shape[1] * src.element_size(), _ptr(rows), rows.numel(),
                              _ptr(dst), _stream(stream)))
    return dst


def kd_scatter_rows(src, rows, n_dst: int, dst=None, stream=None):
    """dst[rows[i]] = src[i]; ``dst`` (default: zeros of n_dst rows) keeps its other rows."""
    lib = load_library()
    _check_rows(rows)
    if src.dim() != 2 or not src.is_contiguous():
        raise ValueError("src must be a contiguous 2-D tensor")
    if dst is None:
        dst = torch.zeros(n_dst, src.shape[1], dtype=src.dtype, device=src.device)
    _check(lib.kd_scatter_rows(_ptr(src), rows.numel(), src.shape[1] * src.element_size(), _ptr(rows), _ptr(dst),
                               n_dst, _stream(stream)))
    return dst


# ---------------------------------------------------------------------------
# autograd losses
# ---------------------------------------------------------------------------
class _KD(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xs, ws, xt, wt, beta, tau, chunk_V):
        loss, lse_s, lse_t, aux = kd_fwd(xs, ws, xt, wt, beta, tau)
        ctx.save_for_backward(xs, ws, xt, wt, lse_s, lse_t, aux)
        ctx.beta, ctx.tau, ctx.chunk_V = beta, tau, chunk_V
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        # the student hidden state and unembedding receive gradients; the
        # teacher's inputs are frozen
        xs, ws, xt, wt, lse_s, lse_t, aux = ctx.saved_tensors
        if ctx.needs_input_grad[2] or ctx.needs_input_grad[3]:
            raise NotImplementedError("the teacher's hidden state and unembedding receive no gradient")
        want_dh, want_dW = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not want_dh and not want_dW:
            return None, None, None, None, None, None, None
        out = kd_bwd(xs, ws, xt, wt, ctx.beta, ctx.tau, lse_s, lse_t, aux,
                     grad_loss=grad_loss.float().contiguous(), chunk_V=ctx.chunk_V, want_dh=want_dh,
                     want_dW=want_dW)
        dh, dW = out if want_dW else (out, None)
        return (dh.to(xs.dtype) if dh is not None else None, dW.to(ws.dtype) if dW is not None else None,
                None, None, None, None, None)


class _Rows(torch.autograd.Function):
    """Row gather (forward) / scatter (backward) of the tokens that carry a loss."""

    @staticmethod
    def forward(ctx, x, rows):
        ctx.save_for_backward(rows)
        ctx.n = x.shape[0]
        return kd_gather_rows(x, rows)

    @staticmethod
    def backward(ctx, g):
        (rows,) = ctx.saved_tensors
        return kd_scatter_rows(g.contiguous(), rows, ctx.n), None


class _Unrows(torch.autograd.Function):
    """Row scatter into zeros (forward) / gather (backward)."""

    @staticmethod
    def forward(ctx, x, rows, n):
        ctx.save_for_backward(rows)
        return kd_scatter_rows(x, rows, n)

    @staticmethod
    def backward(ctx, g):
        (rows,) = ctx.saved_tensors
        return kd_gather_rows(g.contiguous(), rows), None, None


def _no_tokens(xs, xt, ws, wt, lead, reduction):
    """The value of a loss over zero tokens (or zero kept tokens): 0, still
    attached to the inputs; per-token zeros for reduction="none"."""
    for name, t in (("xs", xs), ("xt", xt), ("ws", ws), ("wt", wt)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    zero = (xs.sum() + xt.sum() + ws.sum() + wt.sum()).float() * 0.0
    if reduction == "none":
        return (torch.zeros(lead, device=xs.device) + zero)
    if reduction not in ("sum", "mean"):
        raise ValueError(f"unknown reduction {reduction!r}")
    return zero


def _divergence(xs, xt, ws, wt, beta, temperature, reduction, chunk_V, labels, ignore_index):
    d_s, d_t = xs.shape[-1], xt.shape[-1]
    lead = xs.shape[:-1]
    xs2 = xs.reshape(-1, d_s).contiguous()
    xt2 = xt.reshape(-1, d_t).contiguous()
    if xs2.shape[0] == 0:
        return _no_tokens(xs, xt, ws, wt, lead, reduction)
    rows = None
    if labels is not None:
        valid = labels.reshape(-1) != ignore_index
        if not bool(valid.all()):
            # only the tokens that carry a loss are computed ([Top-K KD] 二.4)
            rows = torch.nonzero(valid).reshape(-1).to(torch.int32)
            if rows.numel() == 0:  # nothing carries a loss
                return _no_tokens(xs, xt, ws, wt, lead, reduction)
            xs2, xt2 = _Rows.apply(xs2, rows), _Rows.apply(xt2, rows)
    per_tok = _KD.apply(xs2, ws.contiguous(), xt2, wt.contiguous(), float(beta), float(temperature), int(chunk_V))
    count = torch.tensor(float(per_tok.numel()), device=per_tok.device)
    if rows is not None and reduction == "none":  # back to one value per position, 0 where ignored
        per_tok = _Unrows.apply(per_tok.reshape(-1, 1).contiguous(), rows, labels.numel()).reshape(-1)
    if reduction == "none":
        return per_tok.reshape(lead)
    if reduction == "sum":
        return per_tok.sum()
    if reduction == "mean":  # per-token mean over non-ignored positions
        return per_tok.sum() / count.clamp_min(1.0)
    raise ValueError(f"unknown reduction {reduction!r}")


def forward_kl(xs, xt, ws, wt, temperature=1.0, reduction="mean", chunk_V=0, labels=None, ignore_index=-100):
    """KL(teacher || student) from hidden states xs [.., D_s], xt [.., D_t] and
    unembeddings ws [V, D_s], wt [V, D_t]. ``chunk_V`` is the backward's
    recompute chunk (0: ``default_chunk``), here and in the other losses."""
    return _divergence(xs, xt, ws, wt, 0.0, temperature, reduction, chunk_V, labels, ignore_index)


def reverse_kl(xs, xt, ws, wt, temperature=1.0, reduction="mean", chunk_V=0, labels=None, ignore_index=-100):
    """KL(student || teacher) from hidden states and unembeddings."""
    return _divergence(xs, xt, ws, wt, 1.0, temperature, reduction, chunk_V, labels, ignore_index)


def jsd(xs, xt, ws, wt, beta=0.5, temperature=1.0, reduction="mean", chunk_V=0, labels=None, ignore_index=-100):
    """beta KL(teacher || m) + (1 - beta) KL(student || m), m = beta teacher + (1 - beta) student;
    beta = 0 / 1 give forward / reverse KL."""
    return _divergence(xs, xt, ws, wt, beta, temperature, reduction, chunk_V, labels, ignore_index)


class _TopK(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xs, ws, xt, wt, k, tau, lab, chunk_V, holder):
        out = kd_topk_fwd(xs, ws, xt, wt, k, tau, labels=lab)
        holder.update(out)
        ctx.save_for_backward(xs, ws)
        ctx.out, ctx.k, ctx.tau, ctx.lab, ctx.chunk_V = out, k, tau, lab, chunk_V
        ce = out["ce"] if out["ce"] is not None else torch.zeros_like(out["binary"])
        return out["binary"], out["cond"], ce

    @staticmethod
    def backward(ctx, g_binary, g_cond, g_ce):
        xs, ws = ctx.saved_tensors
        if ctx.needs_input_grad[1] or ctx.needs_input_grad[2] or ctx.needs_input_grad[3]:
            raise NotImplementedError("the top-k terms give a gradient to the student hidden state only")
        if not ctx.needs_input_grad[0]:
            return (None,) * 9
        f = lambda g: None if g is None else g.float().contiguous()  # noqa: E731
        dh = kd_topk_bwd(xs, ws, ctx.out, ctx.k, ctx.tau, labels=ctx.lab, grad_binary=f(g_binary),
                         grad_cond=f(g_cond), grad_ce=f(g_ce) if ctx.lab is not None else None,
                         chunk_V=ctx.chunk_V)
        return (dh.to(xs.dtype),) + (None,) * 8


def topk_kd(xs, xt, ws, wt, k=64, labels=None, temperature=1.0, ignore_index=-100, chunk_V=0):
    """Top-k three-term KD terms per token: dict with ``binary``, ``cond``,
    ``ce`` (when labels are given; these three carry the gradient to ``xs``,
    one value per position), masses, LSEs and the selection.

    Tokens whose label is ``ignore_index`` are gathered out before the sweep
    ([Top-K KD] 二.4), as in the other losses: their binary / cond / ce are 0
    and get no gradient, and the other entries of the dict (masses, LSEs,
    ``idx``, ...) then cover the kept tokens only, listed in ``rows`` (None
    when every token is kept)."""
    d_s, d_t = xs.shape[-1], xt.shape[-1]
    xs2 = xs.reshape(-1, d_s).contiguous()
    xt2 = xt.reshape(-1, d_t).contiguous()
    n_all = xs2.shape[0]
    lab = None
    rows = None
    if labels is not None:
        lab = labels.reshape(-1).to(torch.int32).contiguous()
        valid = lab != ignore_index
        if not bool(valid.all()):
            rows = torch.nonzero(valid).reshape(-1).to(torch.int32)
            if rows.numel() == 0:  # nothing carries a loss
                zero = _no_tokens(xs, xt, ws, wt, (n_all,), "none")
                return dict(binary=zero, cond=zero.clone(), ce=zero.clone(), rows=rows)
            xs2, xt2 = _Rows.apply(xs2, rows), _Rows.apply(xt2, rows)
            lab = lab.index_select(0, rows.long()).contiguous()
    holder = {}
    binary, cond, ce = _TopK.apply(xs2, ws.contiguous(), xt2, wt.contiguous(), int(k), float(temperature), lab,
                                   int(chunk_V), holder)
    if rows is not None:  # back to one value per position, 0 where ignored
        binary, cond, ce = (_Unrows.apply(t.reshape(-1, 1).contiguous(), rows, n_all).reshape(-1)
                            for t in (binary, cond, ce))
    holder.update(binary=binary, cond=cond, ce=ce if lab is not None else None, rows=rows)
    return holder


class _Tail(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xs, ws, xt, wt, k, beta, tau, support, lab, chunk_V, holder):
        out = kd_tail_fwd(xs, ws, xt, wt, k, beta, tau, support, labels=lab)
        holder.update(out)
        ctx.save_for_backward(xs, ws)
        ctx.out, ctx.k, ctx.beta, ctx.tau, ctx.support, ctx.chunk_V = out, k, beta, tau, support, chunk_V
        return out["loss"]

    @staticmethod
    def backward(ctx, g):
        xs, ws = ctx.saved_tensors
        if ctx.needs_input_grad[1] or ctx.needs_input_grad[2] or ctx.needs_input_grad[3]:
            raise NotImplementedError("the tail-bucket divergence gives a gradient to the student hidden state only")
        if not ctx.needs_input_grad[0]:
            return (None,) * 11
        dh = kd_tail_bwd(xs, ws, ctx.out, ctx.k, ctx.beta, ctx.tau, ctx.support, grad_loss=g.float().contiguous(),
                         chunk_V=ctx.chunk_V)
        return (dh.to(xs.dtype),) + (None,) * 10


def tail_kd(xs, xt, ws, wt, k=1, beta=0.0, labels=None, temperature=1.0, support=None, reduction="mean",
            ignore_index=-100, chunk_V=0, return_dict=False):
    """Beta-divergence over a top-k support plus a tail bucket (ars-opd-rebuild
    "03 · 层 2：White-box OPD 基线", section 2.4), per-token mean over
    non-ignored labels by default. ``support`` defaults to
    ``tail_default_support(k, beta, labels is not None)``. Tokens whose label
    is ignored are gathered out before the sweep ([Top-K KD] 二.4) and count
    as 0. With ``return_dict`` also returns the forward's per-token dict (over
    the computed rows: all tokens, or the kept ones when some are ignored)."""
    d_s, d_t = xs.shape[-1], xt.shape[-1]
    lead = xs.shape[:-1]
    xs2 = xs.reshape(-1, d_s).contiguous()
    xt2 = xt.reshape(-1, d_t).contiguous()
    if xs2.shape[0] == 0:
        res = _no_tokens(xs, xt, ws, wt, lead, reduction)
        return (res, {}) if return_dict else res
    lab = None
    rows = None
    if labels is not None:
        lab = labels.reshape(-1).to(torch.int32).contiguous()
        valid = lab != ignore_index
        if not bool(valid.all()):
            rows = torch.nonzero(valid).reshape(-1).to(torch.int32)
            if rows.numel() == 0:
                res = _no_tokens(xs, xt, ws, wt, lead, reduction)
                return (res, {}) if return_dict else res
            xs2, xt2 = _Rows.apply(xs2, rows), _Rows.apply(xt2, rows)
            lab = lab.index_select(0, rows.long()).contiguous()
    if support is None:
        support = tail_default_support(int(k), float(beta), lab is not None)
    holder = {}
    per_tok = _Tail.apply(xs2, ws.contiguous(), xt2, wt.contiguous(), int(k), float(beta), float(temperature),
                          int(support), lab if support & KD_SUPPORT_LABEL else None, int(chunk_V), holder)
    count = torch.tensor(float(per_tok.numel()), device=per_tok.device)
    if reduction == "none":
        if rows is not None:  # back to one value per position, 0 where ignored
            per_tok = _Unrows.apply(per_tok.reshape(-1, 1).contiguous(), rows, xs.reshape(-1, d_s).shape[0])
        res = per_tok.reshape(lead)
    elif reduction == "sum":
        res = per_tok.sum()
    elif reduction == "mean":
        res = per_tok.sum() / count.clamp_min(1.0)
    else:
        raise ValueError(f"unknown reduction {reduction!r}")
    return (res, holder) if return_dict else res
