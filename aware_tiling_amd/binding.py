"""ctypes binding of ``libaware_tiling.so`` (the C ABI in include/aware_tiling.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory (output and
workspace tensors) and the current HIP stream.  If the shared library is not
built, loading it raises immediately; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libaware_tiling.so")

ATTN_F32, ATTN_BF16 = 0, 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
          3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_LAUNCH"}

# Every symbol include/aware_tiling.h declares, with (restype, argtypes).
_vp, _i64, _f32, _int, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                               ctypes.c_size_t)
SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [_int]),
    "attn_last_hip_error": (ctypes.c_char_p, []),
    "attn_version": (ctypes.c_char_p, []),
    "attn_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _vp]),
    "attn_fwd_onchip_elems": (_i64, [_i64, _int]),
    "attn_fwd_query_block": (_i64, [_i64, _int]),
    "attn_fwd_budget": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _i64, _vp]),
    "attn_fwd_budget_onchip_elems": (_i64, [_i64]),
    "attn_calib_mfma_loop": (_int, [_vp, _i64, ctypes.c_int32, _f32, _vp]),
    "attn_fwd_splitk_splits": (_i64, [_i64, _i64, _i64, _i64, _i64]),
    "attn_fwd_splitk_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "attn_fwd_splitk": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _i64,
                               _vp, _sz, _vp]),
    "attn_fwd_blocksparse_workspace_size": (_sz, [_i64, _i64, _i64]),
    "attn_fwd_blocksparse": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _vp,
                                    _i64, _vp, _sz, _vp]),
    "attn_fwd_smallcache_workspace_size": (_sz, [_i64, _i64, _i64, _i64]),
    "attn_fwd_smallcache": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _i64,
                                   _vp, _sz, _vp]),
    "attn_smallcache_tile": (_i64, [_i64, _i64]),
    "attn_smallcache_onchip_elems": (_i64, [_i64]),
    "attn_bwd_workspace_size": (_sz, [_i64, _i64, _i64]),
    "attn_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int,
                        _vp, _sz, _vp]),
    "attn_bwd_smallcache_tile": (_i64, [_i64, _i64]),
    "attn_bwd_smallcache_onchip_elems": (_i64, [_i64, _i64]),
    "attn_bwd_smallcache_workspace_size": (_sz, [_i64, _i64, _i64, _i64]),
    "attn_bwd_smallcache": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                   _f32, _int, _i64, _vp, _sz, _vp]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int, hip: str = ""):
        self.code = code
        msg = f"{fn} failed: {STATUS.get(code, code)}"
        if hip:
            msg += f" ({hip})"
        super().__init__(msg)


def lib(path: str | None = None):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m aware_tiling_amd.build`")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(l):
    for name, (res, args) in SIGNATURES.items():
        f = getattr(l, name)
        f.restype = res
        f.argtypes = args
    return l


def _check(fn: str, rc: int):
    if rc != 0:
        hip = lib().attn_last_hip_error().decode() if rc == 4 else ""
        raise AttnError(fn, rc, hip)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_inputs(*ts: torch.Tensor):
    ref = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.device != ref.device:
            raise ValueError("tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dim() != 3:
            raise ValueError("tensors must be [bh, n, d]")


def _stream(t: torch.Tensor, stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream


def default_scale(d: int) -> float:
    return float(torch.tensor(d, dtype=torch.float32).rsqrt())


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
             out: torch.Tensor | None = None, lse: torch.Tensor | bool = True, stream=None):
    """Fused streaming forward. Returns (O fp32 [bh,n,d], lse fp32 [bh,n] or None)."""
    _check_inputs(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q, K, V must share shape and dtype")
    bh, n, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((bh, n, d), dtype=torch.float32, device=q.device)
    if lse is True:
        lse = torch.empty((bh, n), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    rc = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                        _dtype_code(q), _stream(q, stream))
    _check("attn_fwd", rc)
    return out, lse


def fwd_budget_onchip_elems(d: int) -> int:
    """On-chip elements of one attn_fwd_budget workgroup (0 = unsupported d)."""
    return int(lib().attn_fwd_budget_onchip_elems(d))


def attn_fwd_budget(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, m_elems: int,
                    scale: float | None = None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | bool = True, stream=None):
    """Fused streaming forward with 32-row query blocks, for an on-chip budget
    of m_elems elements below d^2. Returns (O, lse)."""
    _check_inputs(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q, K, V must share shape and dtype")
    bh, n, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((bh, n, d), dtype=torch.float32, device=q.device)
    if lse is True:
        lse = torch.empty((bh, n), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    rc = lib().attn_fwd_budget(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                               _dtype_code(q), int(m_elems), _stream(q, stream))
    _check("attn_fwd_budget", rc)
    return out, lse


def calib_mfma_loop(out: torch.Tensor, iters: int, amp: float = 1.0, stream=None) -> int:
    """Calibration matrix-core loop (no memory traffic) over out.numel() // 256
    workgroups; returns the flops it issues. out: float32 CUDA tensor."""
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 CUDA tensor")
    wgs = out.numel() // 256
    rc = lib().attn_calib_mfma_loop(out.data_ptr(), wgs, int(iters), float(amp),
                                    _stream(out, stream))
    _check("attn_calib_mfma_loop", rc)
    return wgs * int(iters) * 4 * 4 * 2 * 32 * 32 * 16


def splitk_splits(bh: int, nq: int, nk: int, d: int, splits: int = 0) -> int:
    """Key chunks attn_fwd_splitk uses for this shape and request (0 = auto)."""
    return int(lib().attn_fwd_splitk_splits(bh, nq, nk, d, splits))


def attn_fwd_splitk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, splits: int = 0,
                    scale: float | None = None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | bool = True, workspace: torch.Tensor | None = None,
                    stream=None):
    """Rectangular forward (nq queries, nk keys per head) with the keys split
    into chunks whose partial results are merged.  Returns (O, lse)."""
    _check_inputs(q, k, v)
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2] \
            or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q [bh,nq,d], K and V [bh,nk,d] must agree in bh, d and dtype")
    bh, nq, d = q.shape
    nk = k.shape[1]
    scale = default_scale(d) if scale is None else float(scale)
    need = int(lib().attn_fwd_splitk_workspace_size(bh, nq, nk, d, int(splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((bh, nq, d), dtype=torch.float32, device=q.device)
    if lse is True:
        lse = torch.empty((bh, nq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    rc = lib().attn_fwd_splitk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, bh, nq, nk, d, scale,
                               _dtype_code(q), int(splits), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(q, stream))
    _check("attn_fwd_splitk", rc)
    return out, lse


SPARSE_BLOCK = 128  # ATTN_SPARSE_BLOCK: queries and keys per mask block


def attn_fwd_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         block_mask: torch.Tensor, scale: float | None = None,
                         out: torch.Tensor | None = None, lse: torch.Tensor | bool = True,
                         workspace: torch.Tensor | None = None, stream=None):
    """Forward over the 128 x 128 blocks that ``block_mask`` ([1 or bh, nb, nb],
    uint8 or bool on the GPU, nonzero = kept) keeps.  Returns (O, lse); rows
    with no kept key give O = 0, lse = -inf."""
    _check_inputs(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q, K, V must share shape and dtype")
    bh, n, d = q.shape
    nb = -(-n // SPARSE_BLOCK)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda or block_mask.dim() != 3
            or tuple(block_mask.shape[1:]) != (nb, nb) or block_mask.shape[0] not in (1, bh)):
        raise ValueError(f"block_mask must be uint8 [1 or {bh}, {nb}, {nb}] on the GPU")
    block_mask = block_mask.contiguous()
    mh = block_mask.shape[0]
    scale = default_scale(d) if scale is None else float(scale)
    need = int(lib().attn_fwd_blocksparse_workspace_size(bh, n, mh))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((bh, n, d), dtype=torch.float32, device=q.device)
    if lse is True:
        lse = torch.empty((bh, n), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    rc = lib().attn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                                    _dtype_code(q), block_mask.data_ptr(), mh,
                                    workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(q, stream))
    _check("attn_fwd_blocksparse", rc)
    return out, lse


def smallcache_tile(d: int, m_elems: int) -> int:
    return int(lib().attn_smallcache_tile(d, m_elems))


def attn_fwd_smallcache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, m_elems: int,
                        scale: float | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | bool = True, workspace: torch.Tensor | None = None,
                        stream=None):
    """Square-tile forward (stores exp(S) in the workspace). Returns (O, lse)."""
    _check_inputs(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q, K, V must share shape and dtype")
    bh, n, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    need = int(lib().attn_fwd_smallcache_workspace_size(bh, n, d, m_elems))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((bh, n, d), dtype=torch.float32, device=q.device)
    if lse is True:
        lse = torch.empty((bh, n), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    rc = lib().attn_fwd_smallcache(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                                   _dtype_code(q), int(m_elems), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(q, stream))
    _check("attn_fwd_smallcache", rc)
    return out, lse


def attn_bwd(q, k, v, o, do, lse, scale: float | None = None, workspace=None, grads=None,
             stream=None):
    """Gradients (dQ, dK, dV) in fp32 from the forward's O and lse."""
    _check_inputs(q, k, v, o, do)
    bh, n, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    need = int(lib().attn_bwd_workspace_size(bh, n, d))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = tuple(torch.empty((bh, n, d), dtype=torch.float32, device=q.device)
                      for _ in range(3))
    dq, dk, dv = grads
    rc = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), bh, n, d,
                        scale, _dtype_code(q), workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), _stream(q, stream))
    _check("attn_bwd", rc)
    return dq, dk, dv


def attn_bwd_smallcache(q, k, v, o, do, lse, m_elems: int, scale: float | None = None,
                        workspace=None, grads=None, stream=None):
    """Square-tile (small-cache) gradients (dQ, dK, dV) in fp32; the n x n
    P^T and dS^T live in the workspace."""
    _check_inputs(q, k, v, o, do)
    bh, n, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    need = int(lib().attn_bwd_smallcache_workspace_size(bh, n, d, int(m_elems)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = tuple(torch.empty((bh, n, d), dtype=torch.float32, device=q.device)
                      for _ in range(3))
    dq, dk, dv = grads
    rc = lib().attn_bwd_smallcache(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), bh, n, d, scale, _dtype_code(q), int(m_elems),
                                   workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(q, stream))
    _check("attn_bwd_smallcache", rc)
    return dq, dk, dv


def bwd_smallcache_tile(d: int, m_elems: int) -> int:
    return int(lib().attn_bwd_smallcache_tile(d, m_elems))


def fwd_onchip_elems(d: int, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib().attn_fwd_onchip_elems(d, ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32))


def fwd_query_block(d: int, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib().attn_fwd_query_block(d, ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32))
