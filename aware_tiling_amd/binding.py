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
    "attn_fwd_tiles": (ctypes.c_char_p, [_i64]),
    "attn_fwd_tile_info": (_int, [ctypes.c_char_p, _i64, _vp, _vp, _vp]),
    "attn_fwd_tile": (_int, [ctypes.c_char_p, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32,
                             _int, _vp]),
    "attn_fwd_budget": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _i64, _vp]),
    "attn_fwd_budget_onchip_elems": (_i64, [_i64]),
    "attn_calib_mfma_loop": (_int, [_vp, _i64, ctypes.c_int32, _f32, _vp]),
    "attn_calib_stream_read": (_int, [_vp, _i64, _vp, _i64, _vp]),
    "attn_fwd_splitk_splits": (_i64, [_i64, _i64, _i64, _i64, _i64]),
    "attn_fwd_splitk_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "attn_fwd_splitk": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _i64,
                               _vp, _sz, _vp]),
    "attn_fwd_splitk_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int,
                                       _i64, _vp]),
    "attn_fwd_blocksparse_workspace_size": (_sz, [_i64, _i64, _i64]),
    "attn_fwd_blocksparse": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _vp,
                                    _i64, _vp, _sz, _vp]),
    "attn_fwd_smallcache_workspace_size": (_sz, [_i64, _i64, _i64, _i64]),
    "attn_fwd_smallcache": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _i64,
                                   _vp, _sz, _vp]),
    "attn_smallcache_tile": (_i64, [_i64, _i64]),
    "attn_smallcache_onchip_elems": (_i64, [_i64]),
    "attn_bwd_workspace_size": (_sz, [_i64, _i64, _i64]),
    "attn_bwd_onchip_elems": (_i64, [_i64]),
    "attn_bwd_tiles": (ctypes.c_char_p, [_i64]),
    "attn_bwd_tile_info": (_int, [ctypes.c_char_p, _i64, _vp, _vp, _vp, _vp]),
    "attn_bwd_tile": (_int, [ctypes.c_char_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                             _i64, _i64, _f32, _int, _vp, _sz, _vp]),
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


def _on_gpu(t: torch.Tensor) -> bool:
    """Whether ``t`` lives in GPU memory (the kernels read and write it)."""
    return t.is_cuda


def _check_inputs(*ts: torch.Tensor):
    """Q, K, V (and dO) style inputs: tensors on one GPU, contiguous,
    [bh, n, d], bf16 or fp32."""
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("inputs must be torch tensors")
        if not _on_gpu(t):
            raise ValueError("tensors must be on the GPU")
        if t.device != ref.device:
            raise ValueError("tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dim() != 3:
            raise ValueError("tensors must be [bh, n, d]")
        if t.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"unsupported dtype {t.dtype}")


def _check_buffer(t, name: str, shape, dtype: torch.dtype, device: torch.device):
    """A caller-supplied output or auxiliary tensor the kernels read or write
    in full: it must have exactly ``shape`` and ``dtype``, be contiguous and
    sit on ``device``; anything else could send a kernel past its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not _on_gpu(t) or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(t, device: torch.device):
    """Workspace: contiguous device memory of any dtype on ``device`` (the
    library checks its byte size and alignment)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if not _on_gpu(t) or t.device != device:
        raise ValueError(f"workspace must be on {device}")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _out_lse(out, lse, bh: int, n: int, d: int, device):
    """Allocate or check the forward's O [bh, n, d] fp32 and lse [bh, n] fp32
    (lse=True allocates, False or None means no lse)."""
    if out is None:
        out = torch.empty((bh, n, d), dtype=torch.float32, device=device)
    else:
        _check_buffer(out, "out", (bh, n, d), torch.float32, device)
    if lse is True:
        lse = torch.empty((bh, n), dtype=torch.float32, device=device)
    elif lse is False or lse is None:
        lse = None
    else:
        _check_buffer(lse, "lse", (bh, n), torch.float32, device)
    return out, lse


def _grads(grads, bh: int, n: int, d: int, device):
    if grads is None:
        return tuple(torch.empty((bh, n, d), dtype=torch.float32, device=device)
                     for _ in range(3))
    if len(grads) != 3:
        raise ValueError("grads must be (dQ, dK, dV)")
    for name, g in zip(("dQ", "dK", "dV"), grads):
        _check_buffer(g, name, (bh, n, d), torch.float32, device)
    return tuple(grads)


def _bwd_operands(q, k, v, o, do, lse):
    """Backward inputs: Q, K, V, dO of one shape and dtype; O fp32 and lse
    fp32 as written by the forward."""
    _check_inputs(q, k, v, do)
    if not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError("Q, K, V and dO must share one shape")
    if not (q.dtype == k.dtype == v.dtype == do.dtype):
        raise ValueError("Q, K, V and dO must share one dtype")
    bh, n, d = q.shape
    _check_buffer(o, "O", (bh, n, d), torch.float32, q.device)
    _check_buffer(lse, "lse", (bh, n), torch.float32, q.device)
    return bh, n, d


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
    out, lse = _out_lse(out, lse, bh, n, d, q.device)
    rc = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                        _dtype_code(q), _stream(q, stream))
    _check("attn_fwd", rc)
    return out, lse


def fwd_tiles(d: int) -> list[str]:
    """Names of the fused forward's compiled tile shapes for head dimension
    d, the default (the one attn_fwd uses) first."""
    return lib().attn_fwd_tiles(d).decode().split()


def fwd_tile_info(tile: str, d: int) -> dict:
    """Query-block rows, keys per tile and on-chip elements of a named
    tile shape at head dimension d."""
    vals = [ctypes.c_int64(0) for _ in range(3)]
    rc = lib().attn_fwd_tile_info(tile.encode(), d, *(ctypes.byref(x) for x in vals))
    _check("attn_fwd_tile_info", rc)
    return {"block_rows": vals[0].value, "key_tile": vals[1].value, "onchip_elems": vals[2].value}


def attn_fwd_tile(tile: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  scale: float | None = None, out: torch.Tensor | None = None,
                  lse: torch.Tensor | bool = True, stream=None):
    """attn_fwd with the named tile shape (tile sweeps and tests).
    Returns (O, lse)."""
    _check_inputs(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q, K, V must share shape and dtype")
    bh, n, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    out, lse = _out_lse(out, lse, bh, n, d, q.device)
    rc = lib().attn_fwd_tile(tile.encode(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             out.data_ptr(), lse.data_ptr() if lse is not None else None, bh, n,
                             d, scale, _dtype_code(q), _stream(q, stream))
    _check("attn_fwd_tile", rc)
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
    out, lse = _out_lse(out, lse, bh, n, d, q.device)
    rc = lib().attn_fwd_budget(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                               _dtype_code(q), int(m_elems), _stream(q, stream))
    _check("attn_fwd_budget", rc)
    return out, lse


def calib_mfma_loop(out: torch.Tensor, iters: int, amp: float = 1.0, stream=None) -> int:
    """Calibration matrix-core loop (no memory traffic) over out.numel() // 256
    workgroups; returns the flops it issues. out: float32 CUDA tensor."""
    if out.dtype != torch.float32 or not _on_gpu(out) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 CUDA tensor")
    wgs = out.numel() // 256
    rc = lib().attn_calib_mfma_loop(out.data_ptr(), wgs, int(iters), float(amp),
                                    _stream(out, stream))
    _check("attn_calib_mfma_loop", rc)
    return wgs * int(iters) * 4 * 4 * 2 * 32 * 32 * 16


def calib_stream_read(src: torch.Tensor, out: torch.Tensor, stream=None) -> int:
    """Calibration streaming read of all of src over out.numel() // 256
    workgroups; returns the bytes it reads. src: contiguous CUDA tensor of a
    multiple of 16 bytes; out: int32 CUDA tensor, one word per thread."""
    if not _on_gpu(src) or not src.is_contiguous():
        raise ValueError("src must be a contiguous CUDA tensor")
    if out.dtype != torch.int32 or not _on_gpu(out) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 CUDA tensor")
    nbytes = src.numel() * src.element_size()
    rc = lib().attn_calib_stream_read(src.data_ptr(), nbytes, out.data_ptr(), out.numel() // 256,
                                      _stream(out, stream))
    _check("attn_calib_stream_read", rc)
    return nbytes


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
    out, lse = _out_lse(out, lse, bh, nq, d, q.device)
    if workspace is None:
        need = int(lib().attn_fwd_splitk_workspace_size(bh, nq, nk, d, int(splits)))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    rc = lib().attn_fwd_splitk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, bh, nq, nk, d, scale,
                               _dtype_code(q), int(splits), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(q, stream))
    _check("attn_fwd_splitk", rc)
    return out, lse


SPLITK_NOALLOC_SCRATCH_BYTES = 16 << 20  # ATTN_SPLITK_NOALLOC_SCRATCH_BYTES


def attn_fwd_splitk_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            out: torch.Tensor, lse: torch.Tensor | None = None, splits: int = 0,
                            scale: float | None = None, stream=None):
    """attn_fwd_splitk with the chunk partials in the library's own device
    array: neither the library nor this wrapper allocates (the caller passes
    O, and lse or None).  Returns (out, lse)."""
    _check_inputs(q, k, v)
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2] \
            or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("Q [bh,nq,d], K and V [bh,nk,d] must agree in bh, d and dtype")
    bh, nq, d = q.shape
    nk = k.shape[1]
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    _check_buffer(out, "out", (bh, nq, d), torch.float32, q.device)
    if lse is not None:
        _check_buffer(lse, "lse", (bh, nq), torch.float32, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    rc = lib().attn_fwd_splitk_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr() if lse is not None else None, bh, nq, nk, d,
                                       scale, _dtype_code(q), int(splits), _stream(q, stream))
    _check("attn_fwd_splitk_noalloc", rc)
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
    if not isinstance(block_mask, torch.Tensor):
        raise TypeError("block_mask must be a torch tensor")
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    if (not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8
            or not _on_gpu(block_mask) or block_mask.device != q.device
            or block_mask.dim() != 3 or tuple(block_mask.shape[1:]) != (nb, nb)
            or block_mask.shape[0] not in (1, bh)):
        raise ValueError(f"block_mask must be uint8 [1 or {bh}, {nb}, {nb}] on {q.device}")
    block_mask = block_mask.contiguous()
    mh = block_mask.shape[0]
    scale = default_scale(d) if scale is None else float(scale)
    out, lse = _out_lse(out, lse, bh, n, d, q.device)
    if workspace is None:
        need = int(lib().attn_fwd_blocksparse_workspace_size(bh, n, mh))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
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
    out, lse = _out_lse(out, lse, bh, n, d, q.device)
    if workspace is None:
        need = int(lib().attn_fwd_smallcache_workspace_size(bh, n, d, m_elems))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    rc = lib().attn_fwd_smallcache(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, bh, n, d, scale,
                                   _dtype_code(q), int(m_elems), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(q, stream))
    _check("attn_fwd_smallcache", rc)
    return out, lse


def bwd_tiles(d: int) -> list[str]:
    """Names of the blockwise backward's compiled tile shapes for head
    dimension d, the default (the one attn_bwd uses) first."""
    return lib().attn_bwd_tiles(d).decode().split()


def bwd_tile_info(tile: str, d: int) -> dict:
    """Keys per dK/dV workgroup, queries per dQ workgroup, keys per dQ tile
    and on-chip elements of a named backward tile shape at head dimension d."""
    vals = [ctypes.c_int64(0) for _ in range(4)]
    rc = lib().attn_bwd_tile_info(tile.encode(), d, *(ctypes.byref(x) for x in vals))
    _check("attn_bwd_tile_info", rc)
    return {"keys_per_block": vals[0].value, "queries_per_block": vals[1].value,
            "key_tile": vals[2].value, "onchip_elems": vals[3].value}


def attn_bwd_tile(tile: str, q, k, v, o, do, lse, scale: float | None = None, workspace=None,
                  grads=None, stream=None):
    """attn_bwd with the named tile shape (tile sweeps and tests)."""
    bh, n, d = _bwd_operands(q, k, v, o, do, lse)
    scale = default_scale(d) if scale is None else float(scale)
    dq, dk, dv = _grads(grads, bh, n, d, q.device)
    if workspace is None:
        need = int(lib().attn_bwd_workspace_size(bh, n, d))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    rc = lib().attn_bwd_tile(tile.encode(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                             dk.data_ptr(), dv.data_ptr(), bh, n, d, scale, _dtype_code(q),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             _stream(q, stream))
    _check("attn_bwd_tile", rc)
    return dq, dk, dv


def attn_bwd(q, k, v, o, do, lse, scale: float | None = None, workspace=None, grads=None,
             stream=None):
    """Gradients (dQ, dK, dV) in fp32 from the forward's O and lse."""
    bh, n, d = _bwd_operands(q, k, v, o, do, lse)
    scale = default_scale(d) if scale is None else float(scale)
    dq, dk, dv = _grads(grads, bh, n, d, q.device)
    if workspace is None:
        need = int(lib().attn_bwd_workspace_size(bh, n, d))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
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
    bh, n, d = _bwd_operands(q, k, v, o, do, lse)
    scale = default_scale(d) if scale is None else float(scale)
    dq, dk, dv = _grads(grads, bh, n, d, q.device)
    if workspace is None:
        need = int(lib().attn_bwd_smallcache_workspace_size(bh, n, d, int(m_elems)))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
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


def bwd_onchip_elems(d: int) -> int:
    """On-chip elements of one attn_bwd workgroup (the larger kernel; 0 =
    unsupported d)."""
    return int(lib().attn_bwd_onchip_elems(d))


def fwd_onchip_elems(d: int, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib().attn_fwd_onchip_elems(d, ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32))


def fwd_query_block(d: int, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib().attn_fwd_query_block(d, ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32))
