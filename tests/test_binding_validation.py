"""The Python binding rejects every malformed tensor before the library is
called (CPU only: the GPU check and the library are stubbed).

A wrong dtype, shape, device or layout of any tensor the kernels read or
write in full (O, lse, dO, the gradients, the block mask, the workspace)
would send a kernel past the end of a buffer, so each must raise ValueError
or TypeError in the binding, before any launch.  The stub library fails the
test if it is reached for a malformed call, and records the well-formed
calls that do reach it.
"""
import pytest
import torch

from aware_tiling_amd import binding


class _FakeStream:
    cuda_stream = 0


class _StubLib:
    """Stands in for libaware_tiling.so: records calls, returns ATTN_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 256 if name.endswith("_workspace_size") else 0
        return fn


@pytest.fixture
def stub(monkeypatch):
    lib = _StubLib()
    monkeypatch.setattr(binding, "_on_gpu", lambda t: True)
    monkeypatch.setattr(binding, "lib", lambda path=None: lib)
    return lib


BH, N, D = 2, 48, 64
S = _FakeStream()


def _qkv(dtype=torch.bfloat16, n=N):
    return tuple(torch.zeros((BH, n, D), dtype=dtype) for _ in range(3))


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def _bwd_args():
    q, k, v = _qkv()
    return dict(q=q, k=k, v=v, o=_f32(BH, N, D), do=torch.zeros((BH, N, D), dtype=torch.bfloat16),
                lse=_f32(BH, N))


def test_well_formed_calls_reach_the_library(stub):
    q, k, v = _qkv()
    binding.attn_fwd(q, k, v, out=_f32(BH, N, D), lse=_f32(BH, N), stream=S)
    binding.attn_fwd(q, k, v, lse=False, stream=S)
    binding.attn_fwd_budget(q, k, v, 50000, out=_f32(BH, N, D), stream=S)
    binding.attn_fwd_splitk(q[:, :1].contiguous(), k, v, 2, out=_f32(BH, 1, D),
                            lse=_f32(BH, 1), workspace=torch.zeros(256, dtype=torch.uint8),
                            stream=S)
    binding.attn_fwd_blocksparse(q, k, v, torch.ones((1, 1, 1), dtype=torch.uint8), stream=S)
    binding.attn_fwd_smallcache(q, k, v, 3000, out=_f32(BH, N, D), stream=S)
    a = _bwd_args()
    binding.attn_bwd(**a, grads=(_f32(BH, N, D), _f32(BH, N, D), _f32(BH, N, D)), stream=S)
    binding.attn_bwd_smallcache(**a, m_elems=3000, stream=S)
    for name in ("attn_fwd", "attn_fwd_budget", "attn_fwd_splitk", "attn_fwd_blocksparse",
                 "attn_fwd_smallcache", "attn_bwd", "attn_bwd_smallcache"):
        assert name in stub.calls


def _no_launch(stub, fn, *args, **kw):
    with pytest.raises((ValueError, TypeError)):
        fn(*args, **kw)
    launched = [c for c in stub.calls if not c.endswith("_workspace_size")]
    assert launched == [], f"library entry point reached: {launched}"


FWD_OUT_CASES = {
    "out bf16": dict(out=torch.zeros((BH, N, D), dtype=torch.bfloat16)),
    "out short": dict(out=_f32(BH, N - 1, D)),
    "out wide": dict(out=_f32(BH, N, 2 * D)),
    "out strided": dict(out=_f32(BH, D, N).transpose(1, 2)),
    "out not a tensor": dict(out=[0.0]),
    "lse bf16": dict(lse=torch.zeros((BH, N), dtype=torch.bfloat16)),
    "lse short": dict(lse=_f32(BH, N - 1)),
    "lse 3-d": dict(lse=_f32(BH, N, 1)),
}


@pytest.mark.parametrize("case", list(FWD_OUT_CASES))
@pytest.mark.parametrize("entry", ["attn_fwd", "attn_fwd_budget", "attn_fwd_smallcache",
                                   "attn_fwd_blocksparse"])
def test_forward_outputs_checked(stub, entry, case):
    q, k, v = _qkv()
    kw = dict(FWD_OUT_CASES[case], stream=S)
    fn = getattr(binding, entry)
    if entry == "attn_fwd":
        _no_launch(stub, fn, q, k, v, **kw)
    elif entry == "attn_fwd_blocksparse":
        _no_launch(stub, fn, q, k, v, torch.ones((1, 1, 1), dtype=torch.uint8), **kw)
    else:
        _no_launch(stub, fn, q, k, v, 3000, **kw)


def test_splitk_outputs_checked(stub):
    q, k, v = _qkv()
    q1 = q[:, :3].contiguous()
    _no_launch(stub, binding.attn_fwd_splitk, q1, k, v, out=_f32(BH, N, D), stream=S)
    _no_launch(stub, binding.attn_fwd_splitk, q1, k, v, lse=_f32(BH, N), stream=S)
    _no_launch(stub, binding.attn_fwd_splitk, q1, k, v,
               workspace=torch.zeros((16, 16), dtype=torch.uint8).t(), stream=S)


INPUT_CASES = {
    "k shorter": lambda: (_qkv()[0], _qkv(n=N - 1)[1], _qkv()[2]),
    "v fp32": lambda: (_qkv()[0], _qkv()[1], _qkv(torch.float32)[2]),
    "q fp16": lambda: (torch.zeros((BH, N, D), dtype=torch.float16),) + _qkv()[1:],
    "q strided": lambda: (torch.zeros((BH, D, N), dtype=torch.bfloat16).transpose(1, 2),)
    + _qkv()[1:],
    "q 2-d": lambda: (torch.zeros((N, D), dtype=torch.bfloat16),) + _qkv()[1:],
}


@pytest.mark.parametrize("case", list(INPUT_CASES))
def test_forward_inputs_checked(stub, case):
    q, k, v = INPUT_CASES[case]()
    _no_launch(stub, binding.attn_fwd, q, k, v, stream=S)


BWD_CASES = {
    "O bf16": dict(o=torch.zeros((BH, N, D), dtype=torch.bfloat16)),
    "O short": dict(o=_f32(BH, N - 1, D)),
    "dO fp32": dict(do=_f32(BH, N, D)),
    "dO short": dict(do=torch.zeros((BH, N - 1, D), dtype=torch.bfloat16)),
    "lse bf16": dict(lse=torch.zeros((BH, N), dtype=torch.bfloat16)),
    "lse short": dict(lse=_f32(BH, N - 2)),
    "lse missing": dict(lse=None),
    "k shorter": dict(k=torch.zeros((BH, N - 1, D), dtype=torch.bfloat16)),
    "v fp32": dict(v=_f32(BH, N, D)),
    "dQ short": dict(grads=(_f32(BH, N - 1, D), _f32(BH, N, D), _f32(BH, N, D))),
    "dK bf16": dict(grads=(_f32(BH, N, D), torch.zeros((BH, N, D), dtype=torch.bfloat16),
                           _f32(BH, N, D))),
    "dV strided": dict(grads=(_f32(BH, N, D), _f32(BH, N, D), _f32(BH, D, N).transpose(1, 2))),
    "two grads": dict(grads=(_f32(BH, N, D), _f32(BH, N, D))),
    "workspace strided": dict(workspace=torch.zeros((16, 16), dtype=torch.uint8).t()),
}


@pytest.mark.parametrize("case", list(BWD_CASES))
@pytest.mark.parametrize("entry", ["attn_bwd", "attn_bwd_smallcache"])
def test_backward_buffers_checked(stub, entry, case):
    a = _bwd_args()
    a.update(BWD_CASES[case])
    if entry == "attn_bwd_smallcache":
        a["m_elems"] = 3000
    _no_launch(stub, getattr(binding, entry), **a, stream=S)


def test_block_mask_checked(stub):
    q, k, v = _qkv()
    for bad in (torch.ones((1, 1, 1), dtype=torch.float32), torch.ones((1, 2, 2), dtype=torch.uint8),
                torch.ones((3, 1, 1), dtype=torch.uint8), torch.ones((1, 1), dtype=torch.uint8),
                [[1]]):
        _no_launch(stub, binding.attn_fwd_blocksparse, q, k, v, bad, stream=S)


def test_device_mismatch_rejected(monkeypatch):
    """A tensor that is not on the GPU is rejected before the library loads."""
    lib = _StubLib()
    monkeypatch.setattr(binding, "lib", lambda path=None: lib)
    q, k, v = _qkv()
    with pytest.raises(ValueError):
        binding.attn_fwd(q, k, v, stream=S)
    assert lib.calls == []
