"""C ABI checks that need no GPU: the library loads, exports every function
include/aware_tiling.h declares, and rejects bad arguments before any HIP call
(CPU only; no compute call is made)."""
import ctypes
import os
import re

import pytest

from aware_tiling_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aware_tiling.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
BF16, F32 = binding.ATTN_BF16, binding.ATTN_F32


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.lib()


def test_header_declares_the_three_entry_points():
    names = header_functions()
    for f in ("attn_fwd", "attn_fwd_smallcache", "attn_bwd"):
        assert f in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = header_functions()
    assert names, "no declarations parsed"
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"
        assert name in binding.SIGNATURES, f"{name} has no binding signature"
    # and the binding binds nothing the header does not declare
    assert set(binding.SIGNATURES) == set(names)


def test_status_strings_and_version(lib):
    for code, name in binding.STATUS.items():
        assert lib.attn_status_string(code).decode() == name
    assert lib.attn_status_string(99).decode() == "ATTN_STATUS_UNKNOWN"
    assert re.fullmatch(r"\d+\.\d+\.\d+", lib.attn_version().decode())


def test_tile_listing(lib):
    """attn_fwd_tiles lists the compiled shapes, the default first, and
    attn_fwd_tile_info of the default agrees with attn_fwd's query block and
    on-chip count; unknown names are refused."""
    expect = {64: ["g2x64p"],
              128: ["d8x64", "r64c32", "r64c64", "r128c32", "r128c64", "r256c32", "r256c64"],
              256: ["d4x32b"]}
    for d, names in expect.items():
        assert binding.fwd_tiles(d) == names
        info = binding.fwd_tile_info(names[0], d)
        assert info["block_rows"] == lib.attn_fwd_query_block(d, BF16)
        assert info["onchip_elems"] == lib.attn_fwd_onchip_elems(d, BF16)
    for name in expect[128][1:]:  # sweep shapes: B_r = 32 x waves, B_c keys per tile
        info = binding.fwd_tile_info(name, 128)
        br, bc = (int(x) for x in name[1:].split("c"))
        assert (info["block_rows"], info["key_tile"]) == (br, bc)
    assert binding.fwd_tiles(96) == []
    z = ctypes.c_int64(0)
    assert lib.attn_fwd_tile_info(b"nope", 128, ctypes.byref(z), None, None) == UNSUPPORTED
    assert lib.attn_fwd_tile_info(b"d8x64", 64, None, None, None) == UNSUPPORTED
    assert lib.attn_fwd_tile_info(None, 128, None, None, None) == INVALID


FAKE = 0x1000  # aligned, never dereferenced: every call below fails validation first


def test_splitk_noalloc_validation(lib):
    """The allocation-free key-split call refuses, before any HIP call, a
    request whose partials exceed its device array, as well as the usual
    bad arguments."""
    def call(q=FAKE, bh=1, nq=4, nk=1000, d=128, splits=0, scale=0.125, dtype=BF16):
        return lib.attn_fwd_splitk_noalloc(q, FAKE, FAKE, FAKE, None, bh, nq, nk, d, scale,
                                           dtype, splits, None)
    assert call(bh=64, nq=200, nk=4096, splits=16) == WORKSPACE  # 64 MiB of partials
    assert lib.attn_fwd_splitk_workspace_size(64, 200, 4096, 128, 16) > \
        binding.SPLITK_NOALLOC_SCRATCH_BYTES
    assert call(q=None) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(dtype=F32) == UNSUPPORTED
    assert call(splits=300) == INVALID
    assert call(nk=0) == INVALID
    assert call(q=None, nq=0) == OK


def test_fwd_tile_validation(lib):
    def call(tile=b"r128c32", q=FAKE, o=FAKE, n=128, d=128, dtype=BF16, scale=0.125):
        return lib.attn_fwd_tile(tile, q, FAKE, FAKE, o, None, 1, n, d, scale, dtype, None)
    assert call(tile=None) == INVALID
    assert call(tile=b"nope") == UNSUPPORTED
    assert call(d=64) == UNSUPPORTED
    assert call(dtype=F32) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(o=FAKE + 8) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(q=None, o=None, n=0) == OK


def test_bwd_tile_listing_and_validation(lib):
    """attn_bwd_tiles lists the backward's compiled shapes, the default first
    (the one attn_bwd runs, whose on-chip count attn_bwd_onchip_elems
    reports); the names decode to keys per dK/dV workgroup, queries per dQ
    workgroup and keys per dQ tile; unknown names are refused before any
    launch."""
    expect = {128: ["k256q256c64", "k128q256c64", "k256q128c64", "k256q256c32"],
              64: ["k256q256c64"], 256: ["k128q128c64"]}
    for d, names in expect.items():
        assert binding.bwd_tiles(d) == names
        assert binding.bwd_tile_info(names[0], d)["onchip_elems"] == lib.attn_bwd_onchip_elems(d)
        for name in names:
            info = binding.bwd_tile_info(name, d)
            k, rest = name[1:].split("q")
            qb, c = rest.split("c")
            assert (info["keys_per_block"], info["queries_per_block"], info["key_tile"]) == (
                int(k), int(qb), int(c))
            assert info["onchip_elems"] >= d * d  # large-cache regime
    assert binding.bwd_tiles(96) == []
    assert lib.attn_bwd_tile_info(b"nope", 128, None, None, None, None) == UNSUPPORTED
    assert lib.attn_bwd_tile_info(b"k128q256c64", 64, None, None, None, None) == UNSUPPORTED
    assert lib.attn_bwd_tile_info(None, 128, None, None, None, None) == INVALID
    ws = lib.attn_bwd_workspace_size(2, 512, 128)

    def call(tile=b"k128q256c64", q=FAKE, dv=FAKE, d=128, dtype=BF16, w=FAKE * 256, n=512):
        return lib.attn_bwd_tile(tile, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dv, 2, n, d,
                                 0.08, dtype, w, ws, None)
    assert call(tile=None) == INVALID
    assert call(tile=b"nope") == UNSUPPORTED
    assert call(d=64) == UNSUPPORTED  # k128q256c64 exists only at d = 128
    assert call(dtype=F32) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(dv=FAKE + 8) == INVALID
    assert call(w=None) == WORKSPACE
    assert call(q=None, dv=None, n=0) == OK


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, bh=1, n=128, d=64, scale=0.125,
        dtype=BF16):
    return lib.attn_fwd(q, k, v, o, lse, bh, n, d, scale, dtype, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == INVALID
    assert fwd(lib, o=None) == INVALID
    assert fwd(lib, q=FAKE + 2) == INVALID  # misaligned
    assert fwd(lib, lse=FAKE + 4) == INVALID
    assert fwd(lib, d=96) == UNSUPPORTED
    assert fwd(lib, d=96, dtype=F32) == UNSUPPORTED
    assert fwd(lib, dtype=7) == UNSUPPORTED
    assert fwd(lib, scale=0.0) == INVALID
    assert fwd(lib, scale=-1.0) == INVALID
    assert fwd(lib, scale=float("nan")) == INVALID
    assert fwd(lib, scale=float("inf")) == INVALID
    assert fwd(lib, bh=-1) == INVALID
    assert fwd(lib, n=-5) == INVALID
    assert fwd(lib, n=1 << 25) == INVALID
    assert fwd(lib, bh=(1 << 9) + 1, n=1 << 20, d=64) == INVALID  # bh * n above 2^29 rows
    # empty problems are a no-op even with null pointers
    assert fwd(lib, q=None, k=None, v=None, o=None, n=0) == OK
    assert fwd(lib, q=None, k=None, v=None, o=None, bh=0) == OK


def test_fwd_tile_queries(lib):
    for d in (64, 128, 256):
        m = lib.attn_fwd_onchip_elems(d, BF16)
        b = lib.attn_fwd_query_block(d, BF16)
        assert b > 0 and b % 32 == 0
        # the fused kernel is the large-cache schedule: M >= d^2
        assert m >= d * d
    assert lib.attn_fwd_onchip_elems(96, BF16) == 0
    # the d = 128 default (256 query rows, 64-key tiles): Q and U blocks, (m, l),
    # both slots of the K and V rings, the current and the next score tile
    assert lib.attn_fwd_onchip_elems(128, BF16) == (2 * 256 * 128 + 2 * 256 + 4 * 64 * 128
                                                    + 2 * 256 * 64) == 131584
    for d in (64, 128, 256):
        assert lib.attn_fwd_query_block(d, F32) == 128
        # single-buffered fp32 tiles: Q and U blocks, (m, l), one K and one V
        # tile of 32 keys, one score tile
        assert lib.attn_fwd_onchip_elems(d, F32) == 2 * 128 * d + 2 * 128 + 2 * 32 * d + 128 * 32
    assert lib.attn_fwd_query_block(96, F32) == 0


def test_smallcache_validation(lib):
    d = 256
    ws = lib.attn_fwd_smallcache_workspace_size(8, 4096, d, 40000)
    b = lib.attn_smallcache_tile(d, 40000)
    if b == 0:
        pytest.skip("small-cache path not built")
    assert ws > 0
    # the page's small-cache regime is M < d^2; the call refuses M >= d^2
    assert lib.attn_smallcache_tile(d, d * d) == 0
    call = lambda m=40000, wsb=ws, w=FAKE * 256, q=FAKE: lib.attn_fwd_smallcache(
        q, FAKE, FAKE, FAKE, None, 8, 4096, d, 0.0625, BF16, m, w, wsb, None)
    assert call(m=d * d) == INVALID
    assert call(q=None) == INVALID
    assert call(w=None) == WORKSPACE
    assert call(wsb=ws - 1) == WORKSPACE
    assert call(w=FAKE * 256 + 16) == WORKSPACE  # not 256-byte aligned
    assert lib.attn_fwd_smallcache(FAKE, FAKE, FAKE, FAKE, None, 8, 4096, d, 0.0625, F32, 40000,
                                   FAKE, ws, None) == UNSUPPORTED


def test_budget_forward_validation(lib):
    # Q and U blocks 2*32*d, (m, l) 64, two slots of K and V 4*32*d, four partial
    # score tiles and the summed one 5*32*32
    assert lib.attn_fwd_budget_onchip_elems(256) == 2 * 32 * 256 + 64 + 4 * 32 * 256 + 5 * 1024
    assert lib.attn_fwd_budget_onchip_elems(256) == 54336 < 256 * 256
    assert lib.attn_fwd_budget_onchip_elems(128) == 29760
    assert lib.attn_fwd_budget_onchip_elems(64) == 0
    call = lambda m=54336, d=256, dtype=BF16, q=FAKE, bh=8, n=4096, scale=0.0625: \
        lib.attn_fwd_budget(q, FAKE, FAKE, FAKE, None, bh, n, d, scale, dtype, m, None)
    assert call(m=54335) == UNSUPPORTED  # the tile does not fit the budget
    assert call(dtype=F32) == UNSUPPORTED
    assert call(d=64) == UNSUPPORTED
    assert call(m=0) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(q=None) == INVALID
    assert call(bh=1 << 20, n=1 << 20) == INVALID  # more workgroups than a grid holds
    assert call(bh=(1 << 9) + 1, n=1 << 20) == INVALID  # bh * n above 2^29 rows
    assert call(q=None, n=0) == OK  # empty: no launch, no pointer needed


def test_bwd_validation(lib):
    ws = lib.attn_bwd_workspace_size(2, 512, 128)
    if lib.attn_bwd_workspace_size(2, 512, 128) == 0 and lib.attn_bwd(
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 512, 128, 0.08, BF16, FAKE,
            1 << 30, None) == UNSUPPORTED:
        pytest.skip("backward not built")
    call = lambda **kw: lib.attn_bwd(*[kw.get(x, FAKE) for x in
                                       ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")],
                                     2, 512, kw.get("d", 128), kw.get("scale", 0.08), BF16,
                                     kw.get("w", FAKE * 256), kw.get("wsb", ws), None)
    assert call(lse=None) == INVALID
    assert call(dv=None) == INVALID
    assert call(dq=FAKE + 8) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(scale=-0.5) == INVALID
    if ws > 0:
        assert call(wsb=ws - 1) == WORKSPACE
        assert call(w=None) == WORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.attn_fwd(q, q, q)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        binding.lib()


def test_library_links_no_oracle(lib):
    # the product library must not reference the oracle's symbols
    so = open(binding.LIB_PATH, "rb").read()
    assert b"oracle_attn" not in so
    with pytest.raises(AttributeError):
        getattr(ctypes.CDLL(binding.LIB_PATH), "oracle_attn_fwd_f64")


def test_smallcache_tile_selection(lib):
    # footprint(b) = max(b^2 + 2*2*b*ks, b*bd + R*(32*bd + b*32)), bd = min(b, d):
    # the score tile plus two slots of the Q and K panels (ks = 64 columns for
    # b = 128, 32 for b = 64), or the output tile plus R slots of the V and E
    # panels (R = 4 for b = 128, 2 for b = 64)
    assert lib.attn_smallcache_onchip_elems(128) == 128 * 128 + 4 * 128 * 64 == 49152
    assert lib.attn_smallcache_onchip_elems(64) == 12288
    assert lib.attn_smallcache_tile(256, 49152) == 128
    assert lib.attn_smallcache_tile(256, 49151) == 64
    assert lib.attn_smallcache_tile(256, 40960) == 64
    assert lib.attn_smallcache_tile(256, 12288) == 64
    assert lib.attn_smallcache_tile(256, 12287) == 0
    assert lib.attn_smallcache_tile(128, 16000) == 64  # b=128 would not be below d^2
    assert lib.attn_smallcache_tile(256, 65536) == 0  # not the small-cache regime
    assert lib.attn_smallcache_tile(64, 4000) == 0  # no tile fits below d^2 = 4096


def test_splitk_validation_and_sizes(lib):
    bh, nq, nk, d = 32, 1, 16384, 128
    call = lambda q=FAKE, o=FAKE, nq_=nq, nk_=nk, d_=d, s=8, w=FAKE * 256, wsb=1 << 30, \
        dt=BF16, scale=0.088: lib.attn_fwd_splitk(q, FAKE, FAKE, o, None, bh, nq_, nk_, d_,
                                                  scale, dt, s, w, wsb, None)
    assert call(q=None) == INVALID
    assert call(o=FAKE + 4) == INVALID
    assert call(nk_=0) == INVALID  # softmax over no keys
    assert call(s=-1) == INVALID
    assert call(s=257) == INVALID
    assert call(d_=96) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(scale=0.0) == INVALID
    assert call(q=None, o=None, nq_=0) == OK  # empty query set is a no-op
    # chunks are whole 64-key tiles: 16384 keys in 8 requested chunks -> 8 of 2048
    assert lib.attn_fwd_splitk_splits(bh, nq, nk, d, 8) == 8
    # 100 keys in 4 requested chunks -> chunks of 64 keys -> 2 chunks
    assert lib.attn_fwd_splitk_splits(bh, nq, 100, d, 4) == 2
    assert lib.attn_fwd_splitk_splits(bh, nq, 64, d, 4) == 1
    # workspace: splits x bh x nq x (d + 1) floats, each part 256-byte aligned
    ws = lib.attn_fwd_splitk_workspace_size(bh, nq, nk, d, 8)
    assert ws == ((8 * bh * nq * d * 4 + 255) // 256 + (8 * bh * nq * 4 + 255) // 256) * 256
    assert lib.attn_fwd_splitk_workspace_size(bh, nq, 64, d, 4) == 0  # one chunk: none needed
    assert call(w=None, wsb=ws) == WORKSPACE
    assert call(wsb=ws - 1) == WORKSPACE
    assert call(w=FAKE * 256 + 16, wsb=ws) == WORKSPACE
    # automatic choice: >= 1 chunk, never more than 256, >= 256 keys per chunk
    for (b_, q_, k_) in ((1, 1, 100), (32, 1, 131072), (8, 512, 8192), (64, 4096, 4096)):
        s = lib.attn_fwd_splitk_splits(b_, q_, k_, d, 0)
        assert 1 <= s <= 256
        assert s == 1 or (k_ + s - 1) // s >= 192


def test_bwd_onchip_elems(lib):
    # the larger of the two kernels' resident sets (every pipeline slot):
    # dK/dV 4 Bkv d + 4 Bq d + 4 Bq + 2 Bkv Bq with Bkv keys per workgroup
    # (256; 128 at d = 256) and Bq = 32 queries (64 at d = 64); dQ 3 Bqb d +
    # 2 Bqb + 4 Bc d + 2 Bqb Bc with Bqb queries per workgroup (256; 128 at
    # d = 256) and Bc = 64 keys; all >= d^2 (the large-cache regime)
    dkdv = lambda d, bkv, bq: 4 * bkv * d + 4 * bq * d + 4 * bq + 2 * bkv * bq
    dq = lambda d, bqb: 3 * bqb * d + 2 * bqb + 4 * 64 * d + 2 * bqb * 64
    assert lib.attn_bwd_onchip_elems(128) == max(dkdv(128, 256, 32), dq(128, 256)) == 164352
    assert lib.attn_bwd_onchip_elems(64) == max(dkdv(64, 256, 64), dq(64, 256))
    assert lib.attn_bwd_onchip_elems(256) == max(dkdv(256, 128, 32), dq(256, 128)) == 180480
    for d in (64, 128, 256):
        assert lib.attn_bwd_onchip_elems(d) >= d * d
    assert lib.attn_bwd_onchip_elems(96) == 0 and lib.attn_bwd_onchip_elems(-1) == 0


def test_bwd_smallcache_tile_selection_and_validation(lib):
    # footprint(b, stages) = max(2 b^2 + 4 b 16 stages, b^2 + 2 b 16 stages)
    tile, onchip = lib.attn_bwd_smallcache_tile, lib.attn_bwd_smallcache_onchip_elems
    assert (tile(256, 49152), onchip(256, 49152)) == (128, 49152)
    assert (tile(256, 40960), onchip(256, 40960)) == (128, 40960)
    assert (tile(256, 40959), onchip(256, 40959)) == (64, 16384)
    assert (tile(256, 16383), onchip(256, 16383)) == (64, 12288)
    assert tile(256, 12287) == 0
    assert (tile(128, 12288), onchip(128, 12288)) == (64, 12288)
    assert tile(128, 16384) == 0  # M >= d^2 is the large-cache regime
    assert tile(64, 4000) == 0  # nothing fits below d^2 = 4096
    b = 64
    npad = (300 + b - 1) // b * b
    ws = lib.attn_bwd_smallcache_workspace_size(2, 300, 128, 12288)
    assert ws == ((2 * 300 * 4 + 255) // 256 * 256
                  + 2 * ((2 * npad * npad * 2 + 255) // 256 * 256))
    call = lambda **kw: lib.attn_bwd_smallcache(
        *[kw.get(x, FAKE) for x in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")],
        2, 300, kw.get("d", 128), kw.get("scale", 0.08), kw.get("dt", BF16),
        kw.get("m", 12288), kw.get("w", FAKE * 256), kw.get("wsb", ws), None)
    assert call(lse=None) == INVALID
    assert call(dk=FAKE + 4) == INVALID
    assert call(d=64, m=4000) == UNSUPPORTED
    assert call(m=16384) == INVALID
    assert call(m=0) == INVALID
    assert call(d=256, m=12000) == UNSUPPORTED  # below d^2 but no tile fits
    assert call(dt=F32) == UNSUPPORTED
    assert call(wsb=ws - 1) == WORKSPACE
    assert call(w=None) == WORKSPACE
    assert call(w=FAKE * 256 + 32) == WORKSPACE


def test_blocksparse_validation_and_sizes(lib):
    bh, n, d = 4, 1000, 128
    nb = (n + 127) // 128
    cap = (n + 63) // 64
    ws = lib.attn_fwd_blocksparse_workspace_size(bh, n, bh)
    assert ws == ((bh * nb * 4 + 255) // 256 + (bh * nb * cap * 4 + 255) // 256) * 256
    assert lib.attn_fwd_blocksparse_workspace_size(bh, n, 1) < ws
    assert lib.attn_fwd_blocksparse_workspace_size(bh, n, 3) == 0  # 1 or bh only
    call = lambda q=FAKE, mask=FAKE, mh=bh, d_=d, dt=BF16, w=FAKE * 256, wsb=ws: \
        lib.attn_fwd_blocksparse(q, FAKE, FAKE, FAKE, None, bh, n, d_, 0.088, dt, mask, mh, w,
                                 wsb, None)
    assert call(q=None) == INVALID
    assert call(mask=None) == INVALID
    assert call(mh=2) == INVALID
    assert call(d_=96) == UNSUPPORTED
    assert call(dt=F32) == UNSUPPORTED
    assert call(w=None) == WORKSPACE
    assert call(wsb=ws - 1) == WORKSPACE
    assert call(w=FAKE * 256 + 64) == WORKSPACE
    assert lib.attn_fwd_blocksparse(None, None, None, None, None, 0, n, d, 0.088, BF16, None, 1,
                                    None, 0, None) == OK  # empty batch


def test_calib_mfma_loop_validation(lib):
    call = lambda out=FAKE, wgs=512, iters=10, amp=1.0: lib.attn_calib_mfma_loop(
        out, wgs, iters, amp, None)
    assert call(out=None) == INVALID
    assert call(out=FAKE + 4) == INVALID
    assert call(wgs=0) == INVALID
    assert call(wgs=1 << 31) == INVALID
    assert call(iters=0) == INVALID
    assert call(amp=float("nan")) == INVALID
    assert call(amp=float("inf")) == INVALID


def test_calib_stream_read_validation(lib):
    call = lambda src=FAKE, nb=1 << 20, out=FAKE, wgs=64: lib.attn_calib_stream_read(
        src, nb, out, wgs, None)
    assert call(src=None) == INVALID
    assert call(src=FAKE + 8) == INVALID
    assert call(nb=0) == INVALID
    assert call(nb=-16) == INVALID
    assert call(nb=(1 << 20) + 4) == INVALID
    assert call(out=None) == INVALID
    assert call(out=FAKE + 4) == INVALID
    assert call(wgs=0) == INVALID
    assert call(wgs=1 << 23) == INVALID
