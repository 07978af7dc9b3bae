"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

No call here reaches a launch: every argument set is invalid in a way the
host-side validation catches first (fake device addresses are never
dereferenced).
"""

import ctypes

import numpy as np
import os
import re

import pytest

import paged_kv_attention_loc_amd as msgl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msgl.h")

OK, NULL, SHAPE, UNSUP, WS, RANGE, HIP = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def _lib():
    if not os.path.exists(msgl.library_path()):
        pytest.fail("libmsgl.so is not built (run __graft_entry__.build())")
    return msgl.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(msgl_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("msgl_store_kv", "msgl_paged_decode", "msgl_paged_extend",
              "msgl_paged_decode_workspace_size", "msgl_status_string", "msgl_abi_version",
              "msgl_debug_gather_kv"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = _lib()
    assert lib.msgl_abi_version() == 2
    for s in range(7):
        assert lib.msgl_status_string(s)
    assert lib.msgl_status_string(99) == b"unknown status"


def _pool(**kw):
    p = dict(data=FAKE, num_layers=2, num_pages=64, page_size=16, num_kv_heads=2, head_dim=128)
    p.update(kw)
    return msgl._Pool(p["data"], p["num_layers"], p["num_pages"], p["page_size"],
                      p["num_kv_heads"], p["head_dim"])


def _ws_bytes(batch, hq, d, max_len):
    """A piece map (int2 per request), then per launch of up to 2048
    requests the fp32 partials of its pieces: at most
    min(512 ranges, ceil(b * (max_len + 63) / 16)) + b (lengths are padded
    to tiles of up to 64 tokens before the split into ranges of >= 16)."""
    a256 = lambda x: -(-x // 256) * 256
    pieces = 0
    for b0 in range(0, batch, 2048):
        b = min(2048, batch - b0)
        pieces += min(512, -(-b * (max_len + 63) // 16)) + b
    return a256(batch * 8) + a256(pieces * hq * d * 4) + pieces * hq * 8


def test_workspace_size_is_host_arithmetic():
    # (batch, num_qo_heads, head_dim, max_seq_len, page_size)
    lib = _lib()
    f = lib.msgl_paged_decode_workspace_size
    n = f(64, 32, 128, 4096, 16)
    assert n == _ws_bytes(64, 32, 128, 4096)
    assert f(8, 32, 128, 512, 16) == _ws_bytes(8, 32, 128, 512)  # 296 pieces
    assert f(3000, 32, 128, 1000, 1) == _ws_bytes(3000, 32, 128, 1000)  # two launches
    assert f(0, 32, 128, 4096, 16) == 0
    assert f(-1, 32, 128, 4096, 16) == 0 and f(4, 32, 128, 4096, 0) == 0
    # the page size does not change the layout
    assert f(64, 32, 128, 4096, 1) == n == f(64, 32, 128, 4096, 13)
    # monotone in batch and length, so one allocation serves smaller calls
    assert f(32, 32, 128, 4096, 16) <= n and f(64, 32, 128, 2048, 16) <= n


def _decode_piece_ids(lens, kb):
    """The piece ids the decode kernel writes for one launch: lengths padded
    to whole tiles of kb tokens and laid end to end, split into ranges of
    per = roundup(max(16, ceil(T / 512)), kb) tokens; a request spread over
    several ranges writes piece i + r from range i."""
    pad = [-(-max(L, 0) // kb) * kb for L in lens]
    pre = np.concatenate([[0], np.cumsum(pad)])
    T = int(pre[-1])
    per = -(-max(16, -(-T // 512)) // kb) * kb
    ids = []
    for r, L in enumerate(lens):
        if L <= 0:
            continue
        first = int(pre[r]) // per
        pieces = (int(pre[r + 1]) - 1) // per - first + 1
        if pieces > 1:
            ids += [first + i + r for i in range(pieces)]
    return ids


def test_workspace_holds_every_piece_the_split_writes():
    # random and adversarial length mixes (short rows padded to a tile
    # push the split past batch * max_seq_len tokens), every tile size the
    # decode kernel uses
    lib = _lib()
    f = lib.msgl_paged_decode_workspace_size
    rng = np.random.default_rng(5)
    cases = [[17] * 100, [65] * 100, [1] * 300 + [40], [9] * 2048, [4096] * 64, [1]]
    cases += [list(rng.integers(0, int(rng.integers(1, 3000)), int(rng.integers(1, 400))))
              for _ in range(200)]
    for lens in cases:
        b, max_len = len(lens), max(max(lens), 1)
        hq, d = 8, 64
        n = f(b, hq, d, max_len, 16)
        map_bytes = -(-b * 8 // 256) * 256
        capacity = (n - map_bytes) // (hq * (d * 4 + 8))  # pieces the partials hold
        for kb in (8, 16, 32, 64):
            ids = _decode_piece_ids(lens, kb)
            assert not ids or max(ids) < capacity, (b, max_len, kb)


def _extend_split_bytes(T, hq, hkv, d, max_len, cus=256, forced=None):
    """Key shares of a small extend and their workspace: shares for one
    workgroup per CU when the 256-row tiles (ceil(T * G / 256) per kv head)
    are fewer than the CUs, at most 8 and at most one per 512 keys of the
    longest row; fp32 o (T, Hq, shares, d), 256-byte aligned, then
    (m, l)."""
    G = hq // hkv
    tiles = -(-T * G // 256) * hkv
    if forced is not None:
        sp = min(max(forced, 1), 8)
    elif tiles >= cus:
        sp = 1
    else:
        sp = max(1, min(-(-cus // tiles), 8, max(1, max_len // 512)))
    if sp <= 1:
        return 0
    return -(-(T * hq * sp * d * 4) // 256) * 256 + T * hq * sp * 8


def test_extend_workspace_size_is_host_arithmetic(monkeypatch):
    # no GPU here: the library takes 256 compute units
    lib = _lib()
    f = lib.msgl_paged_extend_workspace_size
    monkeypatch.delenv("MSGL_EXTEND_SPLITS", raising=False)
    for hkv, d, T, max_len, hq in [(1, 128, 8192, 2560, 4), (8, 128, 512, 9216, 32), (2, 64, 591, 701, 8),
                                   (8, 128, 8192, 2560, 32), (1, 128, 4096, 16384, 4), (8, 128, 100, 100, 32),
                                   (1, 64, 4096, 8192, 8)]:
        pool = _pool(num_kv_heads=hkv, head_dim=d)
        assert f(ctypes.byref(pool), T, max_len, hq) == _extend_split_bytes(T, hq, hkv, d, max_len), \
            (hkv, d, T, max_len, hq)
    pool = _pool(num_kv_heads=8, head_dim=128)
    assert f(ctypes.byref(pool), 8192, 2560, 32) == 0  # 1024 tiles: no split
    assert f(None, 512, 2560, 32) == 0 and f(ctypes.byref(pool), 0, 2560, 32) == 0
    assert f(ctypes.byref(pool), 512, 2560, 30) == 0  # Hq not a multiple of Hkv
    assert f(ctypes.byref(pool), 512, 9216, 32) > 0  # 16 tiles of 64 rows x 8 heads, long rows
    assert f(ctypes.byref(pool), 512, 600, 32) == 0  # the same with short rows: unsplit
    monkeypatch.setenv("MSGL_EXTEND_SPLITS", "3")
    assert f(ctypes.byref(pool), 8192, 2560, 32) == _extend_split_bytes(8192, 32, 8, 128, 2560, forced=3)
    monkeypatch.setenv("MSGL_EXTEND_SPLITS", "1")
    assert f(ctypes.byref(pool), 512, 9216, 32) == 0


def test_store_kv_rejects_bad_arguments_without_launch():
    lib = _lib()
    p = _pool()
    f = lib.msgl_store_kv
    assert f(None, 0, FAKE, 256, FAKE, 256, FAKE, 4, None) == NULL
    assert f(ctypes.byref(_pool(data=0)), 0, FAKE, 256, FAKE, 256, FAKE, 4, None) == NULL
    assert f(ctypes.byref(p), 2, FAKE, 256, FAKE, 256, FAKE, 4, None) == SHAPE  # layer
    assert f(ctypes.byref(p), -1, FAKE, 256, FAKE, 256, FAKE, 4, None) == SHAPE
    assert f(ctypes.byref(p), 0, None, 256, FAKE, 256, FAKE, 4, None) == NULL
    assert f(ctypes.byref(p), 0, FAKE, 255, FAKE, 256, FAKE, 4, None) == SHAPE  # stride < row
    assert f(ctypes.byref(p), 0, FAKE, 256, FAKE, 256, FAKE, -1, None) == SHAPE
    assert f(ctypes.byref(p), 0, FAKE + 1, 256, FAKE, 256, FAKE, 4, None) == SHAPE  # odd address
    assert f(ctypes.byref(p), 0, FAKE, 256, FAKE, 256, FAKE, 0, None) == OK  # empty: no-op
    assert f(ctypes.byref(_pool(page_size=0)), 0, FAKE, 256, FAKE, 256, FAKE, 4, None) == SHAPE


def _decode(lib, pool, **kw):
    a = dict(layer=0, q=FAKE, q_stride=32 * 128, out=FAKE, pt=FAKE, pt_stride=256, ti=FAKE,
             sl=FAKE, batch=4, hq=32, max_len=4096, scale=0.088, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lib.msgl_paged_decode(ctypes.byref(pool) if pool is not None else None, a["layer"],
                                 a["q"], a["q_stride"], a["out"], a["pt"], a["pt_stride"],
                                 a["ti"], a["sl"], a["batch"], a["hq"], a["max_len"], a["scale"],
                                 a["ws"], a["ws_bytes"], None)


def test_decode_rejects_bad_arguments_without_launch():
    lib = _lib()
    p = _pool(num_kv_heads=8)
    assert _decode(lib, None) == NULL
    assert _decode(lib, p, q=None) == NULL
    assert _decode(lib, p, sl=None) == NULL
    assert _decode(lib, p, hq=30) == SHAPE  # not a multiple of kv heads
    assert _decode(lib, p, hq=8 * 17) == UNSUP  # group above 16
    assert _decode(lib, _pool(num_kv_heads=8, head_dim=96), q_stride=32 * 96) == UNSUP
    assert _decode(lib, p, q_stride=32 * 128 - 8) == SHAPE
    assert _decode(lib, p, q=FAKE + 8) == SHAPE  # misaligned
    assert _decode(lib, p, pt_stride=255) == SHAPE  # rows too short for max_seq_len
    assert _decode(lib, p, ws_bytes=16) == WS
    assert _decode(lib, p, ws=None) == WS
    assert _decode(lib, p, batch=-1) == SHAPE
    assert _decode(lib, p, batch=0) == OK
    assert _decode(lib, p, layer=5) == SHAPE
    assert _decode(lib, p, scale=0.0) == SHAPE
    assert _decode(lib, p, scale=float("nan")) == SHAPE
    # one (K or V, layer) sub-tensor of 2^32 bytes or more
    assert _decode(lib, _pool(num_kv_heads=8, num_pages=1 << 17, page_size=16)) == UNSUP
    # the longest sequence: 2048 requests of it, each padded to whole tiles
    # of up to 64 tokens, still sum below 2^31 tokens
    longest = (2**31 - 1) // 2048 - 64
    assert 2048 * (longest + 64) < 2**31
    big_pt = -(-(longest + 1) // 16)
    assert _decode(lib, p, max_len=longest + 1, pt_stride=big_pt, ws_bytes=1 << 40) == UNSUP
    # accepted: the call goes on to the workspace check (too small here, so
    # nothing is launched)
    assert _decode(lib, p, max_len=longest, pt_stride=big_pt, ws_bytes=16) == WS


def test_decode_noalloc_refuses_oversize_without_launch():
    # host arithmetic only: a batch whose workspace exceeds the library's
    # scratch is refused before any HIP call (this container has no GPU)
    lib = _lib()
    p = _pool(num_kv_heads=8)
    cap = lib.msgl_paged_decode_noalloc_max_workspace()
    assert cap == 64 << 20
    big = 8192
    assert lib.msgl_paged_decode_workspace_size(big, 32, 128, 4096, 16) > cap
    f = lib.msgl_paged_decode_noalloc
    assert f(ctypes.byref(p), 0, FAKE, 32 * 128, FAKE, FAKE, 256, FAKE, FAKE, big, 32, 4096, 0.088,
             None) == WS
    assert f(None, 0, FAKE, 32 * 128, FAKE, FAKE, 256, FAKE, FAKE, 4, 32, 4096, 0.088, None) == NULL
    assert f(ctypes.byref(p), 0, FAKE, 32 * 128, FAKE, FAKE, 256, FAKE, FAKE, 0, 32, 4096, 0.088,
             None) == OK


def _extend_split(lib, pool, ws, ws_bytes, **kw):
    a = dict(layer=0, q=FAKE, q_stride=32 * 128, out=FAKE, pt=FAKE, pt_stride=256, ti=FAKE,
             pl=FAKE, el=FAKE, cu=FAKE, batch=2, total=100, max_ext=64, max_len=4096, hq=32,
             scale=0.088)
    a.update(kw)
    return lib.msgl_paged_extend_split(ctypes.byref(pool) if pool is not None else None, a["layer"],
                                       a["q"], a["q_stride"], a["out"], a["pt"], a["pt_stride"], a["ti"],
                                       a["pl"], a["el"], a["cu"], a["batch"], a["total"], a["max_ext"],
                                       a["max_len"], a["hq"], a["scale"], ws, ws_bytes, None)


def test_extend_split_checks_its_workspace_without_launch(monkeypatch):
    # a call small enough to split (16 tiles of 256 rows, 4096-key rows):
    # the workspace is checked before anything touches the GPU
    monkeypatch.delenv("MSGL_EXTEND_SPLITS", raising=False)
    lib = _lib()
    p = _pool(num_kv_heads=8)
    need = lib.msgl_paged_extend_workspace_size(ctypes.byref(p), 100, 4096, 32)
    assert need == _extend_split_bytes(100, 32, 8, 128, 4096) > 0
    assert _extend_split(lib, p, FAKE, need - 1) == WS
    assert _extend_split(lib, p, FAKE, 16) == WS
    assert _extend_split(lib, p, FAKE + 64, need) == SHAPE  # misaligned
    assert _extend_split(lib, None, FAKE, need) == NULL  # no pool: the plain extend's checks


def _extend(lib, pool, **kw):
    a = dict(layer=0, q=FAKE, q_stride=32 * 128, out=FAKE, pt=FAKE, pt_stride=256, ti=FAKE,
             pl=FAKE, el=FAKE, cu=FAKE, batch=2, total=100, max_ext=64, max_len=4096, hq=32,
             scale=0.088)
    a.update(kw)
    return lib.msgl_paged_extend(ctypes.byref(pool) if pool is not None else None, a["layer"],
                                 a["q"], a["q_stride"], a["out"], a["pt"], a["pt_stride"], a["ti"],
                                 a["pl"], a["el"], a["cu"], a["batch"], a["total"], a["max_ext"],
                                 a["max_len"], a["hq"], a["scale"], None)


def test_extend_rejects_bad_arguments_without_launch():
    lib = _lib()
    p = _pool(num_kv_heads=8)
    assert _extend(lib, None) == NULL
    assert _extend(lib, p, cu=None) == NULL
    assert _extend(lib, p, hq=33) == SHAPE
    assert _extend(lib, _pool(num_kv_heads=8, head_dim=80), q_stride=32 * 80) == UNSUP
    assert _extend(lib, p, max_ext=5000) == SHAPE  # extend longer than the sequence bound
    assert _extend(lib, p, pt_stride=10) == SHAPE
    assert _extend(lib, p, out=FAKE + 2) == SHAPE
    assert _extend(lib, p, scale=-0.1) == SHAPE
    assert _extend(lib, _pool(num_kv_heads=8, num_pages=1 << 17, page_size=16)) == UNSUP
    assert _extend(lib, p, total=0) == OK
    assert _extend(lib, p, batch=0) == OK


def test_gather_rejects_bad_arguments_without_launch():
    lib = _lib()
    p = _pool()
    f = lib.msgl_debug_gather_kv
    assert f(ctypes.byref(p), 0, None, 16, 0, 10, FAKE, FAKE, None) == NULL
    assert f(ctypes.byref(p), 0, FAKE, 16, -1, 10, FAKE, FAKE, None) == SHAPE
    assert f(ctypes.byref(p), 0, FAKE, 1, 0, 40, FAKE, FAKE, None) == SHAPE  # row too short
    assert f(ctypes.byref(p), 0, FAKE, 16, 0, 0, FAKE, FAKE, None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("MSGL_LIBRARY", str(tmp_path / "missing.so"))
    saved = msgl._lib
    msgl._lib = None
    try:
        with pytest.raises(RuntimeError):
            msgl.load_library()
    finally:
        msgl._lib = saved


def test_rope_calls_reject_bad_arguments_without_launch():
    lib = _lib()
    P = ctypes.c_void_p
    f = lib.msgl_rope_store_kv
    f.restype = ctypes.c_int32
    f.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int64, P,
                  ctypes.c_int64, P, P, ctypes.c_int32, P, ctypes.c_int32, P]
    assert f(None, 0, None, 0, 0, None, 0, None, 0, None, None, 1, None, 1, None) == 1  # NULL pool
    fake = ctypes.c_void_p(0x1000)
    pool = msgl._Pool(fake.value, 1, 4, 16, 2, 128)
    # max_position 0
    assert f(ctypes.byref(pool), 0, None, 0, 0, fake, 256, fake, 256, fake, fake, 3, fake, 0,
             None) == 2
    # head_dim 96 is not supported
    pool96 = msgl._Pool(fake.value, 1, 4, 16, 2, 96)
    assert f(ctypes.byref(pool96), 0, None, 0, 0, fake, 192, fake, 192, fake, fake, 3, fake, 8,
             None) == 3
    # a q with too short a row
    assert f(ctypes.byref(pool), 0, fake, 64, 4, fake, 256, fake, 256, fake, fake, 3, fake, 8,
             None) == 2
    g = lib.msgl_rope_cos_sin_table
    g.restype = ctypes.c_int32
    g.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P]
    assert g(fake, 16, 63, 10000.0, None) == 2  # odd head_dim
    assert g(fake, 0, 64, 10000.0, None) == 2
    assert g(fake, 16, 64, -1.0, None) == 2
    assert g(None, 16, 64, 10000.0, None) == 1


def test_alloc_pages_rejects_bad_arguments_without_launch():
    lib = _lib()
    P = ctypes.c_void_p
    f = lib.msgl_alloc_pages
    f.restype = ctypes.c_int32
    f.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_int32, ctypes.c_int32,
                  P, ctypes.c_int64, P, P]
    fake = ctypes.c_void_p(0x1000)
    ok_args = [fake, fake, fake, 8, 4, fake, fake, fake, 2, 16, fake, 10, fake, None]
    bad = list(ok_args)
    bad[9] = 0  # page_size
    assert f(*bad) == 2
    bad = list(ok_args)
    bad[8] = -1  # batch
    assert f(*bad) == 2
    bad = list(ok_args)
    bad[1] = None  # num_free
    assert f(*bad) == 1
    bad = list(ok_args)
    bad[10] = None  # out_loc with a capacity
    assert f(*bad) == 1
