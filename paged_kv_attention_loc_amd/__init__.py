"""Paged-KV attention for MI355X: Python binding of libmsgl.so.

Argument marshalling only: every step of store_kv, decode and extend runs in
the HIP kernels of ``libmsgl.so`` (see ``include/msgl.h`` for the contract).
PyTorch supplies device memory and the current stream.  There is no CPU or
PyTorch fallback: if the library is missing or the device is not gfx950,
the calls raise.

Objects follow the Mini-SGLang pages ("Code Notes: mini-sglang", Engine
Layer table, BaseKVCachePool row; Scheduler Layer table, TableManager row):
a bf16 pool shaped (2, num_layers, num_pages, page_size, kv_heads, head_dim),
``out_loc`` slots for store_kv, and one ``page_table`` row per request
picked by ``table_idx``.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MsglError",
    "library_path",
    "load_library",
    "abi_version",
    "msgl_store_kv",
    "msgl_paged_decode",
    "msgl_paged_decode_workspace_size",
    "msgl_paged_decode_noalloc",
    "paged_decode_noalloc",
    "paged_decode_noalloc_max_workspace",
    "msgl_paged_extend",
    "msgl_paged_extend_workspace_size",
    "paged_extend_workspace_size",
    "msgl_debug_gather_kv",
    "store_kv",
    "paged_decode",
    "paged_decode_workspace_size",
    "decode_workspace",
    "paged_extend",
    "debug_gather_kv",
    "DecodeGraph",
    "DecodeGraphRunner",
    "msgl_rope_store_kv",
    "msgl_rope_cos_sin_table",
    "rope_store_kv",
    "rope_cos_sin_table",
    "msgl_alloc_pages",
    "alloc_pages",
    "msgl_paged_mixed",
    "paged_mixed",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmsgl.so"
_lib = None

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_UNSUPPORTED", 4: "ERR_WORKSPACE",
          5: "ERR_RANGE", 6: "ERR_HIP"}


class MsglError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({text})")
        self.status = status


class _Pool(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("num_layers", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


def library_path() -> str:
    return os.environ.get("MSGL_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libmsgl.so (built in-tree by ``paged_kv_attention_loc_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_attention_loc_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    PP = ctypes.POINTER(_Pool)
    lib.msgl_abi_version.restype = I32
    lib.msgl_abi_version.argtypes = []
    lib.msgl_status_string.restype = ctypes.c_char_p
    lib.msgl_status_string.argtypes = [I32]
    lib.msgl_store_kv.restype = I32
    lib.msgl_store_kv.argtypes = [PP, I32, P, I64, P, I64, P, I32, P]
    lib.msgl_paged_decode_workspace_size.restype = SZ
    lib.msgl_paged_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.msgl_paged_decode.restype = I32
    lib.msgl_paged_decode.argtypes = [PP, I32, P, I64, P, P, I32, P, P, I32, I32, I32, F32, P, SZ, P]
    lib.msgl_paged_decode_noalloc.restype = I32
    lib.msgl_paged_decode_noalloc.argtypes = [PP, I32, P, I64, P, P, I32, P, P, I32, I32, I32, F32, P]
    lib.msgl_paged_decode_noalloc_max_workspace.restype = SZ
    lib.msgl_paged_decode_noalloc_max_workspace.argtypes = []
    lib.msgl_paged_extend.restype = I32
    lib.msgl_paged_extend.argtypes = [PP, I32, P, I64, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32,
                                      F32, P]
    lib.msgl_paged_extend_workspace_size.restype = SZ
    lib.msgl_paged_extend_workspace_size.argtypes = [PP, I32, I32, I32]
    lib.msgl_paged_extend_split.restype = I32
    lib.msgl_paged_extend_split.argtypes = [PP, I32, P, I64, P, P, I32, P, P, P, P, I32, I32, I32, I32,
                                            I32, F32, P, SZ, P]
    lib.msgl_debug_gather_kv.restype = I32
    lib.msgl_debug_gather_kv.argtypes = [PP, I32, P, I32, I32, I32, P, P, P]
    lib.msgl_rope_store_kv.restype = I32
    lib.msgl_rope_store_kv.argtypes = [PP, I32, P, I64, I32, P, I64, P, I64, P, P, I32, P, I32, P]
    lib.msgl_rope_cos_sin_table.restype = I32
    lib.msgl_rope_cos_sin_table.argtypes = [P, I32, I32, ctypes.c_double, P]
    lib.msgl_paged_mixed.restype = I32
    lib.msgl_paged_mixed.argtypes = [PP, I32, P, I64, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32,
                                     F32, P, SZ, P]
    lib.msgl_alloc_pages.restype = I32
    lib.msgl_alloc_pages.argtypes = [P, P, P, I32, I32, P, P, P, I32, I32, P, I64, P, P]
    lib.msgl_decode_graph_create.restype = I32
    lib.msgl_decode_graph_create.argtypes = [PP, I32, P, I64, P, I64, P, P, I64, P, P, I32, P, P, I32,
                                             I32, I32, F32, P, SZ, ctypes.POINTER(P)]
    lib.msgl_decode_graph_launch.restype = I32
    lib.msgl_decode_graph_launch.argtypes = [P, P]
    lib.msgl_decode_graph_destroy.restype = I32
    lib.msgl_decode_graph_destroy.argtypes = [P]
    lib.msgl_decode_graph_runner_create.restype = I32
    lib.msgl_decode_graph_runner_create.argtypes = lib.msgl_decode_graph_create.argtypes
    lib.msgl_decode_graph_runner_pick.restype = I32
    lib.msgl_decode_graph_runner_pick.argtypes = [P, I32]
    lib.msgl_decode_graph_runner_launch.restype = I32
    lib.msgl_decode_graph_runner_launch.argtypes = [P, I32, P]
    lib.msgl_decode_graph_runner_destroy.restype = I32
    lib.msgl_decode_graph_runner_destroy.argtypes = [P]
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().msgl_abi_version())


def _check(status: int, where: str):
    if status != 0:
        text = load_library().msgl_status_string(status).decode()
        raise MsglError(status, where, text)


def _pool_struct(pool: torch.Tensor) -> _Pool:
    if pool.dim() != 6 or pool.shape[0] != 2:
        raise ValueError("pool must be shaped (2, num_layers, num_pages, page_size, kv_heads, head_dim)")
    if pool.dtype != torch.bfloat16 or not pool.is_cuda or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous bf16 CUDA tensor")
    _, nl, npg, ps, hkv, d = pool.shape
    return _Pool(pool.data_ptr(), nl, npg, ps, hkv, d)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _rows(t: torch.Tensor, name: str, heads: int, d: int) -> int:
    """Row stride of a (rows, heads, d) bf16 CUDA tensor with heads and dims packed."""
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise ValueError(f"{name} must be a bf16 CUDA tensor")
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != d:
        raise ValueError(f"{name} must be shaped (rows, {heads}, {d}), got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError(f"{name}: heads and head_dim must be contiguous inside a row")
    return int(t.stride(0)) if t.shape[0] > 1 else heads * d


def _i32(t: torch.Tensor, name: str) -> int:
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor")
    return t.data_ptr()


def msgl_store_kv(pool: torch.Tensor, layer: int, k: torch.Tensor, v: torch.Tensor,
                  out_loc: torch.Tensor) -> None:
    """Write row t of k / v into slot out_loc[t] of layer ``layer`` (negative = skip)."""
    ps = _pool_struct(pool)
    T = int(out_loc.numel())
    ks = _rows(k, "k", ps.num_kv_heads, ps.head_dim)
    vs = _rows(v, "v", ps.num_kv_heads, ps.head_dim)
    if k.shape[0] != T or v.shape[0] != T:
        raise ValueError("k, v and out_loc must have the same number of rows")
    st = load_library().msgl_store_kv(ctypes.byref(ps), layer, k.data_ptr(), ks, v.data_ptr(), vs,
                                      _i32(out_loc, "out_loc"), T, _stream(pool))
    _check(st, "msgl_store_kv")


def msgl_paged_decode_workspace_size(batch: int, num_qo_heads: int, head_dim: int,
                                     max_seq_len: int, page_size: int) -> int:
    """Bytes of decode workspace (piece map and fp32 partials of split
    requests); 0 for an empty batch.  Contents need no initialisation."""
    return int(load_library().msgl_paged_decode_workspace_size(batch, num_qo_heads, head_dim,
                                                               max_seq_len, page_size))


def decode_workspace(batch: int, num_qo_heads: int, head_dim: int, max_seq_len: int,
                     page_size: int, device="cuda") -> Optional[torch.Tensor]:
    """A zeroed decode workspace for calls up to these sizes (None if no
    call of that size needs one)."""
    need = msgl_paged_decode_workspace_size(batch, num_qo_heads, head_dim, max_seq_len, page_size)
    if need == 0:
        return None
    return torch.zeros(need, dtype=torch.uint8, device=device)


def msgl_paged_decode(pool: torch.Tensor, layer: int, q: torch.Tensor, page_table: torch.Tensor,
                      table_idx: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                      sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention: q (B, Hq, d) -> out (B, Hq, d), reading each
    request's seq_lens[r] tokens through page_table row table_idx[r]."""
    ps = _pool_struct(pool)
    B, hq, d = q.shape
    qs = _rows(q, "q", hq, d)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(B, hq, d, max_seq_len, ps.page_size, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if page_table.dim() != 2:
        raise ValueError("page_table must be 2-D (rows, entries)")
    st = load_library().msgl_paged_decode(
        ctypes.byref(ps), layer, q.data_ptr(), qs, out.data_ptr(), _i32(page_table, "page_table"),
        int(page_table.shape[1]), _i32(table_idx, "table_idx"), _i32(seq_lens, "seq_lens"), B, hq,
        int(max_seq_len), float(sm_scale), ws_ptr, ws_bytes, _stream(q))
    _check(st, "msgl_paged_decode")
    return out


def msgl_paged_decode_noalloc(pool: torch.Tensor, layer: int, q: torch.Tensor,
                              page_table: torch.Tensor, table_idx: torch.Tensor,
                              seq_lens: torch.Tensor, max_seq_len: int,
                              sm_scale: Optional[float] = None,
                              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_decode with the library's own device scratch instead of a
    workspace (msgl_paged_decode_noalloc): no device allocation in the call
    when ``out`` is given.  Calls on one GPU must not overlap in time."""
    ps = _pool_struct(pool)
    B, hq, d = q.shape
    qs = _rows(q, "q", hq, d)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if page_table.dim() != 2:
        raise ValueError("page_table must be 2-D (rows, entries)")
    st = load_library().msgl_paged_decode_noalloc(
        ctypes.byref(ps), layer, q.data_ptr(), qs, out.data_ptr(), _i32(page_table, "page_table"),
        int(page_table.shape[1]), _i32(table_idx, "table_idx"), _i32(seq_lens, "seq_lens"), B, hq,
        int(max_seq_len), float(sm_scale), _stream(q))
    _check(st, "msgl_paged_decode_noalloc")
    return out


def paged_decode_noalloc_max_workspace() -> int:
    """Bytes of the device scratch msgl_paged_decode_noalloc draws on."""
    return int(load_library().msgl_paged_decode_noalloc_max_workspace())


def msgl_paged_extend(pool: torch.Tensor, layer: int, q: torch.Tensor, page_table: torch.Tensor,
                      table_idx: torch.Tensor, prefix_lens: torch.Tensor, extend_lens: torch.Tensor,
                      cu_extend_lens: torch.Tensor, max_extend_len: int, max_seq_len: int,
                      sm_scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      split: bool = True) -> torch.Tensor:
    """Causal extend attention: q (sum E, Hq, d) -> out (sum E, Hq, d).
    A call too small to fill the device splits its keys over more
    workgroups (msgl_paged_extend_split) when `split` is true: its workspace
    is `workspace`, or allocated here when that is None."""
    ps = _pool_struct(pool)
    T, hq, d = q.shape
    qs = _rows(q, "q", hq, d)
    B = int(table_idx.numel())
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.bfloat16, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if page_table.dim() != 2:
        raise ValueError("page_table must be 2-D (rows, entries)")
    lib = load_library()
    args = (ctypes.byref(ps), layer, q.data_ptr(), qs, out.data_ptr(), _i32(page_table, "page_table"),
            int(page_table.shape[1]), _i32(table_idx, "table_idx"), _i32(prefix_lens, "prefix_lens"),
            _i32(extend_lens, "extend_lens"), _i32(cu_extend_lens, "cu_extend_lens"), B, T,
            int(max_extend_len), int(max_seq_len), hq, float(sm_scale))
    need = int(lib.msgl_paged_extend_workspace_size(ctypes.byref(ps), T, int(max_seq_len), hq)) if split else 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        st = lib.msgl_paged_extend_split(*args, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream(q))
        _check(st, "msgl_paged_extend_split")
    else:
        st = lib.msgl_paged_extend(*args, _stream(q))
        _check(st, "msgl_paged_extend")
    return out


def msgl_paged_extend_workspace_size(pool: torch.Tensor, total_extend_tokens: int, max_seq_len: int,
                                     num_qo_heads: int) -> int:
    """Bytes of workspace a key-split extend of these sizes needs on the
    current device (0: the call fills the device without splitting)."""
    ps = _pool_struct(pool)
    return int(load_library().msgl_paged_extend_workspace_size(ctypes.byref(ps), int(total_extend_tokens),
                                                               int(max_seq_len), int(num_qo_heads)))


def msgl_paged_mixed(pool: torch.Tensor, layer: int, q: torch.Tensor, page_table: torch.Tensor,
                     table_idx: torch.Tensor, prefix_lens: torch.Tensor, extend_lens: torch.Tensor,
                     cu_extend_lens: torch.Tensor, max_extend_len: int, max_seq_len: int,
                     sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A batch of decode rows (one new token) and extend rows in one call:
    q (sum E, Hq, d) -> out, rows dispatched on the device by extend_lens."""
    ps = _pool_struct(pool)
    T, hq, d = q.shape
    qs = _rows(q, "q", hq, d)
    B = int(table_idx.numel())
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.bfloat16, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(B, hq, d, max_seq_len, ps.page_size, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if page_table.dim() != 2:
        raise ValueError("page_table must be 2-D (rows, entries)")
    st = load_library().msgl_paged_mixed(
        ctypes.byref(ps), layer, q.data_ptr(), qs, out.data_ptr(), _i32(page_table, "page_table"),
        int(page_table.shape[1]), _i32(table_idx, "table_idx"), _i32(prefix_lens, "prefix_lens"),
        _i32(extend_lens, "extend_lens"), _i32(cu_extend_lens, "cu_extend_lens"), B, T,
        int(max_extend_len), int(max_seq_len), hq, float(sm_scale), ws_ptr, ws_bytes, _stream(q))
    _check(st, "msgl_paged_mixed")
    return out


def msgl_debug_gather_kv(pool: torch.Tensor, layer: int, page_table: torch.Tensor, row: int,
                         length: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Tokens 0 .. length-1 of page_table row ``row``, in logical order."""
    ps = _pool_struct(pool)
    k = torch.empty((length, ps.num_kv_heads, ps.head_dim), dtype=torch.bfloat16, device=pool.device)
    v = torch.empty_like(k)
    st = load_library().msgl_debug_gather_kv(ctypes.byref(ps), layer, _i32(page_table, "page_table"),
                                             int(page_table.shape[1]), row, length, k.data_ptr(),
                                             v.data_ptr(), _stream(pool))
    _check(st, "msgl_debug_gather_kv")
    return k, v


def msgl_alloc_pages(free_pages: torch.Tensor, num_free: torch.Tensor, page_table: torch.Tensor,
                     table_idx: torch.Tensor, prefix_lens: torch.Tensor, extend_lens: torch.Tensor,
                     page_size: int, out_loc: torch.Tensor, status: torch.Tensor) -> None:
    """One scheduling step's page allocation on the device (see msgl.h):
    new pages from the tail of free_pages[:num_free] into the page_table
    rows, out_loc filled, num_free and status (both 1-element int32 device
    tensors) updated.  Nothing is read back to the host."""
    if page_table.dim() != 2:
        raise ValueError("page_table must be 2-D (rows, entries)")
    B = int(table_idx.numel())
    for name, t in (("num_free", num_free), ("status", status)):
        if t.numel() < 1:
            raise ValueError(f"{name} must hold one int32")
    st = load_library().msgl_alloc_pages(
        _i32(free_pages, "free_pages"), _i32(num_free, "num_free"), _i32(page_table, "page_table"),
        int(page_table.shape[1]), int(page_table.shape[0]), _i32(table_idx, "table_idx"),
        _i32(prefix_lens, "prefix_lens"), _i32(extend_lens, "extend_lens"), B, int(page_size),
        _i32(out_loc, "out_loc"), int(out_loc.numel()), _i32(status, "status"), _stream(page_table))
    _check(st, "msgl_alloc_pages")


def msgl_rope_cos_sin_table(max_position: int, head_dim: int, base: float = 10000.0,
                            device="cuda") -> torch.Tensor:
    """(max_position, head_dim) fp32: cos of p * base^(-2i/d) in columns
    i < d/2, the sines after them (computed by the library kernel)."""
    t = torch.empty((max_position, head_dim), dtype=torch.float32, device=device)
    st = load_library().msgl_rope_cos_sin_table(t.data_ptr(), int(max_position), int(head_dim),
                                                float(base), _stream(t))
    _check(st, "msgl_rope_cos_sin_table")
    return t


def msgl_rope_store_kv(pool: torch.Tensor, layer: int, q: Optional[torch.Tensor], k: torch.Tensor,
                       v: torch.Tensor, out_loc: torch.Tensor, positions: torch.Tensor,
                       cos_sin_table: torch.Tensor) -> None:
    """Rotate q in place and store rotated k and v at out_loc (one launch)."""
    ps = _pool_struct(pool)
    T = int(out_loc.numel())
    ks = _rows(k, "k", ps.num_kv_heads, ps.head_dim)
    vs = _rows(v, "v", ps.num_kv_heads, ps.head_dim)
    if k.shape[0] != T or v.shape[0] != T or positions.numel() != T:
        raise ValueError("k, v, out_loc and positions must have the same number of rows")
    if q is not None:
        hq = int(q.shape[1])
        qs = _rows(q, "q", hq, ps.head_dim)
        if q.shape[0] != T:
            raise ValueError("q must have one row per token")
        qp = q.data_ptr()
    else:
        hq, qs, qp = 0, 0, None
    if (cos_sin_table.dtype != torch.float32 or cos_sin_table.dim() != 2 or not cos_sin_table.is_cuda
            or cos_sin_table.shape[1] != ps.head_dim or not cos_sin_table.is_contiguous()):
        raise ValueError("cos_sin_table must be a contiguous (max_position, head_dim) fp32 CUDA tensor")
    st = load_library().msgl_rope_store_kv(
        ctypes.byref(ps), layer, qp, qs, hq, k.data_ptr(), ks, v.data_ptr(), vs,
        _i32(out_loc, "out_loc"), _i32(positions, "positions"), T, cos_sin_table.data_ptr(),
        int(cos_sin_table.shape[0]), _stream(pool))
    _check(st, "msgl_rope_store_kv")


class _StaticDecodeBuffers:
    """The static tensors a captured store_kv + decode reads and writes,
    for up to `batch` rows, with every row padding (out_loc -1, seq_lens 0,
    table_idx 0: no store, zero output, no KV read)."""

    def __init__(self, pool: torch.Tensor, batch: int, num_qo_heads: int, max_seq_len: int,
                 page_table: torch.Tensor, sm_scale: Optional[float]):
        ps = _pool_struct(pool)
        if page_table.dim() != 2:
            raise ValueError("page_table must be 2-D (rows, entries)")
        dev = pool.device
        d, hkv = ps.head_dim, ps.num_kv_heads
        self.batch, self.max_seq_len = int(batch), int(max_seq_len)
        self.pool, self.page_table = pool, page_table
        self.q = torch.zeros((batch, num_qo_heads, d), dtype=torch.bfloat16, device=dev)
        self.k = torch.zeros((batch, hkv, d), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros((batch, hkv, d), dtype=torch.bfloat16, device=dev)
        self.out = torch.zeros((batch, num_qo_heads, d), dtype=torch.bfloat16, device=dev)
        self.out_loc = torch.full((batch,), -1, dtype=torch.int32, device=dev)
        self.table_idx = torch.zeros((batch,), dtype=torch.int32, device=dev)
        self.seq_lens = torch.zeros((batch,), dtype=torch.int32, device=dev)
        need = msgl_paged_decode_workspace_size(batch, num_qo_heads, d, max_seq_len, ps.page_size)
        self.workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        self.sm_scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
        self._pool_struct = ps
        self._args = (ctypes.byref(ps), None, self.k.data_ptr(), hkv * d, self.v.data_ptr(), hkv * d,
                      self.out_loc.data_ptr(), self.q.data_ptr(), num_qo_heads * d,
                      self.out.data_ptr(), _i32(page_table, "page_table"), int(page_table.shape[1]),
                      self.table_idx.data_ptr(), self.seq_lens.data_ptr(), batch, num_qo_heads,
                      int(max_seq_len), self.sm_scale, self.workspace.data_ptr(),
                      self.workspace.numel())

    _destroy = None  # the library call that frees the handle

    def _create(self, fn: str, layer: int):
        """Capture through the library call `fn` over these buffers."""
        args = list(self._args)
        args[1] = layer
        handle = ctypes.c_void_p()
        torch.cuda.synchronize(self.pool.device)  # the static tensors are initialised
        _check(getattr(load_library(), fn)(*args, ctypes.byref(handle)), fn)
        return handle

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            torch.cuda.synchronize(self.q.device)
            getattr(load_library(), self._destroy)(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def fill(self, q, k, v, out_loc, table_idx, seq_lens, rows: int) -> int:
        """Copy a batch of b rows in and make rows b .. rows-1 padding."""
        b = int(q.shape[0])
        for name, t, shape in (("q", q, self.q.shape[1:]), ("k", k, self.k.shape[1:]),
                               ("v", v, self.v.shape[1:])):
            if t.shape[0] != b or tuple(t.shape[1:]) != tuple(shape) or t.dtype != torch.bfloat16:
                raise ValueError(f"{name} must be bf16 shaped ({b}, {tuple(shape)})")
        for name, t in (("out_loc", out_loc), ("table_idx", table_idx), ("seq_lens", seq_lens)):
            if t.numel() != b or t.dtype != torch.int32:
                raise ValueError(f"{name} must be {b} int32 values")
        self.q[:b].copy_(q)
        self.k[:b].copy_(k)
        self.v[:b].copy_(v)
        self.out_loc[:b].copy_(out_loc)
        self.table_idx[:b].copy_(table_idx)
        self.seq_lens[:b].copy_(seq_lens)
        if b < rows:
            self.out_loc[b:rows].fill_(-1)
            self.table_idx[b:rows].fill_(0)
            self.seq_lens[b:rows].fill_(0)
        return b


class DecodeGraphRunner(_StaticDecodeBuffers):
    """Decode graphs at batch sizes 1, 2, 4, ... and ``max_batch`` over one
    set of static buffers (``msgl_decode_graph_runner_*``; "Code Notes:
    mini-sglang", Engine Layer table, GraphRunner row): a batch of b rows
    replays the smallest captured size >= b, with rows b .. size-1 padded.
    ``page_table`` is referenced, not copied."""

    _destroy = "msgl_decode_graph_runner_destroy"

    def __init__(self, pool: torch.Tensor, layer: int, max_batch: int, num_qo_heads: int,
                 max_seq_len: int, page_table: torch.Tensor, sm_scale: Optional[float] = None):
        super().__init__(pool, max_batch, num_qo_heads, max_seq_len, page_table, sm_scale)
        self._handle = self._create("msgl_decode_graph_runner_create", layer)
        self.sizes = []
        s = 1
        while True:
            self.sizes.append(min(s, self.batch))
            if self.sizes[-1] == self.batch:
                break
            s *= 2

    def pick(self, b: int) -> int:
        """The captured size a batch of b rows runs at (0 outside 1..max_batch)."""
        return int(load_library().msgl_decode_graph_runner_pick(self._handle, int(b)))

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out_loc: torch.Tensor,
            table_idx: torch.Tensor, seq_lens: torch.Tensor) -> torch.Tensor:
        """Store k/v rows at out_loc and decode q through the picked graph;
        returns out[:b] (a view of the static output)."""
        b = int(q.shape[0])
        size = self.pick(b)
        if size == 0:
            raise ValueError(f"batch {b} outside 1..{self.batch}")
        self.fill(q, k, v, out_loc, table_idx, seq_lens, size)
        self.launch(b)
        return self.out[:b]

    def launch(self, b: int) -> None:
        """Replay the graph for b rows on the current stream over the static
        buffers as they stand (rows b .. pick(b)-1 must be padding)."""
        st = load_library().msgl_decode_graph_runner_launch(self._handle, int(b), _stream(self.q))
        _check(st, "msgl_decode_graph_runner_launch")


class DecodeGraph(_StaticDecodeBuffers):
    """store_kv of one new K/V row per request + paged decode, captured once
    for a fixed padded batch and replayed with a single graph launch
    (``msgl_decode_graph_*``; "Code Notes: mini-sglang", Engine Layer
    table, GraphRunner row).

    The graph reads and writes static tensors owned by this object; ``run``
    copies a real batch of ``b <= batch`` rows into them, pads the rest
    (out_loc -1, seq_lens 0, table_idx 0: no store, zero output, no KV read)
    and launches on the current stream.  ``page_table`` is referenced, not
    copied: the caller keeps it allocated and updates it in place.  One
    graph's launches share its buffers, so they are stream-ordered here.
    """

    _destroy = "msgl_decode_graph_destroy"

    def __init__(self, pool: torch.Tensor, layer: int, batch: int, num_qo_heads: int,
                 max_seq_len: int, page_table: torch.Tensor, sm_scale: Optional[float] = None):
        super().__init__(pool, batch, num_qo_heads, max_seq_len, page_table, sm_scale)
        self._handle = self._create("msgl_decode_graph_create", layer)

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out_loc: torch.Tensor,
            table_idx: torch.Tensor, seq_lens: torch.Tensor) -> torch.Tensor:
        """Store k/v rows at out_loc and decode q; returns out[:b] (a view of
        the static output, overwritten by the next run)."""
        b = int(q.shape[0])
        if b < 1 or b > self.batch:
            raise ValueError(f"batch {b} outside 1..{self.batch}")
        self.fill(q, k, v, out_loc, table_idx, seq_lens, self.batch)
        self.launch()
        return self.out[:b]

    def launch(self) -> None:
        """Replay the graph on the current stream over the static buffers as
        they stand."""
        st = load_library().msgl_decode_graph_launch(self._handle, _stream(self.q))
        _check(st, "msgl_decode_graph_launch")


# short names
store_kv = msgl_store_kv
rope_store_kv = msgl_rope_store_kv
rope_cos_sin_table = msgl_rope_cos_sin_table
alloc_pages = msgl_alloc_pages
paged_mixed = msgl_paged_mixed
paged_decode = msgl_paged_decode
paged_decode_noalloc = msgl_paged_decode_noalloc
paged_decode_workspace_size = msgl_paged_decode_workspace_size
paged_extend = msgl_paged_extend
paged_extend_workspace_size = msgl_paged_extend_workspace_size
debug_gather_kv = msgl_debug_gather_kv
