"""CPU oracle for attention over the paged KV cache -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import or run this module.  The product path never does;
it shares no code, header, table or helper with the HIP library, and neither
side imports the other.

Everything here is plain NumPy, written to be checked against the pages by
eye: a gather through the page table followed by one softmax per query row in
logical key order.  Floating point is fp32 by default (the precision the
oracle is specified in); every function also runs in fp64 for the pins.

Definitions followed:
  * Pool layout and ``store_kv``: "Code Notes: mini-sglang", section
    "Engine Layer: how to compute", table row BaseKVCachePool -- the pool is
    one tensor shaped (2, num_layers, num_pages, page_size, heads, head_dim)
    and store_kv writes rows by ``out_loc`` indices.
  * ``page_table`` / ``table_idx``: same page, section "Scheduler Layer: what
    to compute", table row TableManager -- one page_table row per request's
    KV mapping, the row picked by table_idx; row CacheManager -- the
    allocator hands out free token positions (slots).
  * Prefill over a cached prefix (radix reuse, chunked prefill): same page,
    PrefillManager row, and "Introduction" (Mini-SGLang docs), "Key
    Features": Radix Cache and Chunked Prefill.
  * The attention itself: out = softmax(Q K^T * sm_scale) V with sm_scale =
    1/sqrt(head_dim), each new query attending to every key at or before its
    own absolute position.

Readings taken where the pages are silent:
  * a page_table entry is a page id; token p of a request lives in slot
    page_table[row, p // page_size] * page_size + p % page_size of the
    (slots, kv_heads, head_dim) view of one (K or V, layer);
  * ``out_loc`` holds such flat slots; index 0 of the leading pool axis is K;
  * query head h reads kv head h // (q_heads / kv_heads);
  * causal alignment is bottom-right: new token i of a request with prefix
    P sits at absolute position P + i and sees keys 0 .. P + i;
  * padding conventions: out_loc < 0 skips a row, seq_len 0 yields zeros.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_float",
    "float_to_bf16_bits",
    "store_kv",
    "token_slots",
    "gather_kv",
    "paged_attention",
    "paged_attention_blocked",
    "paged_decode",
]


def bf16_bits_to_float(bits: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Widen bf16 bit patterns (uint16/int16) to float, exactly.

    A bf16 value is the upper 16 bits of an IEEE binary32, so placing the
    pattern in the upper half of a 32-bit word gives the same number.
    """
    b = np.asarray(bits)
    if b.dtype == np.int16:
        b = b.view(np.uint16)
    assert b.dtype == np.uint16, "expected bf16 bit patterns"
    f = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f.astype(dtype, copy=False)


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (round to nearest, ties to even).

    Used only to state what a bf16 output should be; NaN stays NaN.
    """
    x32 = np.atleast_1d(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    r[np.isnan(x32)] = np.uint16(0x7FC0)
    return r.reshape(np.shape(x))


def _as_bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.int16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, "expected bf16 bit patterns"
    return a


def store_kv(pool: np.ndarray, layer: int, k: np.ndarray, v: np.ndarray,
             out_loc: np.ndarray) -> np.ndarray:
    """Return a copy of ``pool`` with row t of k / v written to slot out_loc[t].

    Follows the BaseKVCachePool row of "Code Notes: mini-sglang" (Engine
    Layer table): the K half (leading index 0) and the V half (index 1) of
    layer ``layer`` are viewed as (slots, kv_heads, head_dim) and indexed by
    out_loc.  It is a copy of bit patterns; no value is converted.
    Negative out_loc entries are padding and write nothing.  Slots must be
    distinct and inside the pool, since a repeated slot has no single
    result.
    """
    pool = _as_bits(pool)
    k = _as_bits(k)
    v = _as_bits(v)
    two, nl, npg, ps, hkv, d = pool.shape
    assert two == 2 and 0 <= layer < nl
    S = npg * ps
    loc = np.asarray(out_loc, dtype=np.int64)
    assert k.shape == (len(loc), hkv, d) and v.shape == k.shape
    keep = loc >= 0
    live = loc[keep]
    assert np.all(live < S), "out_loc outside the pool"
    assert len(np.unique(live)) == len(live), "out_loc repeats a slot"
    out = pool.copy()
    kview = out[0, layer].reshape(S, hkv, d)
    vview = out[1, layer].reshape(S, hkv, d)
    kview[live] = k[keep]
    vview[live] = v[keep]
    return out


def token_slots(page_table_row: np.ndarray, length: int, page_size: int) -> np.ndarray:
    """Slots of tokens 0 .. length-1 of one request.

    One page_table row maps a request's logical pages to pool pages
    ("Code Notes: mini-sglang", Scheduler Layer table, TableManager row);
    token p is at offset p % page_size of page row[p // page_size].
    """
    p = np.arange(length, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[p // page_size]
    assert np.all(pages >= 0), "page_table row shorter than the sequence"
    return pages * page_size + p % page_size


def gather_kv(pool: np.ndarray, layer: int, page_table: np.ndarray, row: int,
              length: int) -> Tuple[np.ndarray, np.ndarray]:
    """K and V bit patterns of one request's first ``length`` tokens, in
    logical order, read through its page_table row."""
    pool = _as_bits(pool)
    two, nl, npg, ps, hkv, d = pool.shape
    S = npg * ps
    slots = token_slots(page_table[row], length, ps)
    assert np.all(slots < S)
    k = pool[0, layer].reshape(S, hkv, d)[slots]
    v = pool[1, layer].reshape(S, hkv, d)[slots]
    return k, v


def paged_attention(pool: np.ndarray, layer: int, q: np.ndarray, page_table: np.ndarray,
                    table_idx: np.ndarray, prefix_lens: np.ndarray, extend_lens: np.ndarray,
                    sm_scale: Optional[float] = None, dtype=np.float32,
                    only_tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """Causal GQA attention of each request's new tokens over its paged KV.

    Request r has prefix_lens[r] tokens already in the pool and
    extend_lens[r] new tokens (already stored), whose queries are rows
    cu[r] .. cu[r+1]-1 of ``q`` (shape (sum E, q_heads, head_dim), bf16
    bits).  New token i sits at absolute position a = P + i and attends to
    keys 0 .. a.  For each such query row and q head h (kv head h // G):

        s_j = sm_scale * q . K_j      for j = 0 .. a
        m   = max_j s_j
        w_j = exp(s_j - m)
        out = sum_j w_j V_j / sum_j w_j

    Returns float ``dtype`` values of shape (sum E, q_heads, head_dim).
    With ``only_tokens`` only those query rows are computed; the others are
    NaN.  A request with no keys (prefix 0, extend 0) has no rows.
    """
    pool = _as_bits(pool)
    qb = _as_bits(q)
    two, nl, npg, ps, hkv, d = pool.shape
    T, hq, dq = qb.shape
    assert dq == d and hq % hkv == 0
    G = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    P = np.asarray(prefix_lens, dtype=np.int64)
    E = np.asarray(extend_lens, dtype=np.int64)
    assert len(P) == len(E) == len(table_idx)
    cu = np.concatenate([[0], np.cumsum(E)])
    assert cu[-1] == T
    wanted = None if only_tokens is None else set(int(t) for t in only_tokens)
    out = np.full((T, hq, d), np.nan, dtype=dtype)
    scale = dtype(sm_scale)
    for r in range(len(P)):
        L = int(P[r] + E[r])
        if E[r] == 0:
            continue
        rows = [t for t in range(int(cu[r]), int(cu[r + 1])) if wanted is None or t in wanted]
        if not rows:
            continue
        kb, vb = gather_kv(pool, layer, page_table, int(table_idx[r]), L)
        K = bf16_bits_to_float(kb, dtype)  # (L, hkv, d)
        V = bf16_bits_to_float(vb, dtype)
        for t in rows:
            a = int(P[r]) + (t - int(cu[r]))  # absolute position of this query
            Qt = bf16_bits_to_float(qb[t], dtype)  # (hq, d)
            for g in range(hkv):
                Qg = Qt[g * G:(g + 1) * G]  # the q heads that read kv head g
                Kg = K[: a + 1, g, :]
                Vg = V[: a + 1, g, :]
                s = (Qg @ Kg.T) * scale  # (G, a+1)
                m = s.max(axis=1, keepdims=True)
                w = np.exp(s - m)
                out[t, g * G:(g + 1) * G] = (w @ Vg) / w.sum(axis=1, keepdims=True)
    return out


def paged_attention_blocked(pool: np.ndarray, layer: int, q: np.ndarray, page_table: np.ndarray,
                            table_idx: np.ndarray, prefix_lens: np.ndarray,
                            extend_lens: np.ndarray, sm_scale: Optional[float] = None,
                            dtype=np.float32, only_tokens: Optional[Iterable[int]] = None,
                            block: int = 256) -> np.ndarray:
    """The same causal GQA attention as ``paged_attention``, evaluated for a
    block of up to ``block`` query tokens of one request and one kv head at
    a time, in matrix form:

        S = sm_scale * Q K^T          (rows: the block's (token, q head) pairs)
        S[row, j] = -inf  for every key j after the row's position a
        W = exp(S - rowmax(S));  out = (W V) / rowsum(W)

    Masked keys get weight exp(-inf) = 0 exactly, so each row is the
    per-row definition above; only the summation order inside the matrix
    products differs.  This is the form that finishes in seconds at the
    full workload sizes (tens of thousands of keys per row).  Arguments and
    result are those of ``paged_attention``.
    """
    pool = _as_bits(pool)
    qb = _as_bits(q)
    two, nl, npg, ps, hkv, d = pool.shape
    T, hq, dq = qb.shape
    assert dq == d and hq % hkv == 0 and block >= 1
    G = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    P = np.asarray(prefix_lens, dtype=np.int64)
    E = np.asarray(extend_lens, dtype=np.int64)
    assert len(P) == len(E) == len(table_idx)
    cu = np.concatenate([[0], np.cumsum(E)])
    assert cu[-1] == T
    wanted = None if only_tokens is None else np.unique(np.asarray(list(only_tokens), np.int64))
    out = np.full((T, hq, d), np.nan, dtype=dtype)
    scale = dtype(sm_scale)
    for r in range(len(P)):
        if E[r] == 0:
            continue
        rows = np.arange(cu[r], cu[r + 1], dtype=np.int64)
        if wanted is not None:
            rows = rows[np.isin(rows, wanted)]
        if len(rows) == 0:
            continue
        L = int(P[r] + E[r])
        kb, vb = gather_kv(pool, layer, page_table, int(table_idx[r]), L)
        for g in range(hkv):
            Kg = np.ascontiguousarray(bf16_bits_to_float(kb[:, g, :], dtype))  # (L, d)
            Vg = np.ascontiguousarray(bf16_bits_to_float(vb[:, g, :], dtype))
            for b0 in range(0, len(rows), block):
                blk = rows[b0:b0 + block]
                a = P[r] + (blk - cu[r])  # absolute positions of the block's tokens
                n = int(a.max()) + 1
                Q = bf16_bits_to_float(qb[blk, g * G:(g + 1) * G, :], dtype).reshape(-1, d)
                S = (Q @ Kg[:n].T) * scale  # (len(blk)*G, n)
                pos = np.repeat(a, G)
                S[np.arange(n)[None, :] > pos[:, None]] = -np.inf
                S -= S.max(axis=1, keepdims=True)
                np.exp(S, out=S)
                o = (S @ Vg[:n]) / S.sum(axis=1, keepdims=True)
                out[blk, g * G:(g + 1) * G] = o.reshape(len(blk), G, d)
    return out


def paged_decode(pool: np.ndarray, layer: int, q: np.ndarray, page_table: np.ndarray,
                 table_idx: np.ndarray, seq_lens: np.ndarray, sm_scale: Optional[float] = None,
                 dtype=np.float32, only_tokens: Optional[Iterable[int]] = None,
                 blocked: bool = False) -> np.ndarray:
    """Decode: one new token per request whose row is already stored, so
    seq_len counts it; the query attends to all seq_len keys.  A request
    with seq_len 0 (a padding row) returns zeros.  ``blocked`` evaluates it
    with ``paged_attention_blocked`` (same definition, matrix form)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    qb = _as_bits(q)
    B = len(L)
    assert qb.shape[0] == B
    live = L > 0
    out = np.zeros(qb.shape, dtype=dtype)
    if np.any(live):
        idx = np.nonzero(live)[0]
        sub_only = None
        if only_tokens is not None:
            keep = set(int(t) for t in only_tokens)
            sub_only = [j for j, r in enumerate(idx) if int(r) in keep]
        attend = paged_attention_blocked if blocked else paged_attention
        sub = attend(pool, layer, qb[idx], page_table, np.asarray(table_idx)[idx],
                     L[idx] - 1, np.ones(len(idx), np.int64), sm_scale, dtype,
                     only_tokens=sub_only)
        out[idx] = sub
        if only_tokens is not None:
            keep = set(int(t) for t in only_tokens)
            for r in idx:
                if int(r) not in keep:
                    out[r] = np.nan
    return out
