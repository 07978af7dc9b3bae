"""Seeded synthetic inputs for the paged-KV attention path.

This module only draws inputs: page assignments, lengths, the initial pool
contents and the q/k/v rows of each step.  It contains none of the attention
arithmetic, so both the CPU oracle's tests and the HIP path's tests and bench
can take their inputs from it without sharing any of the method.

Objects follow the pages' vocabulary:
  * the KV pool is one tensor shaped (2, num_layers, num_pages, page_size,
    kv_heads, head_dim) whose leading index 0 holds K and 1 holds V
    (Code Notes: mini-sglang, "Engine Layer" table, BaseKVCachePool row);
  * each request owns one ``page_table`` row, picked by ``table_idx``
    (same page, "Scheduler Layer" table, TableManager row);
  * ``out_loc`` lists the pool slots that this step's new tokens are written
    to, as handed out by the cache manager from its free token positions
    (same table, CacheManager row).

A page_table entry is a page id; token ``p`` of a request lives in slot
``page_id * page_size + p % page_size`` of the (slots, kv_heads, head_dim)
view.  Producing ``out_loc`` from the pages given to a request is the
allocator's side of that contract, which is why it appears here.

Random numbers: metadata comes from ``numpy.random.default_rng(seed)`` in
the call order documented per builder; tensor values come from a
``torch.Generator`` seeded with the same number, drawn in the order
pool, then per phase k, v, q.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "Phase",
    "Workload",
    "build_case",
    "config_tiny",
    "config_llama3_8b_decode",
    "config_radix_shared_extend",
    "config_chunked_prefill",
    "config_qwen3_moe_decode",
    "CONFIG_BUILDERS",
]


@dataclasses.dataclass
class Phase:
    """One step of the path: store this step's rows, then attend.

    ``kind`` is "decode" (one new token per request) or "extend"
    (prefill/extend over a cached prefix).  Lengths are per request of this
    phase; ``table_idx`` picks each request's page_table row.  Token rows of
    ``q``, ``k``, ``v`` and ``out_loc`` are in request order, each request's
    new tokens contiguous (so request r owns rows cu[r]:cu[r+1]).
    """

    kind: str
    table_idx: np.ndarray  # (B,) int32
    prefix_lens: np.ndarray  # (B,) int32, tokens already in the pool
    extend_lens: np.ndarray  # (B,) int32, new tokens this step
    out_loc: np.ndarray  # (T,) int32 slots for the new tokens
    q: torch.Tensor  # (T, Hq, d) bf16
    k: torch.Tensor  # (T, Hkv, d) bf16
    v: torch.Tensor  # (T, Hkv, d) bf16

    @property
    def seq_lens(self) -> np.ndarray:
        return (self.prefix_lens + self.extend_lens).astype(np.int32)

    @property
    def cu_extend_lens(self) -> np.ndarray:
        cu = np.zeros(len(self.extend_lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.extend_lens)
        return cu

    @property
    def batch(self) -> int:
        return int(len(self.table_idx))

    @property
    def num_tokens(self) -> int:
        return int(self.extend_lens.sum())


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_layers: int
    layer: int
    num_pages: int
    page_size: int
    num_kv_heads: int
    num_qo_heads: int
    head_dim: int
    std: float
    page_table: np.ndarray  # (rows, width) int32, unused entries -1
    pool: torch.Tensor  # (2, num_layers, num_pages, page_size, Hkv, d) bf16
    phases: List[Phase]
    note: str = ""

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size


def _slots_for(pages: np.ndarray, positions: np.ndarray, page_size: int) -> np.ndarray:
    """Slots that the allocator hands out for token positions of one request."""
    return (pages[positions // page_size].astype(np.int64) * page_size
            + positions % page_size).astype(np.int32)


def _randn_bf16(gen: torch.Generator, shape, std: float, device) -> torch.Tensor:
    """N(0, std^2) values rounded to bf16, drawn in slabs to bound fp32 memory."""
    numel = int(np.prod(shape))
    out = torch.empty(numel, dtype=torch.bfloat16, device=device)
    slab = 1 << 26
    for s in range(0, numel, slab):
        e = min(numel, s + slab)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s:e] = x.to(torch.bfloat16)
    return out.view(*shape)


def _generator(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


def _fill_page_table(rows: int, pages_per_req: Sequence[np.ndarray],
                     table_idx: np.ndarray, width: Optional[int] = None) -> np.ndarray:
    w = width if width is not None else max(1, max(len(p) for p in pages_per_req))
    pt = np.full((rows, w), -1, dtype=np.int32)
    for r, pages in enumerate(pages_per_req):
        pt[table_idx[r], : len(pages)] = pages
    return pt


def _phase_tensors(gen, T, Hq, Hkv, d, std, device):
    k = _randn_bf16(gen, (T, Hkv, d), std, device)
    v = _randn_bf16(gen, (T, Hkv, d), std, device)
    q = _randn_bf16(gen, (T, Hq, d), std, device)
    return q, k, v


def build_case(seed: int, *, num_qo_heads: int, num_kv_heads: int, head_dim: int,
               page_size: int, prefix_lens: Sequence[int], extend_lens: Sequence[int],
               num_pages: Optional[int] = None, shared_prefix: bool = False,
               kind: Optional[str] = None, std: float = 1.0, device="cpu",
               spare_rows: int = 1, name: str = "case") -> Workload:
    """A single-phase workload with explicit lengths, for sweeps and edge cases.

    rng call order: (1) page permutation, (2) table_idx.
    With ``shared_prefix`` every request's row starts with the same pages for
    the common prefix (radix reuse); the prefix must then be whole pages and
    equal for all requests.
    """
    rng = np.random.default_rng(seed)
    P = np.asarray(prefix_lens, dtype=np.int32)
    E = np.asarray(extend_lens, dtype=np.int32)
    B = len(P)
    L = P + E
    ps = page_size
    npages_req = [int(math.ceil(int(l) / ps)) for l in L]
    if shared_prefix:
        assert B > 0 and np.all(P == P[0]) and P[0] % ps == 0
        n_shared = int(P[0]) // ps
        need = n_shared + sum(n - n_shared for n in npages_req)
    else:
        need = sum(npages_req)
    if num_pages is None:
        num_pages = max(need + 3, 8)
    assert need <= num_pages, "pool too small for the requested lengths"
    perm = rng.permutation(num_pages).astype(np.int32)[:need]
    pages_per_req = []
    if shared_prefix:
        shared = perm[:n_shared]
        cur = n_shared
        for n in npages_req:
            own = perm[cur: cur + n - n_shared]
            cur += n - n_shared
            pages_per_req.append(np.concatenate([shared, own]))
    else:
        cur = 0
        for n in npages_req:
            pages_per_req.append(perm[cur: cur + n])
            cur += n
    rows = B + spare_rows
    table_idx = rng.choice(rows, B, replace=False).astype(np.int32)
    page_table = _fill_page_table(rows, pages_per_req, table_idx,
                                  width=max(1, max(npages_req) if B else 1))
    out_loc = (np.concatenate([_slots_for(pages_per_req[r], np.arange(P[r], L[r]), ps)
                               for r in range(B)]) if B else np.zeros(0, np.int32))
    gen = _generator(seed, device)
    pool = _randn_bf16(gen, (2, 1, num_pages, ps, num_kv_heads, head_dim), std, device)
    T = int(E.sum())
    q, k, v = _phase_tensors(gen, T, num_qo_heads, num_kv_heads, head_dim, std, device)
    if kind is None:
        kind = "decode" if (B > 0 and np.all(E == 1)) else "extend"
    ph = Phase(kind, table_idx, P, E, out_loc.astype(np.int32), q, k, v)
    return Workload(name, seed, 1, 0, num_pages, ps, num_kv_heads, num_qo_heads,
                    head_dim, std, page_table, pool, [ph])


def config_tiny(device="cpu", seed: int = 1) -> Workload:
    """Tiny paged attention: 1 layer, 4 q heads / 1 kv head, head_dim 64,
    page_size 16, pool of 64 pages, N(0,1).  Requests have total lengths
    17, 100 and 256 (the decode token included), on pages taken in request
    order from a permutation of the pool.  Phase 0 stores the 3 decode rows
    and decodes; phase 1 extends request 1 by 16 tokens on its 100-token
    prefix (the prefix is not page aligned).

    rng call order: (1) page permutation, (2) table_idx.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, ps, NP = 4, 1, 64, 16, 64
    final_lens = [17, 116, 256]  # request 1 ends at 100 + 16 after the extend
    npages = [int(math.ceil(l / ps)) for l in final_lens]
    perm = rng.permutation(NP).astype(np.int32)
    pages, cur = [], 0
    for n in npages:
        pages.append(perm[cur: cur + n])
        cur += n
    B = 3
    table_idx = rng.choice(2 * B, B, replace=False).astype(np.int32)
    page_table = _fill_page_table(2 * B, pages, table_idx)
    gen = _generator(seed, device)
    pool = _randn_bf16(gen, (2, 1, NP, ps, Hkv, d), 1.0, device)
    # phase 0: decode with L = 17, 100, 256
    L0 = np.array([17, 100, 256], dtype=np.int32)
    P0, E0 = L0 - 1, np.ones(B, dtype=np.int32)
    loc0 = np.concatenate([_slots_for(pages[r], np.array([L0[r] - 1]), ps) for r in range(B)])
    q0, k0, v0 = _phase_tensors(gen, B, Hq, Hkv, d, 1.0, device)
    ph0 = Phase("decode", table_idx.copy(), P0, E0, loc0.astype(np.int32), q0, k0, v0)
    # phase 1: request 1 extends by 16 on its 100-token prefix
    P1, E1 = np.array([100], np.int32), np.array([16], np.int32)
    loc1 = _slots_for(pages[1], np.arange(100, 116), ps)
    q1, k1, v1 = _phase_tensors(gen, 16, Hq, Hkv, d, 1.0, device)
    ph1 = Phase("extend", table_idx[1:2].copy(), P1, E1, loc1.astype(np.int32), q1, k1, v1)
    return Workload("tiny", seed, 1, 0, NP, ps, Hkv, Hq, d, 1.0, page_table, pool,
                    [ph0, ph1], note="4q/1kv d64 ps16 pool64 L={17,100,256} + extend 16 on 100")


def config_llama3_8b_decode(device="cpu", seed: int = 2, batch: int = 64, num_qo_heads: int = 32,
                            num_kv_heads: int = 8) -> Workload:
    """Llama-3-8B attention geometry decode: 32 q / 8 kv heads, head_dim 128,
    page_size 16, 64 requests with total lengths uniform in [512, 4096],
    pages scattered in a pool of 32768 pages, N(0,1); store_kv of the 64 new
    rows, then decode.  Other head counts (4 q / 1 kv: one GPU's share under
    8-way tensor parallelism) keep the same lengths and pages.

    rng call order: (1) lengths, (2) page permutation, (3) table_idx.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, ps, NP = num_qo_heads, num_kv_heads, 128, 16, 32768
    B = batch
    L = rng.integers(512, 4096, B, endpoint=True).astype(np.int32)
    return _decode_from_lengths("llama3_8b_decode", seed, rng, L, Hq, Hkv, d, ps, NP, 1.0, device,
                                note=f"{Hq}q/{Hkv}kv d128 ps16 B{B} L~U[512,4096] pool 32768 pages")


def config_qwen3_moe_decode(device="cpu", seed: int = 5, batch: int = 256) -> Workload:
    """Qwen3-30B-A3B attention geometry decode: 32 q / 4 kv heads, head_dim
    128, page_size 1 (token-granular slots), 256 requests with lognormal
    lengths (median 2048, sigma 1 on the natural-log scale, rounded, clipped
    to [16, 32768]), slots scattered in a pool of 2^21, N(0,1).

    rng call order: (1) lengths, (2) slot permutation, (3) table_idx.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, ps, NP = 32, 4, 128, 1, 1 << 21
    B = batch
    L = rng.lognormal(math.log(2048.0), 1.0, B)
    L = np.clip(np.rint(L), 16, 32768).astype(np.int32)
    return _decode_from_lengths("qwen3_moe_decode", seed, rng, L, Hq, Hkv, d, ps, NP, 1.0, device,
                                note="32q/4kv d128 ps1 B256 L~lognormal(med 2048) pool 2^21 slots")


def _decode_from_lengths(name, seed, rng, L, Hq, Hkv, d, ps, NP, std, device, note):
    B = len(L)
    npages = -(-L // ps)
    perm = rng.permutation(NP).astype(np.int32)[: int(npages.sum())]
    pages, cur = [], 0
    for n in npages:
        pages.append(perm[cur: cur + int(n)])
        cur += int(n)
    table_idx = rng.choice(2 * B, B, replace=False).astype(np.int32)
    page_table = _fill_page_table(2 * B, pages, table_idx)
    gen = _generator(seed, device)
    pool = _randn_bf16(gen, (2, 1, NP, ps, Hkv, d), std, device)
    P, E = (L - 1).astype(np.int32), np.ones(B, dtype=np.int32)
    loc = np.concatenate([_slots_for(pages[r], np.array([L[r] - 1]), ps) for r in range(B)])
    q, k, v = _phase_tensors(gen, B, Hq, Hkv, d, std, device)
    ph = Phase("decode", table_idx, P, E, loc.astype(np.int32), q, k, v)
    return Workload(name, seed, 1, 0, NP, ps, Hkv, Hq, d, std, page_table, pool, [ph], note=note)


def config_radix_shared_extend(device="cpu", seed: int = 3, batch: int = 16,
                               prefix: int = 2048, extend: int = 512, num_qo_heads: int = 32,
                               num_kv_heads: int = 8) -> Workload:
    """Radix-shared prefix extend: 32 q / 8 kv heads, head_dim 128,
    page_size 16, pool of 32768 pages; 16 requests whose rows all start with
    the same 128 pages holding a 2048-token prefix, each extending 512 new
    tokens on private pages with a causal mask over prefix + extend; N(0,1).

    Other head counts keep the same pages and lengths.

    rng call order: (1) page permutation, (2) table_idx.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, ps, NP = num_qo_heads, num_kv_heads, 128, 16, 32768
    B = batch
    n_shared, n_own = prefix // ps, extend // ps
    perm = rng.permutation(NP).astype(np.int32)[: n_shared + B * n_own]
    shared = perm[:n_shared]
    pages = [np.concatenate([shared, perm[n_shared + r * n_own: n_shared + (r + 1) * n_own]])
             for r in range(B)]
    table_idx = rng.choice(2 * B, B, replace=False).astype(np.int32)
    page_table = _fill_page_table(2 * B, pages, table_idx)
    gen = _generator(seed, device)
    pool = _randn_bf16(gen, (2, 1, NP, ps, Hkv, d), 1.0, device)
    P = np.full(B, prefix, np.int32)
    E = np.full(B, extend, np.int32)
    loc = np.concatenate([_slots_for(pages[r], np.arange(prefix, prefix + extend), ps)
                          for r in range(B)])
    q, k, v = _phase_tensors(gen, B * extend, Hq, Hkv, d, 1.0, device)
    ph = Phase("extend", table_idx, P, E, loc.astype(np.int32), q, k, v)
    return Workload("radix_shared_extend", seed, 1, 0, NP, ps, Hkv, Hq, d, 1.0, page_table,
                    pool, [ph], note=f"{Hq}q/{Hkv}kv d128 ps16 B{B} shared prefix {prefix} + extend {extend}")


def config_chunked_prefill(device="cpu", seed: int = 4, total: int = 32768,
                           chunk: int = 4096, num_qo_heads: int = 32, num_kv_heads: int = 8) -> Workload:
    """Chunked prefill of one 32768-token request as 8 extend chunks of 4096
    over the growing prefix: 32 q / 8 kv heads, head_dim 128, page_size 16,
    pool of 32768 pages, values N(0, 0.5^2) (standard deviation 0.5).

    Other head counts keep the same pages and lengths.

    rng call order: (1) page permutation, (2) table_idx.
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, ps, NP, std = num_qo_heads, num_kv_heads, 128, 16, 32768, 0.5
    pages = rng.permutation(NP).astype(np.int32)[: total // ps]
    table_idx = rng.choice(2, 1, replace=False).astype(np.int32)
    page_table = _fill_page_table(2, [pages], table_idx)
    gen = _generator(seed, device)
    pool = _randn_bf16(gen, (2, 1, NP, ps, Hkv, d), std, device)
    phases = []
    for c in range(total // chunk):
        P = np.array([c * chunk], np.int32)
        E = np.array([chunk], np.int32)
        loc = _slots_for(pages, np.arange(c * chunk, (c + 1) * chunk), ps)
        q, k, v = _phase_tensors(gen, chunk, Hq, Hkv, d, std, device)
        phases.append(Phase("extend", table_idx.copy(), P, E, loc.astype(np.int32), q, k, v))
    return Workload("chunked_prefill", seed, 1, 0, NP, ps, Hkv, Hq, d, std, page_table, pool,
                    phases, note=f"{Hq}q/{Hkv}kv d128 ps16 1x{total} as {total // chunk} chunks of {chunk}, std 0.5")


CONFIG_BUILDERS = {
    "tiny": config_tiny,
    "llama3_8b_decode": config_llama3_8b_decode,
    "radix_shared_extend": config_radix_shared_extend,
    "chunked_prefill": config_chunked_prefill,
    "qwen3_moe_decode": config_qwen3_moe_decode,
}
