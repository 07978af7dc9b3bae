"""The calls at the edges of what they accept, on gfx950, against the oracle.

  * decode of a request at the longest length the decode call takes
    (1,048,511 tokens), beside a short one: every output element;
  * decode of a batch above one launch's 2048 requests (three launches),
    with padding rows on both sides of each launch boundary;
  * a mixed batch above 2048 requests (the separate-launch form);
  * extend of one 32768-token chunk with no prefix (512 row tiles per kv
    head), on sampled rows and the whole last tile;
  * extend of 3000 requests of a few new tokens each (a grid of 3000
    request columns);
  * store_kv, decode and extend on the last pages of the largest pool the
    attention calls take (one K or V sub-tensor just under 2^32 bytes), so
    that the 32-bit byte offsets of the page reads reach their top.

Tolerances are those of the parity tests: per element
|gpu - oracle| <= 1e-2 + 1e-2 |oracle|, relative L2 <= 5e-3.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits, close_report, widen
from workloads import build_case

pytestmark = pytest.mark.gpu

ATOL = RTOL = 1e-2
REL_L2 = 5e-3


def _say(msg):
    print(f"[gpu-limits] {msg}", file=sys.stderr, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _check(got_bf16, ref, rows=None, what=""):
    got = widen(bits(got_bf16), np.float64)
    ref = np.asarray(ref, np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ok, max_abs, max_rel, rel_l2 = close_report(got, ref, ATOL, RTOL)
    _say(f"{what}: max_abs={max_abs:.3e} max_rel={max_rel:.3e} rel_l2={rel_l2:.3e}")
    assert ok, f"{what}: max_abs={max_abs} max_rel={max_rel}"
    assert rel_l2 <= REL_L2, f"{what}: rel_l2={rel_l2}"


def _stored(wl, ph):
    """The case on the GPU after its store_kv, and the oracle's pool."""
    pool = wl.pool.cuda()
    msgl.store_kv(pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    return pool, torch.from_numpy(wl.page_table).cuda(), pool_bits


def test_decode_longest_sequence():
    longest = 1_048_511  # the decode call's bound on max_seq_len
    L = [longest, 3]
    wl = build_case(41, num_qo_heads=8, num_kv_heads=1, head_dim=128, page_size=16,
                    prefix_lens=[l - 1 for l in L], extend_lens=[1, 1])
    ph = wl.phases[0]
    _say(f"decode of {L} tokens, 8 q / 1 kv heads, d 128, ps 16")
    pool, pt, pool_bits = _stored(wl, ph)
    out = msgl.paged_decode(pool, 0, ph.q.cuda(), pt, _i32(ph.table_idx), _i32(ph.seq_lens), longest)
    torch.cuda.synchronize()
    ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx, ph.seq_lens,
                              dtype=np.float64, blocked=True)
    _check(out, ref, what="longest decode")
    with pytest.raises(msgl.MsglError):  # one token more is refused on the host
        msgl.paged_decode(pool, 0, ph.q.cuda(), pt, _i32(ph.table_idx), _i32(ph.seq_lens), longest + 1)


def test_decode_batch_over_three_launches():
    B = 4100  # launches of 2048, 2048 and 4 requests
    rng = np.random.default_rng(42)
    L = rng.integers(1, 100, B)
    wl = build_case(42, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=list(L - 1), extend_lens=[1] * B)
    ph = wl.phases[0]
    seq = ph.seq_lens.astype(np.int32).copy()
    pad = [0, 2046, 2047, 2048, 2049, 4095, 4096, 4099]  # padding rows around the launch edges
    seq[pad] = 0
    _say(f"decode of {B} requests, padding rows {pad}")
    pool, pt, pool_bits = _stored(wl, ph)
    out = msgl.paged_decode(pool, 0, ph.q.cuda(), pt, _i32(ph.table_idx), _i32(seq), int(seq.max()))
    torch.cuda.synchronize()
    ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx, seq, blocked=True)
    assert np.all(bits(out)[pad] == 0), "padding rows must be zeros"
    _check(out, ref, what=f"decode B={B}")


def test_mixed_batch_over_one_launch():
    rng = np.random.default_rng(43)
    B = 2100  # above 2048 requests: the decode and extend launches of the batch
    P = [int(x) for x in rng.integers(0, 300, B)]
    E = [1] * B
    for r, e in zip([5, 700, 2047, 2048, 2099], [2, 300, 65, 1000, 7]):
        E[r] = e
    E[9] = 0  # a row with no new token
    wl = build_case(43, num_qo_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                    prefix_lens=P, extend_lens=E)
    ph = wl.phases[0]
    _say(f"mixed batch of {B} requests")
    pool, pt, pool_bits = _stored(wl, ph)
    out = msgl.paged_mixed(pool, 0, ph.q.cuda(), pt, _i32(ph.table_idx), _i32(ph.prefix_lens),
                           _i32(ph.extend_lens), _i32(ph.cu_extend_lens), int(ph.extend_lens.max()),
                           int(ph.seq_lens.max()))
    torch.cuda.synchronize()
    ref = oracle.paged_attention_blocked(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                         ph.prefix_lens, ph.extend_lens)
    _check(out, ref, what=f"mixed B={B}")


def test_extend_one_long_chunk():
    E = 32768
    wl = build_case(44, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=[0], extend_lens=[E], std=0.5)
    ph = wl.phases[0]
    _say(f"extend of one {E}-token chunk, no prefix")
    pool, pt, pool_bits = _stored(wl, ph)
    out = msgl.paged_extend(pool, 0, ph.q.cuda(), pt, _i32(ph.table_idx), _i32(ph.prefix_lens),
                            _i32(ph.extend_lens), _i32(ph.cu_extend_lens), E, E)
    torch.cuda.synchronize()
    # every 257th row (all residues of a 256-row tile), the first rows and
    # the whole last row tile (64 tokens of 4 q heads each)
    rows = np.unique(np.concatenate([np.arange(0, E, 257), np.arange(0, 40), np.arange(E - 64, E)]))
    ref = oracle.paged_attention_blocked(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                         ph.prefix_lens, ph.extend_lens, only_tokens=rows)
    _check(out, ref, rows=rows, what=f"extend E={E} ({len(rows)} rows)")


def test_extend_many_requests():
    B = 3000
    rng = np.random.default_rng(45)
    P = [int(x) for x in rng.integers(0, 400, B)]
    E = [int(x) for x in rng.integers(1, 4, B)]
    wl = build_case(45, num_qo_heads=16, num_kv_heads=4, head_dim=64, page_size=16,
                    prefix_lens=P, extend_lens=E)
    ph = wl.phases[0]
    _say(f"extend of {B} requests, {ph.num_tokens} new tokens")
    pool, pt, pool_bits = _stored(wl, ph)
    out = msgl.paged_extend(pool, 0, ph.q.cuda(), pt, _i32(ph.table_idx), _i32(ph.prefix_lens),
                            _i32(ph.extend_lens), _i32(ph.cu_extend_lens), int(ph.extend_lens.max()),
                            int(ph.seq_lens.max()))
    torch.cuda.synchronize()
    ref = oracle.paged_attention_blocked(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                         ph.prefix_lens, ph.extend_lens)
    _check(out, ref, what=f"extend B={B}")


def _randn_bits(gen, shape):
    return bits(torch.randn(shape, generator=gen).to(torch.bfloat16))


def test_last_pages_of_the_largest_pool():
    hq, hkv, d, ps = 32, 8, 128, 16
    row_bytes = hkv * d * 2
    num_pages = ((1 << 32) - 1) // (ps * row_bytes)  # 131071: K (or V) just under 2^32 bytes
    dec_lens = [3000, 1, 777, 4096]
    ext = [(2000, 300), (0, 129)]  # (prefix, new tokens)
    lens = dec_lens + [p + e for p, e in ext]
    npg = [-(-l // ps) for l in lens]
    used = sum(npg)
    rng = np.random.default_rng(46)
    gen = torch.Generator().manual_seed(46)
    # the requests' pages are the last `used` pages of the pool, shuffled;
    # the oracle sees the same pages renumbered 0 .. used-1
    page_ids = rng.permutation(np.arange(num_pages - used, num_pages)).astype(np.int32)
    rows = len(lens)
    width = max(npg)
    pt_real = np.zeros((rows, width), np.int32)
    pt_comp = np.zeros((rows, width), np.int32)
    cur = 0
    for r, n in enumerate(npg):
        pt_real[r, :n] = page_ids[cur:cur + n]
        pt_comp[r, :n] = np.arange(cur, cur + n)
        cur += n

    def slots(table, r, positions):
        positions = np.asarray(positions, np.int64)
        return (table[r, positions // ps].astype(np.int64) * ps + positions % ps).astype(np.int32)

    _say(f"pool of {num_pages} pages ({num_pages * ps * row_bytes} bytes per K or V), "
         f"requests on its last {used} pages")
    pool = torch.zeros((2, 1, num_pages, ps, hkv, d), dtype=torch.bfloat16, device="cuda")
    init = _randn_bits(gen, (2, 1, used, ps, hkv, d))
    pool[:, :, torch.from_numpy(page_ids.astype(np.int64)).cuda()] = (
        torch.from_numpy(init.view(np.int16)).view(torch.bfloat16).cuda())
    comp = init.copy()
    pt = _i32(pt_real)

    # decode phase: the new token of each decode request, then attention
    B = len(dec_lens)
    loc_real = np.concatenate([slots(pt_real, r, [dec_lens[r] - 1]) for r in range(B)])
    loc_comp = np.concatenate([slots(pt_comp, r, [dec_lens[r] - 1]) for r in range(B)])
    kd, vd, qd = (_randn_bits(gen, (B, hkv, d)), _randn_bits(gen, (B, hkv, d)),
                  _randn_bits(gen, (B, hq, d)))
    tb = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    msgl.store_kv(pool, 0, tb(kd), tb(vd), _i32(loc_real))
    comp = oracle.store_kv(comp, 0, kd, vd, loc_comp)
    ti = np.arange(B, dtype=np.int32)
    sl = np.asarray(dec_lens, np.int32)
    out = msgl.paged_decode(pool, 0, tb(qd), pt, _i32(ti), _i32(sl), int(sl.max()))
    torch.cuda.synchronize()
    ref = oracle.paged_decode(comp, 0, qd, pt_comp, ti, sl, blocked=True)
    _check(out, ref, what="decode on the last pages")

    # extend phase
    P = np.array([p for p, _ in ext], np.int32)
    E = np.array([e for _, e in ext], np.int32)
    eti = np.arange(B, B + len(ext), dtype=np.int32)
    loc_real = np.concatenate([slots(pt_real, r, np.arange(p, p + e)) for r, (p, e) in zip(eti, ext)])
    loc_comp = np.concatenate([slots(pt_comp, r, np.arange(p, p + e)) for r, (p, e) in zip(eti, ext)])
    T = int(E.sum())
    ke, ve, qe = (_randn_bits(gen, (T, hkv, d)), _randn_bits(gen, (T, hkv, d)),
                  _randn_bits(gen, (T, hq, d)))
    msgl.store_kv(pool, 0, tb(ke), tb(ve), _i32(loc_real))
    comp = oracle.store_kv(comp, 0, ke, ve, loc_comp)
    cu = np.concatenate([[0], np.cumsum(E)]).astype(np.int32)
    out = msgl.paged_extend(pool, 0, tb(qe), pt, _i32(eti), _i32(P), _i32(E), _i32(cu), int(E.max()),
                            int((P + E).max()))
    torch.cuda.synchronize()
    ref = oracle.paged_attention_blocked(comp, 0, qe, pt_comp, eti, P, E)
    _check(out, ref, what="extend on the last pages")

    # the pages hold exactly what the oracle's store_kv wrote, bit for bit
    got = bits(pool[:, :, torch.from_numpy(page_ids.astype(np.int64)).cuda()])
    assert np.array_equal(got, comp), "store_kv on the last pages differs from the oracle"
    del pool
    torch.cuda.empty_cache()
