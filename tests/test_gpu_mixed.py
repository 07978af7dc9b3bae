"""Mixed batches (msgl_paged_mixed): decode rows and extend rows in one
call, dispatched on the device by extend_lens, on gfx950.

  * against the oracle over the whole batch (attention tolerance);
  * decode rows equal msgl_paged_decode on those rows bit for bit (the
    same workgroup body over the same token ranges);
  * extend rows equal msgl_paged_extend on the batch bit for bit;
  * the single launch (power-of-two page sizes) equals the decode + extend
    launches that MSGL_MIXED_SPLIT=1 selects, bit for bit, on batches
    whose decode rows are split over several ranges.
"""

import os
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits, close_report, widen
from workloads import build_case

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-mixed] {msg}", file=sys.stderr, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("hq,hkv,d,ps", [(8, 2, 128, 16), (6, 3, 64, 5), (32, 4, 128, 1),
                                         (16, 8, 64, 16), (4, 1, 128, 2)])
def test_mixed_batch_matches_oracle_and_separate_calls(hq, hkv, d, ps):
    P = [900, 0, 37, 2000, 4, 130, 600]
    E = [1, 70, 1, 1, 0, 300, 1]
    wl = build_case(500 + ps, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=P, extend_lens=E)
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    pt = torch.from_numpy(wl.page_table).cuda()
    k, v, q = ph.k.cuda(), ph.v.cuda(), ph.q.cuda()
    msgl.store_kv(pool, 0, k, v, _i32(ph.out_loc))
    ti, pl, el, cu = _i32(ph.table_idx), _i32(ph.prefix_lens), _i32(ph.extend_lens), _i32(ph.cu_extend_lens)
    max_e, max_l = int(ph.extend_lens.max()), int(ph.seq_lens.max())
    _say(f"mixed hq={hq} hkv={hkv} d={d} ps={ps}")
    out = msgl.paged_mixed(pool, 0, q, pt, ti, pl, el, cu, max_e, max_l)
    # the extend rows against the unsplit extend kernel, which the mixed
    # launch runs
    ref_ext = msgl.paged_extend(pool, 0, q, pt, ti, pl, el, cu, max_e, max_l, split=False)
    # the decode rows alone, through paged_decode with the same grid bound
    dec = [r for r in range(len(P)) if E[r] == 1]
    rows = [int(ph.cu_extend_lens[r]) for r in dec]
    out_dec = msgl.paged_decode(pool, 0, q[rows].contiguous(), pt, _i32(ph.table_idx[dec]),
                                _i32(np.array(P)[dec] + 1), max_l)
    torch.cuda.synchronize()
    assert torch.equal(out[rows].view(torch.int16), out_dec.view(torch.int16))
    ext_rows = [i for r in range(len(P)) if E[r] > 1
                for i in range(int(ph.cu_extend_lens[r]), int(ph.cu_extend_lens[r + 1]))]
    assert torch.equal(out[ext_rows].view(torch.int16), ref_ext[ext_rows].view(torch.int16))
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    ref = oracle.paged_attention(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                 ph.prefix_lens, ph.extend_lens)
    ok, max_abs, max_rel, rel_l2 = close_report(widen(bits(out), np.float64), ref, 1e-2, 1e-2)
    _say(f"max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}")
    assert ok and rel_l2 <= 5e-3


def test_all_decode_rows_through_mixed_equal_decode():
    hq, hkv, d, ps = 8, 2, 128, 16
    L = [300, 1, 2500, 64]
    wl = build_case(551, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[l - 1 for l in L], extend_lens=[1] * len(L))
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    pt = torch.from_numpy(wl.page_table).cuda()
    q = ph.q.cuda()
    msgl.store_kv(pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    out = msgl.paged_mixed(pool, 0, q, pt, _i32(ph.table_idx), _i32(ph.prefix_lens),
                           _i32(ph.extend_lens), _i32(ph.cu_extend_lens), 1, max(L))
    ref = msgl.paged_decode(pool, 0, q, pt, _i32(ph.table_idx), _i32(ph.seq_lens), max(L))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def _mixed_split(fn):
    os.environ["MSGL_MIXED_SPLIT"] = "1"
    try:
        return fn()
    finally:
        del os.environ["MSGL_MIXED_SPLIT"]


@pytest.mark.parametrize("hq,hkv,d,ps,seed", [(32, 8, 128, 16, 0), (32, 4, 128, 1, 1),
                                              (16, 2, 64, 4, 2)])
def test_single_launch_equals_split_launches(hq, hkv, d, ps, seed):
    # 40 decode rows (lengths up to 3000: several share a range, the long
    # ones are split over several), extend rows of 2 .. 600 new tokens
    # (one to three 256-row tiles a kv head), rows with no new token
    rng = np.random.default_rng(700 + seed)
    P = [int(x) for x in rng.integers(0, 3000, 40)] + [0, 1500, 77, 900, 5]
    E = [1] * 40 + [600, 257, 2, 0, 33]
    order = rng.permutation(len(P))
    P, E = [P[i] for i in order], [E[i] for i in order]
    wl = build_case(710 + seed, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=P, extend_lens=E)
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    pt = torch.from_numpy(wl.page_table).cuda()
    q = ph.q.cuda()
    msgl.store_kv(pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    args = (pool, 0, q, pt, _i32(ph.table_idx), _i32(ph.prefix_lens), _i32(ph.extend_lens),
            _i32(ph.cu_extend_lens), int(ph.extend_lens.max()), int(ph.seq_lens.max()))
    _say(f"single vs split hq={hq} hkv={hkv} d={d} ps={ps}")
    one = msgl.paged_mixed(*args)
    split = _mixed_split(lambda: msgl.paged_mixed(*args))
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), split.view(torch.int16))
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    ref = oracle.paged_attention(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                 ph.prefix_lens, ph.extend_lens)
    ok, max_abs, max_rel, rel_l2 = close_report(widen(bits(one), np.float64), ref, 1e-2, 1e-2)
    _say(f"max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}")
    assert ok and rel_l2 <= 5e-3


def test_single_launch_all_extend_rows():
    # no decode row at all: every decode workgroup of the grid exits at once
    hq, hkv, d, ps = 8, 8, 128, 16
    P, E = [0, 300, 1000], [700, 45, 256]
    wl = build_case(720, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=P, extend_lens=E)
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    pt = torch.from_numpy(wl.page_table).cuda()
    q = ph.q.cuda()
    msgl.store_kv(pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    args = (pool, 0, q, pt, _i32(ph.table_idx), _i32(ph.prefix_lens), _i32(ph.extend_lens),
            _i32(ph.cu_extend_lens), max(E), max(p + e for p, e in zip(P, E)))
    out = msgl.paged_mixed(*args)
    ref = msgl.paged_extend(*args, split=False)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
