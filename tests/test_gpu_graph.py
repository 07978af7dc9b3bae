"""Decode graphs (msgl_decode_graph_*, msgl_decode_graph_runner_*):
store_kv + decode captured once per padded batch size and replayed, on
gfx950.

Every replay is checked three ways on the same inputs:
  * against the same two calls made eagerly on a copy of the pool:
    bit-identical output and pool (the graph runs the same kernels);
  * against the oracle, to the attention tolerance of the parity tests;
  * padding rows (out_loc -1, seq_lens 0) give zeros and store nothing.
Replays alternate with eager work on the same stream, and the real batch
size and the sequence lengths change from one replay to the next.
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
    print(f"[gpu-graph] {msg}", file=sys.stderr, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _slot(page_table, row, pos, ps):
    return int(page_table[row, pos // ps]) * ps + pos % ps


@pytest.mark.parametrize("ps,hq,hkv", [(16, 8, 2), (1, 8, 4), (7, 6, 3)])
def test_decode_graph_replays_match_eager_and_oracle(ps, hq, hkv):
    d, cap, max_b = 128, 700, 8
    # one pool and page table for every replay: 8 requests with room for
    # `cap` tokens each
    wl = build_case(300 + ps, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[cap - 1] * max_b, extend_lens=[1] * max_b)
    pt = wl.page_table
    pool = wl.pool.cuda()
    pt_dev = torch.from_numpy(pt).cuda()
    layer = wl.layer
    _say(f"capture ps={ps} hq={hq} hkv={hkv} batch={max_b} max_seq_len={cap}")
    g = msgl.DecodeGraph(pool, layer, max_b, hq, cap, pt_dev)
    rng = np.random.default_rng(7 + ps)
    gen = torch.Generator().manual_seed(11 + ps)
    for it, b in enumerate([8, 5, 1, 8, 3]):
        rows = rng.choice(max_b, b, replace=False)
        table_idx = wl.phases[0].table_idx[rows].astype(np.int32)
        seq_lens = rng.integers(1, cap + 1, b).astype(np.int32)
        seq_lens[0] = cap  # the longest length the graph is sized for
        out_loc = np.array([_slot(pt, table_idx[i], int(seq_lens[i]) - 1, ps) for i in range(b)],
                           np.int32)
        q = (torch.randn((b, hq, d), generator=gen)).to(torch.bfloat16)
        k = (torch.randn((b, hkv, d), generator=gen)).to(torch.bfloat16)
        v = (torch.randn((b, hkv, d), generator=gen)).to(torch.bfloat16)
        # eager reference on a copy of the pool as it stands
        pool_e = pool.clone()
        msgl.store_kv(pool_e, layer, k.cuda(), v.cuda(), _i32(out_loc))
        out_e = msgl.paged_decode(pool_e, layer, q.cuda(), pt_dev, _i32(table_idx), _i32(seq_lens),
                                  cap)
        pool_before = bits(pool)
        _say(f"replay {it}: b={b} lens={seq_lens.tolist()}")
        out_g = g.run(q.cuda(), k.cuda(), v.cuda(), _i32(out_loc), _i32(table_idx),
                      _i32(seq_lens)).clone()
        pad = g.out[b:].clone()
        # unrelated eager work on the same stream between replays
        scratch = torch.ones(1 << 20, device="cuda").cumsum(0)
        torch.cuda.synchronize()
        assert float(scratch[-1]) == float(1 << 20)
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), "graph != eager"
        assert torch.equal(pool.view(torch.int16), pool_e.view(torch.int16)), "pool differs"
        assert torch.count_nonzero(pad.view(torch.int16)).item() == 0, "padding rows not zero"
        ref_pool = oracle.store_kv(pool_before, layer, bits(k), bits(v), out_loc)
        assert np.array_equal(bits(pool), ref_pool)
        ref = oracle.paged_decode(ref_pool, layer, bits(q), pt, table_idx, seq_lens)
        got = widen(bits(out_g), np.float64)
        ok, max_abs, max_rel, rel_l2 = close_report(got, ref, ATOL, RTOL)
        _say(f"replay {it}: max_abs={max_abs:.3e} max_rel={max_rel:.3e} rel_l2={rel_l2:.3e}")
        assert ok and rel_l2 <= REL_L2
    g.close()


@pytest.mark.parametrize("ps,hq,hkv,max_b", [(16, 32, 8, 8), (1, 8, 4, 13)])
def test_graph_runner_picks_nearest_size_and_matches_oracle(ps, hq, hkv, max_b):
    # one graph per size 1, 2, 4, ... and max_b; each batch replays the
    # smallest size >= b and equals the eager calls and the oracle
    d, cap = 128, 600
    wl = build_case(340 + ps, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[cap - 1] * max_b, extend_lens=[1] * max_b)
    pt = wl.page_table
    pool = wl.pool.cuda()
    pt_dev = torch.from_numpy(pt).cuda()
    _say(f"runner ps={ps} hq={hq} hkv={hkv} max_batch={max_b}")
    g = msgl.DecodeGraphRunner(pool, 0, max_b, hq, cap, pt_dev)
    expect = sorted({min(1 << i, max_b) for i in range(8)})
    assert g.sizes == expect
    assert g.pick(0) == 0 and g.pick(max_b + 1) == 0
    for b in range(1, max_b + 1):
        assert g.pick(b) == min(s for s in expect if s >= b)
    rng = np.random.default_rng(17 + ps)
    gen = torch.Generator().manual_seed(19 + ps)
    for it, b in enumerate([max_b, 5, 1, 3, 2, max_b - 1, 4]):
        rows = rng.choice(max_b, b, replace=False)
        table_idx = wl.phases[0].table_idx[rows].astype(np.int32)
        seq_lens = rng.integers(1, cap + 1, b).astype(np.int32)
        out_loc = np.array([_slot(pt, table_idx[i], int(seq_lens[i]) - 1, ps) for i in range(b)],
                           np.int32)
        q = (torch.randn((b, hq, d), generator=gen)).to(torch.bfloat16)
        k = (torch.randn((b, hkv, d), generator=gen)).to(torch.bfloat16)
        v = (torch.randn((b, hkv, d), generator=gen)).to(torch.bfloat16)
        pool_e = pool.clone()
        msgl.store_kv(pool_e, 0, k.cuda(), v.cuda(), _i32(out_loc))
        out_e = msgl.paged_decode(pool_e, 0, q.cuda(), pt_dev, _i32(table_idx), _i32(seq_lens), cap)
        pool_before = bits(pool)
        _say(f"runner replay {it}: b={b} size={g.pick(b)}")
        out_g = g.run(q.cuda(), k.cuda(), v.cuda(), _i32(out_loc), _i32(table_idx),
                      _i32(seq_lens)).clone()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), "graph != eager"
        assert torch.equal(pool.view(torch.int16), pool_e.view(torch.int16)), "pool differs"
        ref_pool = oracle.store_kv(pool_before, 0, bits(k), bits(v), out_loc)
        ref = oracle.paged_decode(ref_pool, 0, bits(q), pt, table_idx, seq_lens)
        ok, max_abs, max_rel, rel_l2 = close_report(widen(bits(out_g), np.float64), ref, ATOL, RTOL)
        _say(f"runner replay {it}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}")
        assert ok and rel_l2 <= REL_L2
    with pytest.raises(ValueError):
        g.run(*(torch.zeros((max_b + 1,) + t, dtype=torch.bfloat16, device="cuda")
                for t in ((hq, d), (hkv, d), (hkv, d))),
              *(torch.zeros(max_b + 1, dtype=torch.int32, device="cuda") for _ in range(3)))
    g.close()


def test_decode_graph_static_buffers_and_repeat_launch():
    # filling the static buffers directly and launching twice gives the same
    # output twice (no state carried between launches)
    ps, hq, hkv, d, cap, B = 16, 8, 2, 64, 300, 4
    wl = build_case(321, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[cap - 1] * B, extend_lens=[1] * B)
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    pt_dev = torch.from_numpy(wl.page_table).cuda()
    g = msgl.DecodeGraph(pool, 0, B, hq, cap, pt_dev)
    g.q.copy_(ph.q.cuda())
    g.k.copy_(ph.k.cuda())
    g.v.copy_(ph.v.cuda())
    g.out_loc.copy_(_i32(ph.out_loc))
    g.table_idx.copy_(_i32(ph.table_idx))
    g.seq_lens.copy_(_i32(ph.seq_lens))
    _say("static-buffer launches")
    g.launch()
    first = g.out.clone()
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), g.out.view(torch.int16))
    ref_pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    ref = oracle.paged_decode(ref_pool, 0, bits(ph.q), wl.page_table, ph.table_idx, ph.seq_lens)
    ok, max_abs, max_rel, rel_l2 = close_report(widen(bits(first), np.float64), ref, ATOL, RTOL)
    assert ok and rel_l2 <= REL_L2
    g.close()


def test_decode_graph_rejects_bad_arguments():
    pool = torch.zeros((2, 1, 8, 16, 2, 128), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(msgl.MsglError):
        msgl.DecodeGraph(pool, 0, 4, 7, 64, pt)  # 7 q heads over 2 kv heads
    with pytest.raises(msgl.MsglError):
        msgl.DecodeGraph(pool, 0, 4, 8, 16 * 9, pt)  # max_seq_len beyond the table width


def test_eager_calls_capture_in_a_torch_graph_over_layers():
    # the eager calls are capturable as they are: several layers of store_kv
    # + decode in one torch graph, replayed with fresh inputs, equal the
    # eager calls bit for bit
    ps, hq, hkv, d, cap, B, NL = 16, 8, 2, 128, 400, 4, 3
    wl = build_case(331, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[cap - 1] * B, extend_lens=[1] * B)
    ph = wl.phases[0]
    gen = torch.Generator().manual_seed(5)
    pool = torch.randn((2, NL) + tuple(wl.pool.shape[2:]), generator=gen).to(torch.bfloat16).cuda()
    pool_e = pool.clone()
    pt = torch.from_numpy(wl.page_table).cuda()
    loc, ti, sl = _i32(ph.out_loc), _i32(ph.table_idx), _i32(ph.seq_lens)
    q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    ws = torch.zeros(max(msgl.paged_decode_workspace_size(B, hq, d, cap, ps), 256), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(NL)]

    def step(pl, o):
        for layer in range(NL):
            msgl.store_kv(pl, layer, k, v, loc)
            msgl.paged_decode(pl, layer, q, pt, ti, sl, cap, out=o[layer], workspace=ws)

    step(pool, outs)  # warm up outside the capture
    torch.cuda.synchronize()
    tg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(tg):
        step(pool, outs)
    step(pool_e, [torch.empty_like(o) for o in outs])  # keep the two pools in step
    for it in range(3):
        q.copy_(torch.randn((B, hq, d), generator=gen).to(torch.bfloat16))
        k.copy_(torch.randn((B, hkv, d), generator=gen).to(torch.bfloat16))
        v.copy_(torch.randn((B, hkv, d), generator=gen).to(torch.bfloat16))
        _say(f"torch-graph replay {it}")
        tg.replay()
        ref = [torch.empty_like(o) for o in outs]
        step(pool_e, ref)
        torch.cuda.synchronize()
        for layer in range(NL):
            assert torch.equal(outs[layer].view(torch.int16), ref[layer].view(torch.int16))
        assert torch.equal(pool.view(torch.int16), pool_e.view(torch.int16))
