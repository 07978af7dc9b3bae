"""Device-side page allocation (msgl_alloc_pages) against the oracle, on
gfx950: bit-exact page tables, out_loc and free counts over a sequence of
steps that drain the free list, batches above one workgroup's 1024
requests, every failure code (nothing changed), and an allocate -> store_kv
-> decode pipeline against the oracle.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-alloc] {msg}", file=sys.stderr, flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class State:
    def __init__(self, rng, B, ps, npages, width, spare=3):
        self.ps = ps
        self.rows = rng.permutation(B + spare)[:B].astype(np.int32)
        self.pt = np.full((B + spare, width), -1, np.int32)
        self.free = rng.permutation(npages).astype(np.int32)
        self.nfree = npages
        self.P = np.zeros(B, np.int64)


def _step_both(st, d_free, d_nfree, d_pt, E, cap=None):
    B = len(st.rows)
    ok, nf2, pt2, loc = oracle.alloc_pages(st.free, st.nfree, st.pt, st.rows, st.P, E, st.ps)
    cap = int(E.sum()) if cap is None else cap
    d_loc = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")
    d_status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    msgl.alloc_pages(d_free, d_nfree, d_pt, _dev(st.rows), _dev(st.P), _dev(E), st.ps,
                     d_loc[:cap] if cap > 0 else d_loc[:0], d_status)
    torch.cuda.synchronize()
    return ok, nf2, pt2, loc, d_loc, int(d_status.item())


@pytest.mark.parametrize("B,ps", [(50, 16), (1500, 1), (2100, 7)])
def test_alloc_steps_match_oracle(B, ps):
    rng = np.random.default_rng(B + ps)
    width = 64
    st = State(rng, B, ps, npages=B * width, width=width)
    d_free, d_nfree, d_pt = _dev(st.free), _dev([st.nfree]), _dev(st.pt)
    for it in range(4):
        E = rng.integers(0, 3 * ps + 2, B).astype(np.int64)
        E[rng.integers(0, B)] = 0
        if it == 0:
            E[:2] = [ps * 5 + 1, 1]
        _say(f"B={B} ps={ps} step {it}: {int(E.sum())} new tokens")
        ok, nf2, pt2, loc, d_loc, code = _step_both(st, d_free, d_nfree, d_pt, E)
        assert ok and code == 0
        assert int(d_nfree.item()) == nf2
        assert np.array_equal(d_pt.cpu().numpy(), pt2)
        assert np.array_equal(d_loc[:len(loc)].cpu().numpy(), loc)
        st.pt, st.nfree, st.P = pt2, nf2, st.P + E


def test_alloc_failures_change_nothing():
    rng = np.random.default_rng(9)
    B, ps, width = 6, 4, 8
    st = State(rng, B, ps, npages=10, width=width)
    d_free, d_nfree, d_pt = _dev(st.free), _dev([st.nfree]), _dev(st.pt)
    cases = [
        ("not enough pages", np.full(B, 8), None, 1),          # 12 pages > 10 free
        ("row too short", np.array([40, 0, 0, 0, 0, 0]), None, 2),  # 10 pages > 8 entries
        ("negative length", np.array([1, -1, 0, 0, 0, 0]), None, 3),
        ("out_loc too small", np.array([3, 3, 0, 0, 0, 0]), 5, 4),
    ]
    for what, E, cap, want in cases:
        _say(what)
        before_pt = d_pt.clone()
        _, _, _, _, d_loc, code = _step_both(st, d_free, d_nfree, d_pt, E.astype(np.int64), cap)
        assert code == want, (what, code)
        assert int(d_nfree.item()) == 10
        assert torch.equal(d_pt, before_pt)
        assert torch.all(d_loc == -7)


def test_allocate_store_decode_pipeline():
    # allocate pages for a batch's prompt, store its K/V rows, then decode one
    # new token per request, all through device-side metadata
    rng = np.random.default_rng(21)
    B, ps, hq, hkv, d, npages = 5, 16, 8, 2, 128, 64
    st = State(rng, B, ps, npages=npages, width=16)
    d_free, d_nfree, d_pt = _dev(st.free), _dev([st.nfree]), _dev(st.pt)
    gen = torch.Generator().manual_seed(3)
    pool = (torch.randn((2, 1, npages, ps, hkv, d), generator=gen)).to(torch.bfloat16)
    d_pool = pool.cuda()
    pool_bits = bits(pool)
    for E in (rng.integers(1, 120, B), np.ones(B, np.int64)):
        E = E.astype(np.int64)
        ok, nf2, pt2, loc, d_loc, code = _step_both(st, d_free, d_nfree, d_pt, E)
        assert ok and code == 0
        T = int(E.sum())
        k = torch.randn((T, hkv, d), generator=gen).to(torch.bfloat16)
        v = torch.randn((T, hkv, d), generator=gen).to(torch.bfloat16)
        msgl.store_kv(d_pool, 0, k.cuda(), v.cuda(), d_loc[:T])
        pool_bits = oracle.store_kv(pool_bits, 0, bits(k), bits(v), loc)
        st.pt, st.nfree, st.P = pt2, nf2, st.P + E
    torch.cuda.synchronize()
    assert np.array_equal(bits(d_pool), pool_bits)
    q = torch.randn((B, hq, d), generator=gen).to(torch.bfloat16)
    L = st.P.astype(np.int32)
    out = msgl.paged_decode(d_pool, 0, q.cuda(), d_pt, _dev(st.rows), _dev(L), int(L.max()))
    torch.cuda.synchronize()
    ref = oracle.paged_decode(pool_bits, 0, bits(q), st.pt, st.rows, L)
    got = oracle.bf16_bits_to_float(bits(out), np.float64)
    assert np.all(np.abs(got - ref) <= 1e-2 + 1e-2 * np.abs(ref))
