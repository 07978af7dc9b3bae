"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against an independent fact: a library attention
routine on contiguous KV, scalar brute force, invariances the definition
implies, closed forms, a hand-worked example, and mask probes.  Together they
are meant to fail on a dropped term, a wrong sign or index, a swapped K/V,
a wrong head mapping, a wrong slot formula or a misaligned causal mask.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import build_case, config_tiny
from tests._util import bits, widen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _place_contiguous(K, V, page_size, pages, num_pages):
    """Pool (bits) holding logical K/V rows (L, Hkv, d) on the given pages,
    placed with explicit 6-D indexing, plus random filler elsewhere."""
    L, hkv, d = K.shape
    rng = np.random.default_rng(123)
    pool = rng.integers(0, 1 << 16, size=(2, 1, num_pages, page_size, hkv, d), dtype=np.uint32).astype(np.uint16)
    # keep filler finite: clear the exponent's top bit pattern 0xFF
    pool &= np.uint16(0xBFFF)
    for p in range(L):
        pool[0, 0, pages[p // page_size], p % page_size] = K[p]
        pool[1, 0, pages[p // page_size], p % page_size] = V[p]
    return pool


def _sdpa_dense(Q, K, V, P, sm_scale):
    """float64 attention on contiguous KV via torch SDPA with an explicit
    bottom-right causal mask; K/V heads expanded to q heads by h // G."""
    E, hq, d = Q.shape
    L, hkv, _ = K.shape
    G = hq // hkv
    q = torch.from_numpy(Q).permute(1, 0, 2).unsqueeze(0)  # (1, hq, E, d)
    k = torch.from_numpy(K).repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
    v = torch.from_numpy(V).repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
    i = torch.arange(E).unsqueeze(1)
    j = torch.arange(L).unsqueeze(0)
    mask = j <= (P + i)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=sm_scale)
    return o.squeeze(0).permute(1, 0, 2).numpy()


def _rand_bf16_bits(rng, shape, std=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(std)
    return oracle.float_to_bf16_bits(x)


@pytest.mark.parametrize("hq,hkv,d,ps,P,E", [
    (4, 1, 64, 16, 100, 16),
    (8, 2, 128, 16, 37, 29),
    (4, 4, 64, 1, 0, 40),
    (6, 2, 64, 4, 63, 1),
    (16, 2, 128, 8, 200, 5),
])
@pytest.mark.parametrize("layout", ["identity", "permuted"])
def test_p1_dense_contiguous(hq, hkv, d, ps, P, E, layout):
    rng = np.random.default_rng(hash((hq, hkv, d, ps, P, E)) & 0xFFFF)
    L = P + E
    Kb = _rand_bf16_bits(rng, (L, hkv, d))
    Vb = _rand_bf16_bits(rng, (L, hkv, d))
    Qb = _rand_bf16_bits(rng, (E, hq, d))
    npg = -(-L // ps) + 3
    pages = np.arange(npg) if layout == "identity" else rng.permutation(npg)
    pool = _place_contiguous(Kb, Vb, ps, pages, npg)
    pt = np.full((2, npg), -1, np.int32)
    pt[1, : -(-L // ps)] = pages[: -(-L // ps)]
    sm = 1.0 / math.sqrt(d)
    ref = _sdpa_dense(widen(Qb), widen(Kb), widen(Vb), P, sm)
    got32 = oracle.paged_attention(pool, 0, Qb, pt, [1], [P], [E])
    got64 = oracle.paged_attention(pool, 0, Qb, pt, [1], [P], [E], dtype=np.float64)
    assert np.abs(got64 - ref).max() <= 1e-10
    assert np.abs(got32 - ref).max() <= 1e-5
    # the blocked (matrix) form, with blocks that split the query rows
    for block in (1, 7, 256):
        b32 = oracle.paged_attention_blocked(pool, 0, Qb, pt, [1], [P], [E], block=block)
        b64 = oracle.paged_attention_blocked(pool, 0, Qb, pt, [1], [P], [E], dtype=np.float64,
                                             block=block)
        assert np.abs(b64 - ref).max() <= 1e-10
        assert np.abs(b32 - ref).max() <= 1e-5


def _brute(pool, layer, q, page_table, table_idx, P, E, sm_scale):
    """Scalar loops with math.exp; slots from the 6-D pool index directly."""
    two, nl, npg, ps, hkv, d = pool.shape
    T, hq, _ = q.shape
    G = hq // hkv
    out = np.zeros((T, hq, d))
    t0 = 0
    for r in range(len(P)):
        row = page_table[table_idx[r]]
        for i in range(E[r]):
            a = P[r] + i
            for h in range(hq):
                g = h // G
                qv = [widen(q[t0 + i, h, c]) for c in range(d)]
                s = []
                for j in range(a + 1):
                    page, off = row[j // ps], j % ps
                    kj = pool[0, layer, page, off, g]
                    s.append(sm_scale * sum(float(qv[c]) * float(widen(kj[c])) for c in range(d)))
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = sum(w)
                for c in range(d):
                    acc = 0.0
                    for j in range(a + 1):
                        page, off = row[j // ps], j % ps
                        acc += w[j] * float(widen(pool[1, layer, page, off, g, c]))
                    out[t0 + i, h, c] = acc / tot
        t0 += E[r]
    return out


def test_p2_brute_force_tiny_config():
    wl = config_tiny()
    pool = bits(wl.pool)
    for ph in wl.phases:
        pool = oracle.store_kv(pool, 0, bits(ph.k), bits(ph.v), ph.out_loc)
        q = bits(ph.q)
        got = oracle.paged_attention(pool, 0, q, wl.page_table, ph.table_idx, ph.prefix_lens,
                                     ph.extend_lens, dtype=np.float64)
        # brute force over a subset of rows/heads keeps the loop short
        ref = _brute(pool, 0, q, wl.page_table, ph.table_idx, ph.prefix_lens, ph.extend_lens,
                     1.0 / math.sqrt(wl.head_dim))
        assert np.abs(got - ref).max() <= 1e-9


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_p2_brute_force_random_tiny(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    ps = int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 4))
    P = rng.integers(0, 9, B)
    E = rng.integers(1, 5, B)
    wl = build_case(seed, num_qo_heads=hkv * G, num_kv_heads=hkv, head_dim=8, page_size=ps,
                    prefix_lens=P, extend_lens=E)
    ph = wl.phases[0]
    pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    q = bits(ph.q)
    got = oracle.paged_attention(pool, 0, q, wl.page_table, ph.table_idx, P, E, dtype=np.float64)
    ref = _brute(pool, 0, q, wl.page_table, ph.table_idx, P, E, 1.0 / math.sqrt(8))
    assert np.abs(got - ref).max() <= 1e-9
    got32 = oracle.paged_attention(pool, 0, q, wl.page_table, ph.table_idx, P, E)
    assert np.abs(got32 - ref).max() <= 1e-5
    blk = oracle.paged_attention_blocked(pool, 0, q, wl.page_table, ph.table_idx, P, E,
                                         dtype=np.float64, block=2)
    assert np.abs(blk - ref).max() <= 1e-9


def _stored_case(seed=21, **kw):
    args = dict(num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                prefix_lens=[40, 0, 130], extend_lens=[9, 33, 1])
    args.update(kw)
    wl = build_case(seed, **args)
    ph = wl.phases[0]
    pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    return wl, ph, pool


def test_p3_page_permutation_invariance():
    wl, ph, pool = _stored_case()
    base = oracle.paged_attention(pool, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                  ph.prefix_lens, ph.extend_lens)
    rng = np.random.default_rng(5)
    perm = rng.permutation(wl.num_pages)
    pool2 = np.empty_like(pool)
    pool2[:, :, perm] = pool
    pt2 = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1).astype(np.int32)
    moved = oracle.paged_attention(pool2, 0, bits(ph.q), pt2, ph.table_idx, ph.prefix_lens,
                                   ph.extend_lens)
    assert np.array_equal(base, moved)


def test_p4_page_size_1_vs_16():
    wl, ph, pool = _stored_case()
    base = oracle.paged_attention(pool, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                  ph.prefix_lens, ph.extend_lens)
    two, nl, npg, ps, hkv, d = pool.shape
    pool1 = pool.reshape(2, nl, npg * ps, 1, hkv, d)
    # token-granular table: entry p of a row is the slot of token p
    width = wl.page_table.shape[1] * ps
    pt1 = np.full((wl.page_table.shape[0], width), -1, np.int32)
    for row in range(wl.page_table.shape[0]):
        for p in range(width):
            page = wl.page_table[row, p // ps]
            if page >= 0:
                pt1[row, p] = page * ps + p % ps
    tok = oracle.paged_attention(pool1, 0, bits(ph.q), pt1, ph.table_idx, ph.prefix_lens,
                                 ph.extend_lens)
    assert np.array_equal(base, tok)
    # and scattered differently at page size 1
    rng = np.random.default_rng(9)
    perm = rng.permutation(npg * ps)
    pool1b = np.empty_like(pool1)
    pool1b[:, :, perm] = pool1
    pt1b = np.where(pt1 >= 0, perm[np.maximum(pt1, 0)], -1).astype(np.int32)
    tok2 = oracle.paged_attention(pool1b, 0, bits(ph.q), pt1b, ph.table_idx, ph.prefix_lens,
                                  ph.extend_lens)
    assert np.array_equal(base, tok2)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_p5_single_key_returns_v(dtype):
    for kind, P, E in (("decode", [0], [1]), ("extend", [0], [1])):
        wl = build_case(31, num_qo_heads=4, num_kv_heads=2, head_dim=128, page_size=16,
                        prefix_lens=P, extend_lens=E, kind=kind)
        ph = wl.phases[0]
        pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
        if kind == "decode":
            out = oracle.paged_decode(pool, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                      ph.seq_lens, dtype=dtype)
        else:
            out = oracle.paged_attention(pool, 0, bits(ph.q), wl.page_table, ph.table_idx, P, E,
                                         dtype=dtype)
        v = widen(bits(ph.v), dtype)  # (1, hkv, d)
        expect = np.repeat(v, 2, axis=1)  # q head h reads kv head h // 2
        assert np.array_equal(out, expect)


def test_p6_uniform_weights_closed_form():
    d, ps = 64, 16
    P, E = 1000, 37
    L = P + E
    hq, hkv = 4, 2
    # V_j = one-hot(j mod d); q = 0 makes every weight equal
    Kb = oracle.float_to_bf16_bits(np.random.default_rng(1).standard_normal((L, hkv, d)))
    V = np.zeros((L, hkv, d), np.float32)
    V[np.arange(L), :, np.arange(L) % d] = 1.0
    Vb = oracle.float_to_bf16_bits(V)
    npg = -(-L // ps)
    pages = np.random.default_rng(2).permutation(npg)
    pool = _place_contiguous(Kb, Vb, ps, pages, npg)
    pt = pages[None, :].astype(np.int32)
    Qb = np.zeros((E, hq, d), np.uint16)
    got = oracle.paged_attention(pool, 0, Qb, pt, [0], [P], [E])
    blk = oracle.paged_attention_blocked(pool, 0, Qb, pt, [0], [P], [E], block=16)
    for i in range(E):
        a = P + i
        counts = np.array([len(range(c, a + 1, d)) for c in range(d)], np.float64)
        expect = counts / (a + 1)
        assert np.abs(got[i] - expect[None, :]).max() <= 1e-6
        assert np.abs(blk[i] - expect[None, :]).max() <= 1e-6


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_p7_boundary_probes(dtype):
    d, ps, hq, hkv = 64, 16, 2, 1
    P, E = 45, 12
    L = P + E
    rng = np.random.default_rng(77)
    V = rng.standard_normal((L, hkv, d)).astype(np.float32)
    Vb = oracle.float_to_bf16_bits(V)
    Vw = widen(Vb, np.float64)
    npg = -(-L // ps) + 1
    pages = rng.permutation(npg)
    pt = pages[None, :].astype(np.int32)
    Qb = np.zeros((E, hq, d), np.uint16)
    K = np.zeros((L, hkv, d), np.float32)
    # query row i probes with channel c_i; leak probe on key a+1, mirror probe on key a
    for i in range(E):
        Qb[i, :, i] = oracle.float_to_bf16_bits(np.float32(64.0))
    leak_K = K.copy()
    mirror_K = K.copy()
    for i in range(E):
        a = P + i
        if a + 1 < L:
            leak_K[a + 1, :, i] = 64.0
        mirror_K[a, :, i] = 64.0
    for KK, kind in ((leak_K, "leak"), (mirror_K, "mirror")):
        pool = _place_contiguous(oracle.float_to_bf16_bits(KK), Vb, ps, pages, npg)
        for attend in (oracle.paged_attention,
                       lambda *a, **k: oracle.paged_attention_blocked(*a, block=5, **k)):
            got = attend(pool, 0, Qb, pt, [0], [P], [E], dtype=dtype)
            for i in range(E):
                a = P + i
                if kind == "leak":
                    expect = Vw[: a + 1, 0].mean(axis=0)
                    assert np.abs(got[i] - expect[None]).max() <= 1e-5
                else:
                    if dtype == np.float32:
                        assert np.array_equal(got[i], np.repeat(Vw[a:a + 1, 0], hq, 0).astype(dtype))
                    else:
                        assert np.abs(got[i] - Vw[a, 0][None]).max() <= 1e-200


def test_p8_chunked_equals_one_shot():
    d, ps, hq, hkv = 64, 16, 4, 2
    total, chunk = 256, 64
    rng = np.random.default_rng(88)
    Kb = _rand_bf16_bits(rng, (total, hkv, d), 0.5)
    Vb = _rand_bf16_bits(rng, (total, hkv, d), 0.5)
    Qb = _rand_bf16_bits(rng, (total, hq, d), 0.5)
    npg = total // ps + 2
    pages = rng.permutation(npg)
    pool = _place_contiguous(Kb, Vb, ps, pages, npg)
    pt = pages[None, :].astype(np.int32)
    one = oracle.paged_attention(pool, 0, Qb, pt, [0], [0], [total])
    pieces = [oracle.paged_attention(pool, 0, Qb[c:c + chunk], pt, [0], [c], [chunk])
              for c in range(0, total, chunk)]
    assert np.array_equal(one, np.concatenate(pieces))


def test_p9_shared_vs_private_prefix():
    wl = build_case(41, num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                    prefix_lens=[64, 64, 64], extend_lens=[20, 7, 33], shared_prefix=True,
                    num_pages=64)
    ph = wl.phases[0]
    pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    shared = oracle.paged_attention(pool, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                    ph.prefix_lens, ph.extend_lens)
    # copy the shared prefix pages to private pages for requests 1 and 2
    pt = wl.page_table.copy()
    used = set(int(x) for x in pt.ravel() if x >= 0)
    free = [p for p in range(wl.num_pages) if p not in used]
    pool2 = pool.copy()
    for r in (1, 2):
        row = ph.table_idx[r]
        for lp in range(4):
            newp = free.pop()
            pool2[:, :, newp] = pool[:, :, pt[row, lp]]
            pt[row, lp] = newp
    private = oracle.paged_attention(pool2, 0, bits(ph.q), pt, ph.table_idx, ph.prefix_lens,
                                     ph.extend_lens)
    assert np.array_equal(shared, private)


def test_p10_gqa_equals_mha_with_repeated_kv():
    wl, ph, pool = _stored_case(num_qo_heads=8, num_kv_heads=2)
    gqa = oracle.paged_attention(pool, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                 ph.prefix_lens, ph.extend_lens, dtype=np.float64)
    G = 4
    pool_mha = np.repeat(pool, G, axis=4)  # kv head g copied to heads g*G .. g*G+G-1
    mha = oracle.paged_attention(pool_mha, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                 ph.prefix_lens, ph.extend_lens, dtype=np.float64)
    assert np.abs(gqa - mha).max() <= 1e-12


def test_p11_store_kv_roundtrip_and_canaries():
    wl = build_case(51, num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                    prefix_lens=[5, 17, 0], extend_lens=[11, 1, 40])
    ph = wl.phases[0]
    before = bits(wl.pool)
    after = oracle.store_kv(before, 0, bits(ph.k), bits(ph.v), ph.out_loc)
    # rows not named by out_loc are untouched (canaries)
    two, nl, npg, ps, hkv, d = before.shape
    flat_b = before.reshape(2, npg * ps, hkv, d)
    flat_a = after.reshape(2, npg * ps, hkv, d)
    others = np.setdiff1d(np.arange(npg * ps), ph.out_loc)
    assert np.array_equal(flat_a[:, others], flat_b[:, others])
    # brute-force placement through the 6-D index
    kb, vb = bits(ph.k), bits(ph.v)
    for t, s in enumerate(ph.out_loc):
        assert np.array_equal(after[0, 0, s // ps, s % ps], kb[t])
        assert np.array_equal(after[1, 0, s // ps, s % ps], vb[t])
    # store-then-gather through the page table returns the inserted rows
    t0 = 0
    for r in range(ph.batch):
        L = int(ph.seq_lens[r])
        k, v = oracle.gather_kv(after, 0, wl.page_table, int(ph.table_idx[r]), L)
        e = int(ph.extend_lens[r])
        assert np.array_equal(k[L - e:], kb[t0:t0 + e])
        assert np.array_equal(v[L - e:], vb[t0:t0 + e])
        t0 += e
    # padding rows (out_loc < 0) write nothing; repeated slots are refused
    loc = ph.out_loc.copy()
    loc[::2] = -1
    pad = oracle.store_kv(before, 0, kb, vb, loc)
    for t, s in enumerate(ph.out_loc):
        src = before if t % 2 == 0 else None
        got = pad[0, 0, s // ps, s % ps]
        assert np.array_equal(got, before[0, 0, s // ps, s % ps] if src is not None else kb[t])
    dup = ph.out_loc.copy()
    dup[1] = dup[0]
    with pytest.raises(AssertionError):
        oracle.store_kv(before, 0, kb, vb, dup)


def test_p12_convex_hull():
    wl, ph, pool = _stored_case(seed=61)
    out = oracle.paged_attention(pool, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                 ph.prefix_lens, ph.extend_lens)
    G = wl.group
    t0 = 0
    for r in range(ph.batch):
        L = int(ph.seq_lens[r])
        _, vb = oracle.gather_kv(pool, 0, wl.page_table, int(ph.table_idx[r]), L)
        V = widen(vb, np.float32)
        for i in range(int(ph.extend_lens[r])):
            a = int(ph.prefix_lens[r]) + i
            for h in range(wl.num_qo_heads):
                lo = V[: a + 1, h // G].min(axis=0)
                hi = V[: a + 1, h // G].max(axis=0)
                o = out[t0 + i, h]
                assert np.all(o >= lo - 1e-6) and np.all(o <= hi + 1e-6)
        t0 += int(ph.extend_lens[r])


def test_golden_hand_example():
    with open(os.path.join(GOLDEN, "hand_paged_example.json")) as f:
        g = json.load(f)
    geo = g["geometry"]
    npg, ps, hkv, d = geo["num_pages"], geo["page_size"], geo["num_kv_heads"], geo["head_dim"]
    pool = np.zeros((2, 1, npg, ps, hkv, d), np.uint16)
    for s, (kr, vr) in enumerate(zip(g["pool_K_by_slot"], g["pool_V_by_slot"])):
        pool[0, 0, s // ps, s % ps, 0] = oracle.float_to_bf16_bits(np.array(kr, np.float32))
        pool[1, 0, s // ps, s % ps, 0] = oracle.float_to_bf16_bits(np.array(vr, np.float32))
    pt = np.array(g["page_table"], np.int32)
    ti = np.array(g["table_idx"], np.int32)
    qd = oracle.float_to_bf16_bits(np.array(g["decode"]["q"], np.float32))
    out = oracle.paged_decode(pool, 0, qd, pt, ti, g["decode"]["seq_lens"], dtype=np.float64)
    assert np.abs(out - np.array(g["decode"]["expected"])).max() <= 1e-12
    out32 = oracle.paged_decode(pool, 0, qd, pt, ti, g["decode"]["seq_lens"])
    assert np.abs(out32 - np.array(g["decode"]["expected"])).max() <= 1e-6
    qe = oracle.float_to_bf16_bits(np.array(g["extend"]["q"], np.float32))
    oute = oracle.paged_attention(pool, 0, qe, pt, ti, g["extend"]["prefix_lens"],
                                  g["extend"]["extend_lens"], dtype=np.float64)
    assert np.abs(oute - np.array(g["extend"]["expected"])).max() <= 1e-12


@pytest.mark.parametrize("seed", [81, 82])
def test_blocked_form_matches_row_form(seed):
    # the two evaluations of one definition, on ragged requests with
    # several blocks each, a shared prefix and sampled rows
    wl = build_case(seed, num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                    prefix_lens=[64, 64, 64], extend_lens=[70, 1, 33], shared_prefix=True)
    ph = wl.phases[0]
    pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    args = (pool, 0, bits(ph.q), wl.page_table, ph.table_idx, ph.prefix_lens, ph.extend_lens)
    row = oracle.paged_attention(*args, dtype=np.float64)
    blk = oracle.paged_attention_blocked(*args, dtype=np.float64, block=16)
    assert np.abs(row - blk).max() <= 1e-12
    some = [0, 5, 69, 70, 71, 103]
    part = oracle.paged_attention_blocked(*args, dtype=np.float64, block=3, only_tokens=some)
    assert np.abs(part[some] - row[some]).max() <= 1e-12
    others = np.setdiff1d(np.arange(ph.num_tokens), some)
    assert np.all(np.isnan(part[others]))
    dec = oracle.paged_decode(pool, 0, bits(ph.q)[:3], wl.page_table, ph.table_idx,
                              np.array([10, 0, 100]), dtype=np.float64)
    decb = oracle.paged_decode(pool, 0, bits(ph.q)[:3], wl.page_table, ph.table_idx,
                               np.array([10, 0, 100]), dtype=np.float64, blocked=True)
    assert np.abs(dec - decb).max() <= 1e-12 and np.all(decb[1] == 0)


def test_decode_padding_row_is_zero():
    wl = build_case(71, num_qo_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
                    prefix_lens=[20, 7], extend_lens=[1, 1])
    ph = wl.phases[0]
    pool = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    L = ph.seq_lens.copy()
    L[1] = 0
    out = oracle.paged_decode(pool, 0, bits(ph.q), wl.page_table, ph.table_idx, L)
    assert np.all(out[1] == 0)
    full = oracle.paged_decode(pool, 0, bits(ph.q), wl.page_table, ph.table_idx, ph.seq_lens)
    assert np.array_equal(out[0], full[0])


def test_bf16_rounding_helpers():
    # widening is exact and rounding is nearest-even
    x = np.array([1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.0e38, -0.0], np.float32)
    b = oracle.float_to_bf16_bits(x)
    back = oracle.bf16_bits_to_float(b)
    assert back[0] == 1.0 and back[1] == -2.5
    assert back[2] == 1.0  # tie -> even
    assert back[3] == 1.0 + 4 * 2 ** -8  # tie -> even (up)
    # 3.4e38 lies above the midpoint between the largest finite bf16
    # (0x7F7F, about 3.39e38) and 2^128, so round-to-nearest-even overflows
    # to +inf (0x7F80); the largest finite bf16 itself stays put
    assert oracle.float_to_bf16_bits(np.float32(3.4e38)) == 0x7F80
    assert np.isposinf(oracle.bf16_bits_to_float(oracle.float_to_bf16_bits(np.float32(3.4e38))))
    assert oracle.float_to_bf16_bits(oracle.bf16_bits_to_float(np.uint16(0x7F7F))) == 0x7F7F
    t = torch.tensor(x).to(torch.bfloat16)
    assert np.array_equal(bits(t)[:5], b[:5])
