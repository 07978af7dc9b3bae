"""Seeded random cases through store_kv and the three attention calls, on
gfx950: every output element against the oracle.

Each case draws its geometry -- head_dim 64 or 128, 1 to 8 kv heads, 1 to
16 q heads per kv head, page size 1 to 64 (powers of two and not) -- its
q/k/v scale (std 0.5, 1 or 2) and a length mix for one of the calls:
  * decode: up to 200 requests, lengths from a lognormal (median 300,
    up to 4000), some padding rows (length 0);
  * extend: up to 16 requests, prefixes up to 1000 and 0 to 200 new tokens
    (some requests with none);
  * mixed: up to 64 requests, most with one new token, some with none and
    some with 2 to 200.
The pool bits after store_kv must equal the oracle's; attention outputs
meet the parity tolerance (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|,
relative L2 <= 5e-3) and leave the guard rows around them untouched.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits
from tests.test_gpu_parity import Guarded, assert_close
from workloads import build_case

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-random] {msg}", file=sys.stderr, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


KINDS = ("decode", "extend", "mixed")


def _draw(seed):
    rng = np.random.default_rng(20_000 + seed)
    kind = KINDS[seed % 3]
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    ps = int(rng.choice([1, 2, 3, 5, 16, 64]))
    std = float(rng.choice([0.5, 1.0, 2.0]))
    if kind == "decode":
        B = int(rng.integers(1, 201))
        L = np.clip(rng.lognormal(np.log(300), 1.0, B), 1, 4000).astype(np.int64)
        P, E = list(L - 1), [1] * B
    elif kind == "extend":
        B = int(rng.integers(1, 17))
        P = [int(x) for x in rng.integers(0, 1001, B)]
        E = [int(x) for x in rng.integers(0, 201, B)]
        E[int(rng.integers(0, B))] = max(E[0], 1)  # at least one row
    else:
        B = int(rng.integers(2, 65))
        P = [int(x) for x in rng.integers(0, 1500, B)]
        E = [int(x) for x in rng.choice([1, 1, 1, 1, 0, -1], B)]
        E = [int(rng.integers(2, 201)) if e < 0 else e for e in E]
        E[0] = 1
    return kind, d, hkv, G, ps, std, P, E


@pytest.mark.parametrize("seed", range(72))
def test_random_case(seed):
    kind, d, hkv, G, ps, std, P, E = _draw(seed)
    hq = hkv * G
    _say(f"seed {seed}: {kind} d={d} hkv={hkv} G={G} ps={ps} std={std} B={len(P)} "
         f"tokens={sum(E)} max_len={max(p + e for p, e in zip(P, E))}")
    wl = build_case(30_000 + seed, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=P, extend_lens=E, std=std,
                    kind="decode" if kind == "decode" else "extend")
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    pt = torch.from_numpy(wl.page_table).cuda()
    msgl.store_kv(pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    q = ph.q.cuda()
    g = Guarded(q.shape[0], hq, d)
    ti = _i32(ph.table_idx)
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    if kind == "decode":
        seq = ph.seq_lens.astype(np.int32).copy()
        pad = np.random.default_rng(seed).random(len(seq)) < 0.05
        seq[pad] = 0
        msgl.paged_decode(pool, 0, q, pt, ti, _i32(seq), int(max(seq.max(), 1)), out=g.out)
        ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx, seq,
                                  blocked=True)
    else:
        call = msgl.paged_extend if kind == "extend" else msgl.paged_mixed
        call(pool, 0, q, pt, ti, _i32(ph.prefix_lens), _i32(ph.extend_lens),
             _i32(ph.cu_extend_lens), int(ph.extend_lens.max()), int(ph.seq_lens.max()),
             out=g.out)
        ref = oracle.paged_attention_blocked(pool_bits, 0, bits(ph.q), wl.page_table,
                                             ph.table_idx, ph.prefix_lens, ph.extend_lens)
    torch.cuda.synchronize()
    g.check(f"seed {seed}")
    assert np.array_equal(bits(pool), pool_bits), f"seed {seed}: pool differs after store_kv"
    assert_close(g.out, ref, what=f"seed {seed} {kind}")
