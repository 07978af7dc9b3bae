"""Rotary embedding fused with store_kv, and the cos/sin table, on gfx950.

The fused call must match the oracle bit for bit: both read the same fp32
cos/sin table and round the exact rotation once to bf16 (q rotated in
place, rotated k and unchanged v stored at out_loc, padding rows skipped).
The table builder must match the closed form to one fp32 ulp.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits
from workloads import build_case

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-rope] {msg}", file=sys.stderr, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("max_pos,d,base", [(32768, 128, 10000.0), (4096, 64, 500000.0)])
def test_table_matches_closed_form(max_pos, d, base):
    _say(f"table {max_pos}x{d} base {base}")
    got = msgl.rope_cos_sin_table(max_pos, d, base).cpu().numpy()
    want = oracle.rope_table(max_pos, d, base).astype(np.float32)
    gi = got.view(np.int32).astype(np.int64)
    wi = want.view(np.int32).astype(np.int64)
    ulps = np.abs(gi - wi)
    _say(f"max ulp {ulps.max()}, differing {np.count_nonzero(ulps)} of {ulps.size}")
    assert ulps.max() <= 1


@pytest.mark.parametrize("hq,hkv,d,ps,merged", [(32, 8, 128, 16, False), (8, 1, 64, 1, False),
                                                (6, 3, 128, 7, True)])
def test_rope_store_kv_bit_exact(hq, hkv, d, ps, merged):
    T, max_pos = 300, 20000
    wl = build_case(400 + ps, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[0, 100, 37], extend_lens=[120, 100, 80])
    ph = wl.phases[0]
    assert ph.num_tokens == T
    rng = np.random.default_rng(ps)
    pos = rng.integers(0, max_pos, T).astype(np.int32)
    pos[:3] = [0, max_pos - 1, 1]
    loc = ph.out_loc.copy()
    loc[::11] = -1  # padding rows
    table = oracle.rope_table(max_pos, d, 10000.0).astype(np.float32)
    q_cpu, k_cpu, v_cpu = ph.q, ph.k, ph.v
    if merged:  # q, k, v as slices of one (T, hq + 2 hkv, d) projection
        qkv = torch.cat([q_cpu, k_cpu, v_cpu], dim=1).cuda()
        q, k, v = qkv[:, :hq], qkv[:, hq:hq + hkv], qkv[:, hq + hkv:]
    else:
        q, k, v = q_cpu.cuda(), k_cpu.cuda(), v_cpu.cuda()
    pool = wl.pool.cuda()
    _say(f"fused rope+store hq={hq} hkv={hkv} d={d} ps={ps} merged={merged}")
    msgl.rope_store_kv(pool, 0, q, k, v, _i32(loc), _i32(pos), torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    q_ref, pool_ref = oracle.rope_store_kv(bits(wl.pool), 0, bits(q_cpu), bits(k_cpu), bits(v_cpu),
                                           loc, pos, table)
    assert np.array_equal(bits(q.contiguous()), q_ref), "rotated q differs"
    assert np.array_equal(bits(pool), pool_ref), "pool differs"
    if merged:  # k and v inside the projection are left as they were
        assert torch.equal(k.cpu().view(torch.int16), k_cpu.view(torch.int16))
        assert torch.equal(v.cpu().view(torch.int16), v_cpu.view(torch.int16))


def test_rope_rounding_ties_overflow_and_tiny_values():
    # a crafted table and inputs that put the rotated values on the cases of
    # the rounding to bf16: exact ties at half a unit (even and odd
    # neighbours), values just above and below a tie, results past bf16's
    # largest finite value (to infinity), results below its normal range
    # (subnormal bf16), zeros; compared bit for bit with the oracle
    hq, hkv, d, ps, T = 4, 1, 64, 16, 64
    half = d // 2
    wl = build_case(460, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[0], extend_lens=[T])
    ph = wl.phases[0]
    rng = np.random.default_rng(460)
    table = np.zeros((4, d), np.float32)
    table[0, :half] = 1 + 2.0 ** -8                     # cos: x (1 + 2^-8), sin 0
    table[1, :half] = 0.5
    table[1, half:] = 2.0 ** -9                         # mixes x1 and x2 at small weight
    table[2, :half] = np.float32(1 - 2.0 ** -24)
    table[2, half:] = np.float32(2.0 ** -12)
    table[3, :half] = 2.0 ** -100                       # pushes results below 2^-126
    table[3, half:] = 2.0 ** -110
    specials = np.array([1.0, 1 + 2.0 ** -7, 1 + 3 * 2.0 ** -7, 3.3895313892515355e38,
                         -3.3895313892515355e38, 2.0 ** -126, -2.0 ** -120, 0.0, 1.5, -1.0,
                         2.0 ** 100, 3.0e38, 65504.0, 2.0 ** -20], np.float64)

    def make(shape):
        x = rng.standard_normal(shape) * 2.0 ** rng.integers(-30, 30, shape)
        x.reshape(-1)[: specials.size * 3] = np.tile(specials, 3)
        bits16 = oracle.float_to_bf16_bits(x.astype(np.float32))
        return torch.from_numpy(bits16.view(np.int16)).view(torch.bfloat16)

    q_cpu, k_cpu, v_cpu = make((T, hq, d)), make((T, hkv, d)), make((T, hkv, d))
    pos = (np.arange(T) % 4).astype(np.int32)
    pool = wl.pool.cuda()
    q = q_cpu.cuda()
    _say("rope rounding cases")
    msgl.rope_store_kv(pool, 0, q, k_cpu.cuda(), v_cpu.cuda(), _i32(ph.out_loc), _i32(pos),
                       torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    q_ref, pool_ref = oracle.rope_store_kv(bits(wl.pool), 0, bits(q_cpu), bits(k_cpu), bits(v_cpu),
                                           ph.out_loc, pos, table)
    assert np.array_equal(bits(q), q_ref), "rotated q differs"
    assert np.array_equal(bits(pool), pool_ref), "pool differs"
    # the crafted rows reach every case: infinities, subnormals and ties
    qf = oracle.bf16_bits_to_float(q_ref, np.float64)
    assert np.isinf(qf).any() and ((q_ref & 0x7F80) == 0).any() and (q_ref != 0).any()


def test_rope_store_then_decode_matches_oracle():
    # the fused store feeding decode: rotated queries against rotated keys
    hq, hkv, d, ps = 8, 2, 128, 16
    wl = build_case(451, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[500, 77, 1000], extend_lens=[1, 1, 1])
    ph = wl.phases[0]
    L = ph.seq_lens
    pos = (L - 1).astype(np.int32)
    table_np = oracle.rope_table(2048, d, 10000.0).astype(np.float32)
    pool = wl.pool.cuda()
    q = ph.q.cuda()
    msgl.rope_store_kv(pool, 0, q, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc), _i32(pos),
                       torch.from_numpy(table_np).cuda())
    out = msgl.paged_decode(pool, 0, q, torch.from_numpy(wl.page_table).cuda(), _i32(ph.table_idx),
                            _i32(L), int(L.max()))
    torch.cuda.synchronize()
    q_ref, pool_ref = oracle.rope_store_kv(bits(wl.pool), 0, bits(ph.q), bits(ph.k), bits(ph.v),
                                           ph.out_loc, pos, table_np)
    ref = oracle.paged_decode(pool_ref, 0, q_ref, wl.page_table, ph.table_idx, L)
    got = oracle.bf16_bits_to_float(bits(out), np.float64)
    diff = np.abs(got - ref)
    assert np.all(diff <= 1e-2 + 1e-2 * np.abs(ref))
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 5e-3


def test_checked_mode_rejects_bad_rope_metadata(monkeypatch):
    # MSGL_CHECK=1 copies out_loc and positions to the host first: two rows
    # into one slot, a slot past the pool and a position past the table are
    # refused before any launch, and leave q and the pool as they were
    monkeypatch.setenv("MSGL_CHECK", "1")
    hq, hkv, d, ps, max_pos = 8, 2, 64, 16, 512
    wl = build_case(431, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[0, 40], extend_lens=[20, 12])
    ph = wl.phases[0]
    pos = np.arange(ph.num_tokens, dtype=np.int32)
    table = torch.from_numpy(oracle.rope_table(max_pos, d, 10000.0).astype(np.float32)).cuda()
    pool = wl.pool.cuda()
    q, k, v = ph.q.cuda(), ph.k.cuda(), ph.v.cuda()
    pool0, q0 = pool.clone(), q.clone()
    dup = ph.out_loc.copy()
    dup[5] = dup[17]
    far = ph.out_loc.copy()
    far[3] = wl.num_slots
    late = pos.copy()
    late[7] = max_pos
    for loc, p in ((dup, pos), (far, pos), (ph.out_loc, late)):
        with pytest.raises(msgl.MsglError) as e:
            msgl.rope_store_kv(pool, 0, q, k, v, _i32(loc), _i32(p), table)
        assert e.value.status == 5
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.int16), pool0.view(torch.int16))
    assert torch.equal(q.view(torch.int16), q0.view(torch.int16))
    padded = ph.out_loc.copy()
    padded[[2, 9]] = -1  # padding rows may repeat: they write nothing
    msgl.rope_store_kv(pool, 0, q, k, v, _i32(padded), _i32(pos), table)
    torch.cuda.synchronize()
