"""msgl_paged_decode_noalloc (the allocation-free decode) against
msgl_paged_decode, through the C ABI, on two calls in a row -- the second
with a smaller batch and shorter sequences, so that it runs on whatever
the first left in the library's scratch -- and against the oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits, close_report, widen
from workloads import build_case

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _case(seed, lens, hq=32, hkv=8, ps=16):
    wl = build_case(seed, num_qo_heads=hq, num_kv_heads=hkv, head_dim=128, page_size=ps,
                    prefix_lens=[l - 1 for l in lens], extend_lens=[1] * len(lens), kind="decode")
    ph = wl.phases[0]
    pool = wl.pool.cuda()
    msgl.store_kv(pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    return wl, ph, pool


@pytest.mark.parametrize("lens_a,lens_b", [
    ([3000, 17, 4096, 900, 2500, 1], [700, 33]),           # 2nd call: fewer, shorter requests
    ([50000, 12000], [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]),      # long splits, then tiny rows
])
def test_noalloc_matches_workspace_decode(lens_a, lens_b):
    assert torch.cuda.is_available()
    msgl.load_library()
    for seed, lens in ((61, lens_a), (62, lens_b)):
        wl, ph, pool = _case(seed, lens)
        pt = torch.from_numpy(wl.page_table).cuda()
        q = ph.q.cuda()
        L = int(ph.seq_lens.max())
        print(f"[noalloc] seed {seed} batch {len(lens)} max_len {L}", file=sys.stderr, flush=True)
        ref_out = msgl.paged_decode(pool, 0, q, pt, _i32(ph.table_idx), _i32(ph.seq_lens), L)
        out = torch.full_like(q, 7.0)
        got = msgl.paged_decode_noalloc(pool, 0, q, pt, _i32(ph.table_idx), _i32(ph.seq_lens), L,
                                        out=out)
        torch.cuda.synchronize()
        # same kernels, same partition: bit-identical to the workspace call
        assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16))
        pool_bits = bits(pool)
        ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx,
                                  ph.seq_lens, blocked=True)
        ok, max_abs, _, rel_l2 = close_report(widen(bits(got)), ref)
        assert ok and rel_l2 <= 5e-3, (max_abs, rel_l2)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    msgl.load_library()
    wl, ph, pool = _case(63, [100, 200])
    pt = torch.from_numpy(wl.page_table).cuda()
    big = 4096  # requests: partials of 4096 + 2 x 512 pieces x 32 heads x 520 B > 64 MiB
    need = msgl.paged_decode_workspace_size(big, 32, 128, 2048, 16)
    assert need > msgl.paged_decode_noalloc_max_workspace()
    q = torch.zeros((big, 32, 128), dtype=torch.bfloat16, device="cuda")
    ti = torch.zeros(big, dtype=torch.int32, device="cuda")
    sl = torch.ones(big, dtype=torch.int32, device="cuda")
    with pytest.raises(msgl.MsglError) as e:
        msgl.paged_decode_noalloc(pool, 0, q, pt, ti, sl, 2048)
    assert e.value.status == 4  # MSGL_ERR_WORKSPACE
