"""Parity of the HIP path (through the C ABI) with the CPU oracle, on gfx950.

store_kv and the page-table gather must be bit-exact; attention outputs
(bf16 in, fp32 accumulate, bf16 out) must satisfy, per element,
|gpu - oracle| <= 1e-2 + 1e-2 * |oracle| (max-abs 1e-2 and max-rel 1e-2 in
the combined form), with relative L2 <= 5e-3 as a tighter diagnostic that a
wrong mask cannot hide under.

Every attention output is compared element by element with the oracle,
the full-size workloads included (there the oracle's blocked matrix form
computes every row; of the chunked 32k prefill, the first and the last
chunk in full and every eighth row of the others), in the same launch
configuration the benchmark times.  Every output buffer sits between guard
rows that must come back untouched.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_loc_amd as msgl
from tests._util import bits, close_report, widen
from workloads import CONFIG_BUILDERS, build_case

pytestmark = pytest.mark.gpu

ATOL = RTOL = 1e-2
REL_L2 = 5e-3


def _say(msg):
    print(f"[gpu-parity] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msgl.load_library()
    yield
    torch.cuda.synchronize()


class Dev:
    """Device copies of a workload's metadata and its current pool."""

    def __init__(self, wl):
        self.wl = wl
        self.pool = wl.pool.cuda() if not wl.pool.is_cuda else wl.pool.clone()
        self.pt = torch.from_numpy(wl.page_table).cuda()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


GUARD_ROWS = 3
GUARD_BITS = 0x5A5A  # a finite bf16 pattern no kernel writes by chance


class Guarded:
    """An output buffer of `rows` (heads, d) bf16 rows with GUARD_ROWS guard
    rows on each side; `out` is the middle (contiguous) part."""

    def __init__(self, rows, heads, d):
        self.buf = torch.full((rows + 2 * GUARD_ROWS, heads, d), GUARD_BITS, dtype=torch.int16,
                              device="cuda").view(torch.bfloat16)
        self.out = self.buf[GUARD_ROWS:GUARD_ROWS + rows]

    def check(self, what=""):
        b = bits(self.buf)
        g = np.concatenate([b[:GUARD_ROWS], b[b.shape[0] - GUARD_ROWS:]])
        assert np.all(g == GUARD_BITS), f"{what}: a kernel wrote outside its output rows"


def gpu_phase(dev, ph, check_store_against=None):
    wl = dev.wl
    k, v, q = ph.k.cuda(), ph.v.cuda(), ph.q.cuda()
    msgl.store_kv(dev.pool, wl.layer, k, v, _i32(ph.out_loc))
    ti = _i32(ph.table_idx)
    g = Guarded(q.shape[0], q.shape[1], q.shape[2])
    if ph.kind == "decode":
        out = msgl.paged_decode(dev.pool, wl.layer, q, dev.pt, ti, _i32(ph.seq_lens),
                                int(ph.seq_lens.max()), out=g.out)
    else:
        out = msgl.paged_extend(dev.pool, wl.layer, q, dev.pt, ti, _i32(ph.prefix_lens),
                                _i32(ph.extend_lens), _i32(ph.cu_extend_lens),
                                int(ph.extend_lens.max()), int(ph.seq_lens.max()), out=g.out)
    torch.cuda.synchronize()
    g.check(f"{ph.kind} B={ph.batch}")
    return out


def oracle_phase(pool_bits, wl, ph, only_tokens=None, blocked=False):
    """Oracle output of one phase (after its store_kv).  `blocked` selects
    the oracle's matrix form of the same definition (fast at full size)."""
    pool_bits = oracle.store_kv(pool_bits, wl.layer, bits(ph.k), bits(ph.v), ph.out_loc)
    if ph.kind == "decode":
        ref = oracle.paged_decode(pool_bits, wl.layer, bits(ph.q), wl.page_table, ph.table_idx,
                                  ph.seq_lens, only_tokens=only_tokens, blocked=blocked)
    else:
        attend = oracle.paged_attention_blocked if blocked else oracle.paged_attention
        ref = attend(pool_bits, wl.layer, bits(ph.q), wl.page_table, ph.table_idx,
                     ph.prefix_lens, ph.extend_lens, only_tokens=only_tokens)
    return pool_bits, ref


def assert_close(got_bf16, ref, rows=None, what=""):
    got = widen(bits(got_bf16), np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ok, max_abs, max_rel, rel_l2 = close_report(got, ref, ATOL, RTOL)
    _say(f"{what}: max_abs={max_abs:.3e} max_rel={max_rel:.3e} rel_l2={rel_l2:.3e}")
    assert ok, f"{what}: max_abs={max_abs} max_rel={max_rel}"
    assert rel_l2 <= REL_L2, f"{what}: rel_l2={rel_l2}"


def assert_returns_v(got_bits, v_bits, kind, what=""):
    """A row whose softmax has one key of weight 1 (a single key, a mirror
    probe) must return that key's V.  Decode forms P.V in bf16 and returns V
    bit for bit.  Extend forms P.V on the fp16 MFMA: V converts exactly
    wherever |V| >= 2^-14 (fp16's smallest normal), which must then come
    back bit for bit; below that, V is rounded on fp16's subnormal grid of
    2^-24, so the result must lie within half a step of V."""
    got_bits = np.asarray(got_bits)
    v_bits = np.asarray(v_bits)
    if kind == "decode":
        assert np.array_equal(got_bits, v_bits), f"{what}: output is not V exactly"
        return
    v = widen(v_bits, np.float64)
    got = widen(got_bits, np.float64)
    normal = np.abs(v) >= 2.0 ** -14
    assert np.array_equal(got_bits[normal], v_bits[normal]), f"{what}: output is not V exactly"
    assert np.all(np.abs(got[~normal] - v[~normal]) <= 2.0 ** -25), f"{what}: tiny V off grid"


def run_full(wl, what):
    dev = Dev(wl)
    pool_bits = bits(wl.pool)
    for i, ph in enumerate(wl.phases):
        _say(f"{what} phase {i} ({ph.kind}, B={ph.batch}, T={ph.num_tokens})")
        out = gpu_phase(dev, ph)
        pool_bits, ref = oracle_phase(pool_bits, wl, ph)
        assert np.array_equal(bits(dev.pool), pool_bits), f"{what}: pool differs after store_kv"
        assert_close(out, ref, what=f"{what} phase {i}")


# ------------------------------------------------------------------ store/gather


def test_store_kv_bit_exact_with_canaries():
    wl = build_case(101, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                    prefix_lens=[3, 40, 0, 17], extend_lens=[5, 1, 70, 33])
    ph = wl.phases[0]
    dev = Dev(wl)
    _say("store_kv canaries")
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    torch.cuda.synchronize()
    ref = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    assert np.array_equal(bits(dev.pool), ref)


def test_store_kv_strided_views_and_padding():
    # k and v as slices of a merged (T, Hq + 2 Hkv, d) projection; every
    # third row padded with out_loc = -1
    hq, hkv, d = 8, 2, 64
    wl = build_case(102, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=4,
                    prefix_lens=[0, 9], extend_lens=[30, 21])
    ph = wl.phases[0]
    T = ph.num_tokens
    qkv = torch.zeros((T, hq + 2 * hkv, d), dtype=torch.bfloat16)
    qkv[:, hq:hq + hkv] = ph.k
    qkv[:, hq + hkv:] = ph.v
    qkv = qkv.cuda()
    loc = ph.out_loc.copy()
    loc[::3] = -1
    dev = Dev(wl)
    _say("store_kv strided")
    msgl.store_kv(dev.pool, 0, qkv[:, hq:hq + hkv], qkv[:, hq + hkv:], _i32(loc))
    torch.cuda.synchronize()
    ref = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), loc)
    assert np.array_equal(bits(dev.pool), ref)


@pytest.mark.parametrize("hkv,d,pad", [(8, 128, 0), (4, 128, 4), (2, 64, 2)])
def test_store_kv_many_rows_ragged(hkv, d, pad):
    # 2051 rows: enough for the four-tokens-per-lane launch, and not a
    # multiple of four; every fifth row padded; the row pad (in elements)
    # forces 16-, 8- and 4-byte pieces
    wl = build_case(103 + pad, num_qo_heads=hkv, num_kv_heads=hkv, head_dim=d, page_size=16,
                    prefix_lens=[0, 5, 700], extend_lens=[1000, 1048, 3])
    ph = wl.phases[0]
    T = ph.num_tokens
    assert T == 2051

    def padded(x):
        buf = torch.zeros((T, hkv * d + pad), dtype=torch.bfloat16)
        buf[:, :hkv * d] = x.reshape(T, hkv * d)
        return buf.cuda().as_strided((T, hkv, d), (hkv * d + pad, d, 1))

    loc = ph.out_loc.copy()
    loc[::5] = -1
    dev = Dev(wl)
    _say(f"store_kv {T} rows, hkv={hkv} d={d} row pad {pad}")
    msgl.store_kv(dev.pool, 0, padded(ph.k), padded(ph.v), _i32(loc))
    torch.cuda.synchronize()
    ref = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), loc)
    assert np.array_equal(bits(dev.pool), ref)


@pytest.mark.parametrize("ps", [1, 2, 16, 64])
def test_gather_bit_exact(ps):
    wl = build_case(103 + ps, num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=ps,
                    prefix_lens=[100, 7], extend_lens=[1, 90])
    dev = Dev(wl)
    ph = wl.phases[0]
    for r in range(ph.batch):
        L = int(ph.seq_lens[r])
        row = int(ph.table_idx[r])
        _say(f"gather ps={ps} row={row} L={L}")
        k, v = msgl.debug_gather_kv(dev.pool, 0, dev.pt, row, L)
        torch.cuda.synchronize()
        kr, vr = oracle.gather_kv(bits(wl.pool), 0, wl.page_table, row, L)
        assert np.array_equal(bits(k), kr) and np.array_equal(bits(v), vr)


# --------------------------------------------------------------- the configs


def test_tiny_config_full():
    run_full(CONFIG_BUILDERS["tiny"](), "tiny")


def _full_size(wl, ph, what):
    """Run one phase at full size and compare every output element (and
    the stored rows, plus a sample of untouched pool rows)."""
    dev = Dev(wl)
    pool_bits = bits(wl.pool)
    out = gpu_phase(dev, ph)
    pool_after = oracle.store_kv(pool_bits, wl.layer, bits(ph.k), bits(ph.v), ph.out_loc)
    touched = np.unique(ph.out_loc[ph.out_loc >= 0])
    S = wl.num_slots
    gp = bits(dev.pool).reshape(2, S, -1)
    op = pool_after.reshape(2, S, -1)
    assert np.array_equal(gp[:, touched], op[:, touched]), f"{what}: stored rows differ"
    probe = np.random.default_rng(0).choice(S, 4096, replace=False)
    assert np.array_equal(gp[:, probe], op[:, probe]), f"{what}: untouched rows changed"
    del gp, op
    _, ref = oracle_phase(pool_bits, wl, ph, blocked=True)
    assert_close(out, ref, what=f"{what} (all {ph.num_tokens} query rows)")
    return dev, pool_after


def test_llama3_8b_decode_full_size():
    wl = CONFIG_BUILDERS["llama3_8b_decode"](device="cuda")
    _say("llama3_8b_decode full size")
    _full_size(wl, wl.phases[0], "llama3_8b_decode")


def test_qwen3_moe_decode_full_size():
    wl = CONFIG_BUILDERS["qwen3_moe_decode"](device="cuda")
    _say("qwen3_moe_decode full size")
    _full_size(wl, wl.phases[0], "qwen3_moe_decode")


def test_radix_shared_extend_full_size():
    wl = CONFIG_BUILDERS["radix_shared_extend"](device="cuda")
    _say("radix_shared_extend full size")
    _full_size(wl, wl.phases[0], "radix_shared_extend")


def test_chunked_prefill_full_size():
    # chunks 0 and 7 (4096 rows over 4096 and 32768 keys) in full; every
    # eighth row, plus the first and last two, of the others
    wl = CONFIG_BUILDERS["chunked_prefill"](device="cuda")
    dev = Dev(wl)
    pool_bits = bits(wl.pool)
    last = len(wl.phases) - 1
    for c, ph in enumerate(wl.phases):
        _say(f"chunked_prefill chunk {c}")
        out = gpu_phase(dev, ph)
        E = ph.num_tokens
        rows = None if c in (0, last) else sorted(set(range(0, E, 8)) | {1, E - 2, E - 1})
        pool_bits, ref = oracle_phase(pool_bits, wl, ph, only_tokens=rows, blocked=True)
        what = f"chunked_prefill chunk {c} ({'all' if rows is None else len(rows)} rows)"
        assert_close(out, ref, rows=rows, what=what)


@pytest.mark.parametrize("std", [2.0, 3.0])
def test_radix_shared_extend_large_logits(std):
    # the radix-shared geometry (32 q / 8 kv heads, d 128, ps 16, a shared
    # 2048-token prefix, 512 new tokens each) with q/k/v drawn at standard
    # deviation 2 and 3: logits of tens, where any rounding of the scaled
    # query or of the scores would show
    wl = build_case(920 + int(std), num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=[2048] * 4, extend_lens=[512] * 4, shared_prefix=True,
                    num_pages=4096, std=std, kind="extend", device="cuda")
    _say(f"radix-shared geometry extend, std {std}")
    _full_size(wl, wl.phases[0], f"extend std {std}")


@pytest.mark.parametrize("std", [2.0, 3.0])
def test_decode_large_logits(std):
    lens = [1, 300, 2048, 4071, 700]
    wl = build_case(930 + int(std), num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=[l - 1 for l in lens], extend_lens=[1] * len(lens), std=std,
                    kind="decode", device="cuda")
    _say(f"decode std {std}")
    _full_size(wl, wl.phases[0], f"decode std {std}")


def _one_hot_v_case(P, E, hq, hkv, d, ps, seed, kind):
    """A request of P cached + E new tokens whose V rows are one-hot(j mod d)
    in every kv head (K random), stored through store_kv; q = 0."""
    base = build_case(seed, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                      prefix_lens=[P], extend_lens=[E], kind=kind)
    L = P + E
    V = torch.zeros((L, hkv, d), dtype=torch.bfloat16)
    V[torch.arange(L), :, torch.arange(L) % d] = 1.0
    K = torch.randn((L, hkv, d), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    dev = Dev(base)
    slots = oracle.token_slots(base.page_table[base.phases[0].table_idx[0]], L, ps)
    msgl.store_kv(dev.pool, 0, K.cuda(), V.cuda(), _i32(slots))
    return base, dev


@pytest.mark.parametrize("P,E", [(2048, 512), (28672, 4096)])
def test_extend_uniform_weights_closed_form(P, E):
    # q = 0 gives equal weights: row i (position a = P + i) must return the
    # mean of V over keys 0..a, i.e. count(j <= a, j = c mod d) / (a + 1) on
    # channel c, in every head
    hq, hkv, d, ps = 32, 8, 128, 16
    base, dev = _one_hot_v_case(P, E, hq, hkv, d, ps, 940 + E, "extend")
    ph = base.phases[0]
    q = torch.zeros((E, hq, d), dtype=torch.bfloat16, device="cuda")
    g = Guarded(E, hq, d)
    _say(f"uniform weights extend P={P} E={E}")
    out = msgl.paged_extend(dev.pool, 0, q, dev.pt, _i32(ph.table_idx), _i32([P]), _i32([E]),
                            _i32([0, E]), E, P + E, out=g.out)
    torch.cuda.synchronize()
    g.check("uniform weights extend")
    a = P + np.arange(E, dtype=np.int64)
    c = np.arange(d, dtype=np.int64)
    counts = (a[:, None] - c[None, :]) // d + 1  # j = c, c + d, ... <= a
    expect = counts / (a[:, None] + 1.0)
    got = widen(bits(out), np.float64)
    err = np.abs(got - expect[:, None, :])
    _say(f"uniform weights: max abs {err.max():.3e}")
    assert np.all(err <= 2.0 ** -8 * np.abs(expect[:, None, :]) + 1e-6)


def test_decode_uniform_weights_closed_form():
    hq, hkv, d, ps = 32, 8, 128, 16
    lens = [1, 129, 2048, 4096, 32768]
    wl = build_case(945, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[l - 1 for l in lens], extend_lens=[1] * len(lens), kind="decode")
    ph = wl.phases[0]
    dev = Dev(wl)
    for r, L in enumerate(lens):
        V = torch.zeros((L, hkv, d), dtype=torch.bfloat16)
        V[torch.arange(L), :, torch.arange(L) % d] = 1.0
        slots = oracle.token_slots(wl.page_table[ph.table_idx[r]], L, ps)
        msgl.store_kv(dev.pool, 0, torch.zeros_like(V).cuda(), V.cuda(), _i32(slots))
    q = torch.zeros((len(lens), hq, d), dtype=torch.bfloat16, device="cuda")
    g = Guarded(len(lens), hq, d)
    _say("uniform weights decode")
    out = msgl.paged_decode(dev.pool, 0, q, dev.pt, _i32(ph.table_idx), _i32(lens), max(lens),
                            out=g.out)
    torch.cuda.synchronize()
    g.check("uniform weights decode")
    got = widen(bits(out), np.float64)
    for r, L in enumerate(lens):
        c = np.arange(d)
        expect = ((L - 1 - c) // d + 1).clip(min=0) / float(L)
        assert np.all(np.abs(got[r] - expect[None]) <= 2.0 ** -8 * expect[None] + 1e-6), L


@pytest.mark.parametrize("offset", [0, 3])
def test_boundary_probes_radix_geometry(offset):
    # P = 2048, E = 512, G = 4 (32 q / 8 kv heads): every fourth new token
    # (from `offset`) probes its own channel, so every row tile and every
    # diagonal key tile holds probes.  Leak: key a+1 (the first masked key)
    # carries logit 362 on the probe's channel -> a leaked mask returns
    # ~V[a+1] instead of the mean.  Mirror: key a (the last allowed) carries
    # it -> exactly V[a].  Rows with q = 0 see uniform weights.
    hq, hkv, d, ps = 32, 8, 128, 16
    P, E = 2048, 512
    L = P + E
    base = build_case(950 + offset, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                      prefix_lens=[P], extend_lens=[E], kind="extend")
    ph = base.phases[0]
    probes = list(range(offset, E, 4))
    assert len(probes) <= d
    q = torch.zeros((E, hq, d), dtype=torch.bfloat16)
    for n, i in enumerate(probes):
        q[i, :, n] = 64.0
    Vall = torch.randn((L, hkv, d), generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    slots = oracle.token_slots(base.page_table[ph.table_idx[0]], L, ps)
    for mode in ("leak", "mirror"):
        K = torch.zeros((L, hkv, d), dtype=torch.bfloat16)
        for n, i in enumerate(probes):
            a = P + i
            if mode == "leak" and a + 1 < L:
                K[a + 1, :, n] = 64.0
            if mode == "mirror":
                K[a, :, n] = 64.0
        dev = Dev(base)
        msgl.store_kv(dev.pool, 0, K.cuda(), Vall.cuda(), _i32(slots))
        g = Guarded(E, hq, d)
        _say(f"boundary probe {mode}, offset {offset}")
        out = msgl.paged_extend(dev.pool, 0, q.cuda(), dev.pt, _i32(ph.table_idx), _i32([P]),
                                _i32([E]), _i32([0, E]), E, L, out=g.out)
        torch.cuda.synchronize()
        g.check("boundary probe")
        pool_bits = bits(dev.pool)
        ref = oracle.paged_attention_blocked(pool_bits, 0, bits(q), base.page_table, ph.table_idx,
                                             [P], [E])
        assert_close(out, ref, what=f"boundary probe {mode} offset {offset}")
        if mode == "mirror":
            ob = bits(out)
            vb = bits(Vall)
            for i in probes:
                assert_returns_v(ob[i], np.repeat(vb[P + i], hq // hkv, 0), "extend",
                                 f"mirror row {i}")


# ------------------------------------------------------------------- sweeps


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("ps", [1, 2, 16])
def test_decode_sweep(d, G, ps):
    hkv = 2
    lens = [1, 2, 63, 64, 65, 255, 256, 257, 700, 1000]
    wl = build_case(200 + d + G + ps, num_qo_heads=hkv * G, num_kv_heads=hkv, head_dim=d,
                    page_size=ps, prefix_lens=[l - 1 for l in lens], extend_lens=[1] * len(lens),
                    kind="decode")
    run_full(wl, f"decode d={d} G={G} ps={ps}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("ps", [1, 2, 16, 64])
def test_extend_sweep(d, G, ps):
    hkv = 2
    P = [0, 5, 100, 17, 64, 0]
    E = [1, 65, 33, 130, 16, 200]
    wl = build_case(300 + d + G + ps, num_qo_heads=hkv * G, num_kv_heads=hkv, head_dim=d,
                    page_size=ps, prefix_lens=P, extend_lens=E, kind="extend")
    run_full(wl, f"extend d={d} G={G} ps={ps}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [2, 3, 16])
@pytest.mark.parametrize("ps", [3, 13])
def test_decode_sweep_uneven(d, G, ps):
    # page sizes that are not powers of two (the division path of the slot
    # formula) and group sizes the kernel pads up to 4 and 16 heads
    hkv = 1 if G == 16 else 2
    lens = [1, 5, 64, 255, 257, 600, 1029]
    wl = build_case(500 + d + G + ps, num_qo_heads=hkv * G, num_kv_heads=hkv, head_dim=d,
                    page_size=ps, prefix_lens=[l - 1 for l in lens], extend_lens=[1] * len(lens),
                    kind="decode")
    run_full(wl, f"decode d={d} G={G} ps={ps}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [2, 3, 16])
@pytest.mark.parametrize("ps", [3, 13])
def test_extend_sweep_uneven(d, G, ps):
    hkv = 1 if G == 16 else 2
    P = [0, 7, 100, 29]
    E = [3, 70, 45, 130]
    wl = build_case(600 + d + G + ps, num_qo_heads=hkv * G, num_kv_heads=hkv, head_dim=d,
                    page_size=ps, prefix_lens=P, extend_lens=E, kind="extend")
    run_full(wl, f"extend d={d} G={G} ps={ps}")


@pytest.mark.parametrize("kind", ["decode", "extend"])
def test_attention_with_strided_q(kind):
    # q as the leading slice of a merged (T, Hq + 2 Hkv, d) projection
    hq, hkv, d = 8, 2, 128
    if kind == "decode":
        wl = build_case(701, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=16,
                        prefix_lens=[300, 40, 999], extend_lens=[1, 1, 1], kind="decode")
    else:
        wl = build_case(702, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=16,
                        prefix_lens=[0, 130], extend_lens=[77, 260], kind="extend")
    ph = wl.phases[0]
    dev = Dev(wl)
    T = ph.q.shape[0]
    merged = torch.zeros((T, hq + 2 * hkv, d), dtype=torch.bfloat16)
    merged[:, :hq] = ph.q
    merged = merged.cuda()
    q = merged[:, :hq]
    assert q.stride(0) == (hq + 2 * hkv) * d
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    ti = _i32(ph.table_idx)
    _say(f"strided q {kind}")
    if kind == "decode":
        out = msgl.paged_decode(dev.pool, 0, q, dev.pt, ti, _i32(ph.seq_lens), int(ph.seq_lens.max()))
    else:
        out = msgl.paged_extend(dev.pool, 0, q, dev.pt, ti, _i32(ph.prefix_lens), _i32(ph.extend_lens),
                                _i32(ph.cu_extend_lens), int(ph.extend_lens.max()),
                                int(ph.seq_lens.max()))
    torch.cuda.synchronize()
    _, ref = oracle_phase(bits(wl.pool), wl, ph)
    assert_close(out, ref, what=f"strided q {kind}")


def test_extend_four_wave_workgroups(monkeypatch):
    # the 128-row workgroup variant selected by MSGL_EXTEND_WAVES=4
    monkeypatch.setenv("MSGL_EXTEND_WAVES", "4")
    wl = build_case(703, num_qo_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                    prefix_lens=[0, 300, 64], extend_lens=[200, 129, 1], kind="extend")
    run_full(wl, "extend 4-wave workgroups")


def test_extend_workgroup_size_choice(monkeypatch):
    # a small extend (fewer 256-row tiles than CUs) without key splits runs
    # 128-row workgroups unless MSGL_EXTEND_WAVES says otherwise; the rows
    # see the same key tiles in the same order either way, so both sizes
    # give the same bits, and both match the oracle
    wl = build_case(704, num_qo_heads=4, num_kv_heads=1, head_dim=128, page_size=16,
                    prefix_lens=[900, 0, 333], extend_lens=[300, 64, 17], kind="extend")
    ph = wl.phases[0]
    dev = Dev(wl)
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    q = ph.q.cuda()
    args = (dev.pool, 0, q, dev.pt, _i32(ph.table_idx), _i32(ph.prefix_lens), _i32(ph.extend_lens),
            _i32(ph.cu_extend_lens), int(ph.extend_lens.max()), int(ph.seq_lens.max()))
    outs = {}
    for wv in ("", "8", "4"):
        if wv:
            monkeypatch.setenv("MSGL_EXTEND_WAVES", wv)
        else:
            monkeypatch.delenv("MSGL_EXTEND_WAVES", raising=False)
        _say(f"extend workgroup size choice: MSGL_EXTEND_WAVES={wv or 'unset'}")
        outs[wv] = msgl.paged_extend(*args, split=False)
        torch.cuda.synchronize()
    _, ref = oracle_phase(bits(wl.pool), wl, ph, blocked=True)
    assert_close(outs[""], ref, what="extend, automatic workgroup size")
    assert torch.equal(outs[""].view(torch.int16), outs["4"].view(torch.int16))
    assert torch.equal(outs["8"].view(torch.int16), outs["4"].view(torch.int16))


@pytest.mark.parametrize("splits", ["", "2", "3", "8"])
@pytest.mark.parametrize("hq,hkv,d,ps,P,E", [
    (4, 1, 128, 16, [6000, 4096], [512, 300]),     # a tensor-parallel share
    (8, 2, 64, 3, [0, 700, 65], [400, 1, 190]),     # short rows: shares of the first tiles are empty
    (32, 8, 128, 16, [6000], [260]),               # one request in the full geometry
    (12, 3, 128, 1, [5000, 64], [90, 64]),          # page size 1, a long prefix
])
def test_extend_key_split(monkeypatch, splits, hq, hkv, d, ps, P, E):
    # calls too small to fill the device split each row tile's keys over
    # several workgroups (automatically when their rows are long, or
    # MSGL_EXTEND_SPLITS shares) and merge the shares: every element
    # against the oracle, the guard rows untouched, and a workspace one byte
    # short refused
    if splits:
        monkeypatch.setenv("MSGL_EXTEND_SPLITS", splits)
    else:
        monkeypatch.delenv("MSGL_EXTEND_SPLITS", raising=False)
    wl = build_case(720 + sum(E), num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=P, extend_lens=E, kind="extend", std=2.0)
    ph = wl.phases[0]
    dev = Dev(wl)
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    T = int(ph.extend_lens.sum())
    max_len = int(ph.seq_lens.max())
    need = msgl.paged_extend_workspace_size(dev.pool, T, max_len, hq)
    assert (need > 0) == (bool(splits) or max_len >= 1024), "the call should split its keys"
    g = Guarded(T, hq, d)
    args = (dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx), _i32(ph.prefix_lens),
            _i32(ph.extend_lens), _i32(ph.cu_extend_lens), int(ph.extend_lens.max()), max_len)
    _say(f"extend key split shares={splits or 'auto'} hq={hq} hkv={hkv} d={d} ps={ps} P={P} E={E}")
    msgl.paged_extend(*args, out=g.out, workspace=torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    g.check("extend key split")
    _, ref = oracle_phase(bits(wl.pool), wl, ph, blocked=True)
    assert_close(g.out, ref, what=f"extend key split {splits or 'auto'}")
    if need > 0:
        with pytest.raises(msgl.MsglError):
            msgl.paged_extend(*args, workspace=torch.zeros(need - 1, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("E", [1, 2, 7, 31, 32, 33, 63, 64, 65])
def test_extend_lengths(E):
    wl = build_case(400 + E, num_qo_heads=8, num_kv_heads=1, head_dim=128, page_size=16,
                    prefix_lens=[37, 0], extend_lens=[E, E], kind="extend")
    run_full(wl, f"extend E={E}")


def test_extend_shared_prefix_small():
    wl = build_case(411, num_qo_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                    prefix_lens=[128, 128, 128], extend_lens=[40, 129, 3], shared_prefix=True,
                    kind="extend")
    run_full(wl, "extend shared prefix")


def test_extend_with_empty_request():
    wl = build_case(412, num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                    prefix_lens=[20, 50, 3], extend_lens=[10, 0, 5], kind="extend")
    run_full(wl, "extend with an empty request")


# --------------------------------------------------------------- exact cases


def test_single_key_is_exact():
    for kind in ("decode", "extend"):
        wl = build_case(501, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                        prefix_lens=[0, 0], extend_lens=[1, 1], kind=kind)
        dev = Dev(wl)
        ph = wl.phases[0]
        _say(f"single key {kind}")
        out = gpu_phase(dev, ph)
        expect = np.repeat(bits(ph.v), 4, axis=1)  # q head h reads kv head h // 4
        assert_returns_v(bits(out), expect, kind, f"single key {kind}")


def test_boundary_probes_gpu():
    # query row i probes channel i; key a+1 (first masked) or key a (last
    # allowed) carries a huge logit on that channel
    d, hq, hkv, ps = 128, 4, 1, 16
    P, E = 45, 40
    L = P + E
    base = build_case(502, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                      prefix_lens=[P], extend_lens=[E], kind="extend")
    ph = base.phases[0]
    q = torch.zeros_like(ph.q)
    for i in range(E):
        q[i, :, i] = 64.0
    for mode in ("leak", "mirror"):
        K = torch.zeros((L, hkv, d), dtype=torch.bfloat16)
        for i in range(E):
            a = P + i
            if mode == "leak" and a + 1 < L:
                K[a + 1, :, i] = 64.0
            if mode == "mirror":
                K[a, :, i] = 64.0
        # write all L rows (prefix and new) through store_kv
        pool = base.pool.clone()
        slots = oracle.token_slots(base.page_table[ph.table_idx[0]], L, ps)
        Vall = torch.randn((L, hkv, d), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
        dev = Dev(base)
        msgl.store_kv(dev.pool, 0, K.cuda(), Vall.cuda(), _i32(slots))
        _say(f"boundary probe {mode}")
        out = msgl.paged_extend(dev.pool, 0, q.cuda(), dev.pt, _i32(ph.table_idx), _i32([P]),
                                _i32([E]), _i32([0, E]), E, L)
        torch.cuda.synchronize()
        got = widen(bits(out), np.float64)
        Vw = widen(bits(Vall), np.float64)
        for i in range(E):
            a = P + i
            if mode == "leak":
                expect = Vw[: a + 1, 0].mean(axis=0)
                assert np.abs(got[i] - expect[None]).max() <= 2e-2, f"mask leak at row {i}"
            else:
                assert_returns_v(bits(out)[i], np.repeat(bits(Vall)[a:a + 1, 0], hq, 0), "extend",
                                 f"mirror row {i}")


def test_decode_matches_extend_of_one():
    wl = build_case(503, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=[99, 700, 2047, 1], extend_lens=[1, 1, 1, 1], kind="decode")
    ph = wl.phases[0]
    dev = Dev(wl)
    _say("decode vs extend(E=1)")
    dec = gpu_phase(dev, ph)
    ext = msgl.paged_extend(dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx),
                            _i32(ph.prefix_lens), _i32(ph.extend_lens), _i32(ph.cu_extend_lens),
                            1, int(ph.seq_lens.max()))
    torch.cuda.synchronize()
    ok, max_abs, _, rel = close_report(widen(bits(dec)), widen(bits(ext)))
    assert ok and rel <= REL_L2, (max_abs, rel)


def test_decode_padding_rows_are_zero():
    wl = build_case(504, num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                    prefix_lens=[30, 400, 5], extend_lens=[1, 1, 1], kind="decode")
    ph = wl.phases[0]
    dev = Dev(wl)
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    L = ph.seq_lens.copy()
    L[1] = 0
    _say("decode padding row")
    out = msgl.paged_decode(dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx), _i32(L), 401)
    torch.cuda.synchronize()
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx, L)
    assert np.all(bits(out)[1] == 0)
    assert_close(out, ref, rows=[0, 2], what="decode with a padding row")


def test_decode_workspace_reuse():
    # a workspace sized for the largest call serves smaller ones
    wl = build_case(505, num_qo_heads=16, num_kv_heads=2, head_dim=128, page_size=16,
                    prefix_lens=[1500, 37, 900], extend_lens=[1, 1, 1], kind="decode")
    ph = wl.phases[0]
    dev = Dev(wl)
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx, ph.seq_lens)
    need = msgl.paged_decode_workspace_size(64, 16, 128, 8192, 16)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        _say(f"decode with an oversized workspace, call {rep}")
        out = msgl.paged_decode(dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx),
                                _i32(ph.seq_lens), int(ph.seq_lens.max()), workspace=ws)
        torch.cuda.synchronize()
        assert_close(out, ref, what=f"decode, reused workspace {rep}")


@pytest.mark.parametrize("lens,hkv,d,ps", [([17] * 100, 8, 128, 16), ([65] * 100, 8, 128, 16),
                                           ([1] * 300 + [40], 4, 128, 1), ([33] * 70, 1, 64, 5)])
def test_decode_exact_workspace_is_not_overrun(lens, hkv, d, ps):
    # short requests padded to whole tiles split into more ranges than
    # batch * max_seq_len / 16: the workspace of exactly the size the
    # library asks for must hold every piece, and the bytes after it stay
    # untouched
    hq = 4 * hkv
    wl = build_case(507, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    prefix_lens=[L - 1 for L in lens], extend_lens=[1] * len(lens), kind="decode")
    ph = wl.phases[0]
    dev = Dev(wl)
    msgl.store_kv(dev.pool, 0, ph.k.cuda(), ph.v.cuda(), _i32(ph.out_loc))
    max_len = int(ph.seq_lens.max())
    need = msgl.paged_decode_workspace_size(len(lens), hq, d, max_len, ps)
    buf = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    _say(f"decode exact workspace B={len(lens)} L={max_len} hkv={hkv} d={d} ps={ps}")
    out = msgl.paged_decode(dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx),
                            _i32(ph.seq_lens), max_len, workspace=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "decode wrote past its workspace"
    pool_bits = oracle.store_kv(bits(wl.pool), 0, bits(ph.k), bits(ph.v), ph.out_loc)
    ref = oracle.paged_decode(pool_bits, 0, bits(ph.q), wl.page_table, ph.table_idx, ph.seq_lens)
    assert_close(out, ref, what="decode, exact workspace")


# -------------------------------------------------------------- checked mode


def test_checked_mode_rejects_bad_device_metadata(monkeypatch):
    monkeypatch.setenv("MSGL_CHECK", "1")
    wl = build_case(506, num_qo_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
                    prefix_lens=[10, 20], extend_lens=[1, 1], kind="decode")
    ph = wl.phases[0]
    dev = Dev(wl)
    k, v = ph.k.cuda(), ph.v.cuda()
    dup = ph.out_loc.copy()
    dup[1] = dup[0]
    with pytest.raises(msgl.MsglError) as e:
        msgl.store_kv(dev.pool, 0, k, v, _i32(dup))
    assert e.value.status == 5
    far = ph.out_loc.copy()
    far[0] = wl.num_slots
    with pytest.raises(msgl.MsglError):
        msgl.store_kv(dev.pool, 0, k, v, _i32(far))
    bad_pt = wl.page_table.copy()
    bad_pt[ph.table_idx[0], 0] = wl.num_pages + 5
    with pytest.raises(msgl.MsglError):
        msgl.paged_decode(dev.pool, 0, ph.q.cuda(), torch.from_numpy(bad_pt).cuda(),
                          _i32(ph.table_idx), _i32(ph.seq_lens), 32)
    with pytest.raises(msgl.MsglError):  # seq_len above max_seq_len
        msgl.paged_decode(dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx), _i32(ph.seq_lens), 16)
    # the valid call still runs in checked mode
    msgl.store_kv(dev.pool, 0, k, v, _i32(ph.out_loc))
    out = msgl.paged_decode(dev.pool, 0, ph.q.cuda(), dev.pt, _i32(ph.table_idx),
                            _i32(ph.seq_lens), 32)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
