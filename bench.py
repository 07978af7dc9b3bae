"""Benchmark of the paged-KV attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  * Llama-3-8B attention geometry decode (32 q / 8 kv heads, head_dim 128,
    page_size 16, 64 requests with lengths uniform in [512, 4096], pages
    scattered in a pool of 32768): store_kv of the 64 new rows, then
    split-KV decode and its merge;
  * radix-shared prefix extend (same geometry, 16 requests sharing a
    2048-token prefix, 512 new tokens each): store_kv of 8192 rows, then
    causal extend.

Reported: decode KV throughput in GB/s (the `value`, algorithmic bytes:
K/V of every attended token, q, out, page ids and lengths; split partials
not counted) and extend TFLOP/s (4*d FLOP per unmasked (query, key, head)),
each against the MI355X peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s),
with per-kernel times from HIP events on the launch stream, and the CPU
oracle timed on a bounded sample of the same workloads.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per launch from two rocprofv3 --pmc runs of this benchmark
# (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads
# for a plain 512 MiB device copy (x2 for FETCH_SIZE, x1 for WRITE_SIZE),
# taken on the kernel sources with these SHA-256 digests.  When a source has
# changed since, the figure no longer describes the kernel and is reported
# as null.
MEASURED_TRAFFIC = {
    "decode": {  # decode_kernel + decode_merge_kernel
        "sources": {"decode.hip": "fbd27d913855bfce9fe4af51697e9f6a3fc51f177b3b110d3193ce6d7d88fe9c",
                    "decode_block.h": "b9d509ffd8512a1f32625e7aee71e53764368633616a36ed238175582dce0bc8",
                    "common.h": "271cfffca66ec4cea4a54312e57eda0bf94958123a470de6dfa5800153bb9f74"},
        "bytes": 658159887,
        "profile": "profiles/decode_llama3-8b-geometry_B64.md",
    },
    "extend": {
        "sources": {"extend.hip": "af078065bcafd978831e86ea92715ea5ad8165c9cbcbed7127efaaf562e9f37a",
                    "extend_block.h": "411eb8f5d26cc4d860f0d1a87aed9b4ffc28f48e610ee565b7d335b926f40fb3",
                    "common.h": "271cfffca66ec4cea4a54312e57eda0bf94958123a470de6dfa5800153bb9f74"},
        "bytes": 240399440,
        "profile": "profiles/extend_radix-shared_16x2560.md",
    },
}


def measured_traffic(key):
    ent = MEASURED_TRAFFIC.get(key)
    if not ent or not ent["sources"] or ent["bytes"] is None:
        return None
    for rel, digest in ent["sources"].items():
        path = os.path.join(ROOT, "paged_kv_attention_loc_amd", "csrc", rel)
        with open(path, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return ent["bytes"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def decode_bytes(wl, ph):
    L = ph.seq_lens.astype(np.int64)
    B = ph.batch
    d, hkv, hq, ps = wl.head_dim, wl.num_kv_heads, wl.num_qo_heads, wl.page_size
    return int((L * 2 * hkv * d * 2).sum() + 2 * B * hq * d * 2 + (-(-L // ps)).sum() * 4 + 8 * B)


def store_bytes(wl, T):
    return int(2 * (2 * T * wl.num_kv_heads * wl.head_dim * 2) + 4 * T)


def extend_flops(wl, ph, rows=None):
    d, hq = wl.head_dim, wl.num_qo_heads
    tot = 0
    cu = ph.cu_extend_lens
    for r in range(ph.batch):
        P = int(ph.prefix_lens[r])
        for i in range(int(ph.extend_lens[r])):
            if rows is None or (int(cu[r]) + i) in rows:
                tot += (P + i + 1) * hq * 4 * d
    return tot


class Prepared:
    """Device-resident inputs of one phase."""

    def __init__(self, wl, ph, dev):
        self.wl, self.ph = wl, ph
        self.pool = wl.pool
        self.pt = torch.from_numpy(wl.page_table).to(dev)
        self.k, self.v, self.q = ph.k.to(dev), ph.v.to(dev), ph.q.to(dev)
        self.loc = i32(ph.out_loc, dev)
        self.ti = i32(ph.table_idx, dev)
        self.sl = i32(ph.seq_lens, dev)
        self.pl = i32(ph.prefix_lens, dev)
        self.el = i32(ph.extend_lens, dev)
        self.cu = i32(ph.cu_extend_lens, dev)
        self.max_len = int(ph.seq_lens.max())
        self.max_ext = int(ph.extend_lens.max())
        self.out = torch.empty_like(self.q)
        import paged_kv_attention_loc_amd as msgl
        need = msgl.paged_decode_workspace_size(ph.batch, wl.num_qo_heads, wl.head_dim,
                                                self.max_len, wl.page_size)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        # an extend too small to fill the device splits its keys (its own
        # workspace); the full-geometry workloads need none
        need = msgl.paged_extend_workspace_size(wl.pool, ph.num_tokens, self.max_len, wl.num_qo_heads)
        self.ws_ext = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)


def run_store(msgl, p):
    msgl.store_kv(p.pool, p.wl.layer, p.k, p.v, p.loc)


def run_decode(msgl, p):
    msgl.paged_decode(p.pool, p.wl.layer, p.q, p.pt, p.ti, p.sl, p.max_len, out=p.out,
                      workspace=p.ws)


def run_extend(msgl, p):
    msgl.paged_extend(p.pool, p.wl.layer, p.q, p.pt, p.ti, p.pl, p.el, p.cu, p.max_ext, p.max_len,
                      out=p.out, workspace=p.ws_ext)


def cpu_baseline(wl_dec, ph_dec, wl_ext, ph_ext, budget_s):
    """The oracle, as it stands, on bounded samples of the same workloads."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    def bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    cores = len(os.sched_getaffinity(0))
    log(f"cpu baseline: copying pools to host ({cores} cores)")
    pool_d = oracle.store_kv(bits(wl_dec.pool), 0, bits(ph_dec.k), bits(ph_dec.v), ph_dec.out_loc)
    q_d = bits(ph_dec.q)
    with threadpool_limits(limits=cores):
        blas = [i.get("num_threads") for i in threadpool_info()]
        # decode: requests in order, passing over the batch again until half
        # the budget is spent
        t0 = time.perf_counter()
        done = []
        while time.perf_counter() - t0 <= budget_s / 2:
            for r in range(ph_dec.batch):
                sel = np.array([r])
                oracle.paged_decode(pool_d, 0, q_d[sel], wl_dec.page_table, ph_dec.table_idx[sel],
                                    ph_dec.seq_lens[sel])
                done.append(r)
                if time.perf_counter() - t0 > budget_s / 2:
                    break
        t_dec = time.perf_counter() - t0
        passes = len(done) / ph_dec.batch
        L = ph_dec.seq_lens[done].astype(np.int64)
        dec_b = int((L * 2 * wl_dec.num_kv_heads * wl_dec.head_dim * 2).sum()
                    + 2 * len(done) * wl_dec.num_qo_heads * wl_dec.head_dim * 2
                    + (-(-L // wl_dec.page_size)).sum() * 4 + 8 * len(done))
        del pool_d
        pool_e = oracle.store_kv(bits(wl_ext.pool), 0, bits(ph_ext.k), bits(ph_ext.v), ph_ext.out_loc)
        q_e = bits(ph_ext.q)
        rng = np.random.default_rng(0)
        order = rng.permutation(ph_ext.num_tokens)
        rows, t_ext, n = [], 0.0, 16
        while t_ext < budget_s / 2 and len(rows) < ph_ext.num_tokens:
            batch = [int(x) for x in order[len(rows): len(rows) + n]]
            t1 = time.perf_counter()
            oracle.paged_attention(pool_e, 0, q_e, wl_ext.page_table, ph_ext.table_idx,
                                   ph_ext.prefix_lens, ph_ext.extend_lens, only_tokens=batch)
            t_ext += time.perf_counter() - t1
            rows += batch
            n *= 2
        ext_f = extend_flops(wl_ext, ph_ext, set(rows))
    return {
        "value": round(dec_b / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "blas_threads": blas,
        "kind": "oracle",
        "sample": (f"decode: {passes:.2f} passes over the {ph_dec.batch} requests of the Llama-3-8B "
                   f"decode batch ({int(L.sum())} KV tokens, {t_dec:.1f} s); extend: {len(rows)} of "
                   f"{ph_ext.num_tokens} query rows of the radix-shared extend ({t_ext:.1f} s)"),
        "extend_value": round(ext_f / t_ext / 1e9, 4),
        "extend_unit": "GFLOP/s",
    }


def rope_store_stats(msgl, p, dev, iters=20):
    """The fused rotary embedding + store_kv over one extend phase's new
    rows (positions prefix + i), as HBM throughput: algorithmic bytes are q
    read and written, k and v read, K and V written, the table rows read
    (one per token), out_loc and positions."""
    wl, ph = p.wl, p.ph
    pos = np.concatenate([np.arange(int(ph.prefix_lens[r]), int(ph.prefix_lens[r] + ph.extend_lens[r]))
                          for r in range(ph.batch)]).astype(np.int32)
    table = msgl.rope_cos_sin_table(int(pos.max()) + 1, wl.head_dim, 10000.0, device=dev)
    posd = i32(pos, dev)
    q = p.q.clone()
    T, hq, d, hkv = q.shape[0], wl.num_qo_heads, wl.head_dim, wl.num_kv_heads
    nbytes = T * (2 * hq * d * 2 + 2 * 2 * hkv * d * 2 + d * 4 + 8)
    us = back_to_back_us(lambda: msgl.rope_store_kv(p.pool, wl.layer, q, p.k, p.v, p.loc, posd, table),
                         iters)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"rows": T, "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(us, 3),
            "GB/s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "timing": "launches back to back in a torch graph, one replay between two events"}


def back_to_back_us(fn, iters):
    """GPU time per launch of `iters` launches captured back to back in one
    torch graph, from events around a replay: for short kernels, an event
    pair around each eager launch would add the host's launch latency, and
    eager launches back to back would measure the host's launch rate."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / iters)
    del g
    return float(np.median(ts))


def store_chunk_stats(msgl, dev, iters=50):
    """store_kv of one 4096-row chunk (the chunked-prefill workload's chunk:
    32 q / 8 kv heads, d 128, page_size 16), back-to-back launches."""
    from workloads import build_case
    wl = build_case(3, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=[0], extend_lens=[4096], device=dev)
    ph = wl.phases[0]
    k, v, loc = ph.k.to(dev), ph.v.to(dev), i32(ph.out_loc, dev)
    nbytes = 4096 * 2 * 2 * 8 * 128 * 2 + 4096 * 4
    us = back_to_back_us(lambda: msgl.store_kv(wl.pool, 0, k, v, loc), iters)
    gbs = nbytes / (us * 1e-6) / 1e9
    del wl
    return {"rows": 4096, "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(us, 3),
            "GB/s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "timing": "launches back to back in a torch graph, one replay between two events"}


def tp_share_stats(msgl, dev, iters=10):
    """One GPU's share of Llama-3-8B under 8-way tensor parallelism (4 q /
    1 kv head per GPU; the lengths, pages and value recipe of the
    full-geometry workloads): the decode batch, the radix-shared extend and
    the chunked 32k prefill, whose extend calls split their keys.  GPU time
    per call: `iters` calls captured back to back in a torch graph.  Not a
    roofline point: at this share the calls are too small to fill the
    device."""
    from workloads import config_chunked_prefill, config_llama3_8b_decode, config_radix_shared_extend
    res = {"workload": "Llama-3-8B attention at tensor parallelism 8: 4q/1kv d128 ps16 per GPU",
           "timing": "calls back to back in a torch graph, one replay between two events"}
    wl = config_llama3_8b_decode(device=dev, num_qo_heads=4, num_kv_heads=1)
    p = Prepared(wl, wl.phases[0], dev)
    run_store(msgl, p)
    nb = decode_bytes(wl, p.ph)
    us = back_to_back_us(lambda: run_decode(msgl, p), iters)
    res["decode_B64"] = {"algorithmic_bytes": nb, "us": round(us, 2), "GB/s": round(nb / us / 1e3, 1),
                         "frac_of_hbm_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}
    del p, wl
    wl = config_radix_shared_extend(device=dev, num_qo_heads=4, num_kv_heads=1)
    p = Prepared(wl, wl.phases[0], dev)
    run_store(msgl, p)
    fl = extend_flops(wl, p.ph)
    us = back_to_back_us(lambda: run_extend(msgl, p), iters)
    res["radix_shared_extend"] = {"algorithmic_flops": fl, "us": round(us, 2),
                                  "TFLOP/s": round(fl / us / 1e6, 1),
                                  "frac_of_mfma_peak": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del p, wl
    wl = config_chunked_prefill(device=dev, num_qo_heads=4, num_kv_heads=1)
    preps = [Prepared(wl, ph, dev) for ph in wl.phases]
    for p in preps:
        run_store(msgl, p)
    torch.cuda.synchronize()
    chunk_us = [back_to_back_us(lambda p=p: run_extend(msgl, p), max(2, iters // 4)) for p in preps]
    fl = sum(extend_flops(wl, p.ph) for p in preps)
    tot = sum(chunk_us)
    res["chunked_prefill"] = {"algorithmic_flops": fl, "us_per_chunk": [round(x, 1) for x in chunk_us],
                              "us": round(tot, 1), "TFLOP/s": round(fl / tot / 1e6, 1),
                              "frac_of_mfma_peak": round(fl / tot / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "key_split": [msgl.paged_extend_workspace_size(wl.pool, p.ph.num_tokens,
                                                                             p.max_len, 4) > 0
                                            for p in preps]}
    del preps, wl
    torch.cuda.empty_cache()
    return res


def alloc_stats(msgl, p, dev, iters=20):
    """msgl_alloc_pages for one phase's new tokens (a copy of its page table,
    the pool's unused pages as the free list).  GPU time per launch: `iters`
    launches captured back to back in a torch graph (each takes the next
    pages of the list), the free count reset before each timed replay;
    beside it, one eager launch between two events, which adds the host's
    launch latency."""
    wl, ph = p.wl, p.ph
    pt = p.pt.clone()
    used = np.unique(wl.page_table[wl.page_table >= 0])
    free = np.setdiff1d(np.arange(wl.num_pages, dtype=np.int32), used).astype(np.int32)
    d_free = i32(free, dev)
    d_nfree = torch.zeros(1, dtype=torch.int32, device=dev)
    d_status = torch.zeros(1, dtype=torch.int32, device=dev)
    out_loc = torch.empty(ph.num_tokens, dtype=torch.int32, device=dev)

    def launch():
        msgl.alloc_pages(d_free, d_nfree, pt, p.ti, p.pl, p.el, wl.page_size, out_loc, d_status)

    eager = []
    for i in range(13):
        d_nfree.fill_(len(free))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        if i >= 3:
            eager.append(a.elapsed_time(b) * 1e3)
    assert int(d_status.item()) == 0
    d_nfree.fill_(len(free))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            launch()
    ts = []
    for _ in range(6):
        d_nfree.fill_(len(free))
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        assert int(d_status.item()) == 0, "the free list ran out inside the timed launches"
        ts.append(a.elapsed_time(b) * 1e3 / iters)
    del g
    return {"requests": ph.batch, "new_tokens": ph.num_tokens,
            "avg_launch_us": round(float(np.median(ts[1:])), 2),
            "eager_event_us": round(float(np.mean(eager)), 2),
            "timing": "launches back to back in a torch graph, one replay between two events"}


def mixed_stats(msgl, dev, iters=10):
    """Mixed batches -- the 64 decode rows of the Llama-3-8B geometry batch
    (lengths uniform in [512, 4096], seed 2) with chunked-prefill pieces of
    512 new tokens on 2048-token prefixes: one piece (a serving step with a
    prefill chunk in flight: its tiles leave most CUs to the decode rows)
    and four (their tiles alone fill every CU).  Each as one paged_mixed
    call (one attention launch), as a decode call plus an extend call over
    the same rows (the extend with its keys split where it takes them, and
    unsplit), and as a paged_mixed call made of those same launches
    (MSGL_MIXED_SPLIT=1)."""
    res = {}
    for name, n_chunks in (("one_chunk", 1), ("four_chunks", 4)):
        res[name] = _mixed_case(msgl, dev, n_chunks, iters)
    return res


def _mixed_case(msgl, dev, n_chunks, iters):
    from workloads import build_case
    rng = np.random.default_rng(2)
    L = rng.integers(512, 4096, 64, endpoint=True)
    P = [int(x) - 1 for x in L] + [2048] * n_chunks
    E = [1] * 64 + [512] * n_chunks
    wl = build_case(12, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=P, extend_lens=E, device=dev)
    ph = wl.phases[0]
    p = Prepared(wl, ph, dev)
    run_store(msgl, p)
    dec = np.arange(64)
    q_dec = p.q[torch.from_numpy(ph.cu_extend_lens[dec].astype(np.int64)).to(dev)].contiguous()
    sl_dec = i32(np.asarray(P)[dec] + 1, dev)
    ti_dec = i32(ph.table_idx[dec], dev)
    ext = np.arange(64, 64 + n_chunks)
    first = int(ph.cu_extend_lens[64])
    q_ext = p.q[first:].contiguous()
    cu_ext = i32(ph.cu_extend_lens[64:] - first, dev)
    ti_ext, pl_ext = i32(ph.table_idx[ext], dev), i32(ph.prefix_lens[ext], dev)
    el_ext = i32(ph.extend_lens[ext], dev)
    out = torch.empty_like(p.q)
    out_dec, out_ext = torch.empty_like(q_dec), torch.empty_like(q_ext)
    ws_dec = torch.zeros(max(msgl.paged_decode_workspace_size(64, 32, 128, p.max_len, 16), 256),
                         dtype=torch.uint8, device=dev)
    ws_ext = torch.empty(max(msgl.paged_extend_workspace_size(p.pool, 512 * n_chunks, p.max_len, 32),
                             256), dtype=torch.uint8, device=dev)

    def mixed():
        msgl.paged_mixed(p.pool, wl.layer, p.q, p.pt, p.ti, p.pl, p.el, p.cu, p.max_ext, p.max_len,
                         out=out, workspace=p.ws)

    def separate(split=True):
        msgl.paged_decode(p.pool, wl.layer, q_dec, p.pt, ti_dec, sl_dec, p.max_len, out=out_dec,
                          workspace=ws_dec)
        msgl.paged_extend(p.pool, wl.layer, q_ext, p.pt, ti_ext, pl_ext, el_ext, cu_ext, 512,
                          p.max_len, out=out_ext, workspace=ws_ext, split=split)

    def mixed_split():
        os.environ["MSGL_MIXED_SPLIT"] = "1"
        try:
            mixed()
        finally:
            del os.environ["MSGL_MIXED_SPLIT"]

    res = {"decode_rows": 64, "extend_rows": n_chunks, "extend_tokens": 512 * n_chunks}
    for name, fn in (("mixed_call_us", mixed), ("separate_calls_us", separate),
                     ("separate_calls_unsplit_us", lambda: separate(False)),
                     ("mixed_split_launches_us", mixed_split)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        res[name] = round(float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3, 1)
    del p, wl
    return res


def other_workloads(msgl, dev, ext_iters=3, dec_iters=20, only=None):
    """The two remaining workloads, each as store_kv then attention, timed
    with HIP events on the launch stream (warm caches):
      * chunked prefill: one 32768-token request as 8 extend chunks of 4096
        over the growing prefix (32 q / 8 kv heads, d 128, ps 16, std 0.5);
      * Qwen3-30B-A3B attention geometry decode: 32 q / 4 kv heads, d 128,
        page_size 1, 256 requests with lognormal lengths (sum 824055).
    `only` names one of them to run alone (for profiles).
    """
    from workloads import config_chunked_prefill, config_qwen3_moe_decode

    def ev():
        return torch.cuda.Event(enable_timing=True)

    res = {}
    if only not in (None, "chunked_prefill"):
        return res | qwen_decode_stats(msgl, dev, dec_iters)
    wl = config_chunked_prefill(device=dev)
    preps = [Prepared(wl, ph, dev) for ph in wl.phases]
    for p in preps:  # the pool holds every chunk's rows before timing
        run_store(msgl, p)
        run_extend(msgl, p)
    torch.cuda.synchronize()
    st_ms = np.zeros((ext_iters, len(preps)))
    ex_ms = np.zeros((ext_iters, len(preps)))
    for it in range(ext_iters):
        marks = []
        for p in preps:
            e = [ev(), ev(), ev()]
            e[0].record()
            run_store(msgl, p)
            e[1].record()
            run_extend(msgl, p)
            e[2].record()
            marks.append(e)
        torch.cuda.synchronize()
        for c, e in enumerate(marks):
            st_ms[it, c] = e[0].elapsed_time(e[1])
            ex_ms[it, c] = e[1].elapsed_time(e[2])
    fl = [extend_flops(wl, p.ph) for p in preps]
    chunk_ms = np.median(ex_ms, axis=0)
    tot_ms = float(chunk_ms.sum())
    tf = sum(fl) / (tot_ms * 1e-3) / 1e12
    res["chunked_prefill"] = {
        "workload": "1 request of 32768 tokens as 8 extend chunks of 4096; 32q/8kv d128 ps16, std 0.5",
        "algorithmic_flops": int(sum(fl)),
        "extend_us_per_chunk": [round(x * 1e3, 1) for x in chunk_ms],
        "TFLOP/s_per_chunk": [round(f / (m * 1e-3) / 1e12, 1) for f, m in zip(fl, chunk_ms)],
        "extend_total_us": round(tot_ms * 1e3, 1),
        "TFLOP/s": round(tf, 2),
        "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "store_kv_avg_us": round(float(st_ms.mean()) * 1e3, 2),
        "store_kv_GBs": round(store_bytes(wl, preps[0].ph.num_tokens) / (float(st_ms.mean()) * 1e-3) / 1e9, 1),
    }
    del preps, wl
    torch.cuda.empty_cache()
    if only == "chunked_prefill":
        return res
    return res | qwen_decode_stats(msgl, dev, dec_iters)


def qwen_decode_stats(msgl, dev, dec_iters):
    from workloads import config_qwen3_moe_decode

    def ev():
        return torch.cuda.Event(enable_timing=True)

    res = {}
    wl = config_qwen3_moe_decode(device=dev)
    p = Prepared(wl, wl.phases[0], dev)
    for _ in range(3):
        run_store(msgl, p)
        run_decode(msgl, p)
    torch.cuda.synchronize()
    marks = []
    for _ in range(dec_iters):
        e = [ev(), ev(), ev()]
        e[0].record()
        run_store(msgl, p)
        e[1].record()
        run_decode(msgl, p)
        e[2].record()
        marks.append(e)
    torch.cuda.synchronize()
    st = np.array([e[0].elapsed_time(e[1]) for e in marks])
    dm = np.array([e[1].elapsed_time(e[2]) for e in marks])
    db = decode_bytes(wl, p.ph)
    gbs = db / (float(dm.mean()) * 1e-3) / 1e9
    res["qwen3_moe_decode"] = {
        "workload": "32q/4kv d128 ps1, 256 requests, lognormal lengths (sum 824055), slots scattered",
        "algorithmic_bytes": db,
        "decode_avg_us": round(float(dm.mean()) * 1e3, 1),
        "decode_median_us": round(float(np.median(dm)) * 1e3, 1),
        "GB/s": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "store_kv_avg_us": round(float(st.mean()) * 1e3, 2),
    }
    del p, wl
    torch.cuda.empty_cache()
    return res


def measured_ceilings(dev, iters=10):
    """What this GPU sustains, measured in this run beside the spec peaks:
    a 512 MiB device copy (bytes read + written), a 1 GiB read (torch's row
    sums of a (2^18, 4096) fp32 view: 1 GiB read, 1 MiB written; the
    fastest of torch's reductions here, where a flat sum streams at about
    3.6 TB/s) and a 8192^3 bf16 GEMM (hipBLASLt through torch)."""
    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3  # s
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev).view(-1, 4096)
    t_read = timed(lambda: big.sum(dim=1))
    del big
    m = 8192
    a = torch.randn(m, m, device=dev).to(torch.bfloat16)
    b = torch.randn(m, m, device=dev).to(torch.bfloat16)
    t_gemm = timed(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_512MiB_GBs": round(2 * n / t_copy / 1e9, 1),
            "read_1GiB_GBs": round(((1 << 30) + (1 << 20)) / t_read / 1e9, 1),
            "bf16_gemm_8192_TFLOPs": round(2 * m ** 3 / t_gemm / 1e12, 1)}


def graph_vs_eager(msgl, dev, iters=300):
    """A small decode step -- store_kv of 8 new rows, then decode of 8
    requests of 512 tokens in the Llama-3-8B geometry -- issued as the eager
    calls and as one replay of the graph runner's size-8 graph, back to back
    with one synchronisation at the end (launch overhead dominates at this
    size)."""
    from workloads import build_case
    B, L = 8, 512
    wl = build_case(8, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    prefix_lens=[L - 1] * B, extend_lens=[1] * B, num_pages=4096, device=dev)
    ph = wl.phases[0]
    p = Prepared(wl, ph, dev)
    # graphs at 1, 2, 4, 8, 16; the batch of 8 replays the size-8 graph
    g = msgl.DecodeGraphRunner(p.pool, wl.layer, 16, wl.num_qo_heads, L, p.pt)
    g.fill(p.q, p.k, p.v, p.loc, p.ti, p.sl, g.pick(B))

    def eager():
        run_store(msgl, p)
        run_decode(msgl, p)

    res = {"batch": B, "seq_len": L, "captured_sizes": g.sizes, "replayed_size": g.pick(B)}
    for name, fn in (("eager", eager), ("graph", lambda: g.launch(B))):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters):
            fn()
        torch.cuda.synchronize()
        res[f"{name}_us_per_step"] = round((time.perf_counter() - t0) / iters * 1e6, 2)
    res["graph_matches_eager"] = bool(torch.equal(g.out[:B].view(torch.int16), p.out.view(torch.int16)))
    g.close()

    # a whole decode step over NL layers (store_kv + decode per layer, the
    # same calls), eager against one replay of a torch graph capturing them
    NL = 32
    pool = torch.randn((2, NL) + tuple(wl.pool.shape[2:]), device=dev).to(torch.bfloat16)
    out = torch.empty_like(p.q)

    def layers():
        for layer in range(NL):
            msgl.store_kv(pool, layer, p.k, p.v, p.loc)
            msgl.paged_decode(pool, layer, p.q, p.pt, p.ti, p.sl, p.max_len, out=out,
                              workspace=p.ws)

    layers()
    torch.cuda.synchronize()
    tg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(tg):
        layers()
    res["layers"] = NL
    for name, fn in (("eager_layers", layers), ("graph_layers", tg.replay)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters // 10):
            fn()
        torch.cuda.synchronize()
        res[f"{name}_us_per_step"] = round((time.perf_counter() - t0) / (iters // 10) * 1e6, 1)
    del tg, pool
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=16.0, help="seconds of oracle work")
    ap.add_argument("--cold-iters", type=int, default=10)
    ap.add_argument("--step-only", action="store_true",
                    help="skip the extra measurements (decode graphs, mixed batch, page allocation, "
                         "fused rotary embedding, the other two workloads), so that profiles see "
                         "only the step's kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--only", choices=["chunked_prefill", "qwen3_moe_decode", "mixed_batch",
                                       "decode_graph", "rope_store_kv", "alloc_pages", "tp_share"],
                    help="time only this workload (store_kv + attention) and print its figures; "
                         "for profiles of the workloads outside the step")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(attention shards by heads or requests with no exchange between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    import paged_kv_attention_loc_amd as msgl
    from workloads import config_llama3_8b_decode, config_radix_shared_extend

    msgl.load_library()
    if args.only:
        log(f"{args.only} only")
        if args.only == "mixed_batch":
            res = {"mixed_batch": mixed_stats(msgl, dev, iters=max(1, args.steps))}
        elif args.only == "decode_graph":
            res = {"decode_graph": graph_vs_eager(msgl, dev)}
        elif args.only == "tp_share":
            res = {"tp8_share": tp_share_stats(msgl, dev)}
        elif args.only == "alloc_pages":
            wl_dec = config_llama3_8b_decode(device=dev)
            wl_ext = config_radix_shared_extend(device=dev)
            res = {"alloc_pages": {
                "decode_step": alloc_stats(msgl, Prepared(wl_dec, wl_dec.phases[0], dev), dev),
                "extend_step": alloc_stats(msgl, Prepared(wl_ext, wl_ext.phases[0], dev), dev)}}
        elif args.only == "rope_store_kv":
            from workloads import config_radix_shared_extend
            wl_ext = config_radix_shared_extend(device=dev)
            pe = Prepared(wl_ext, wl_ext.phases[0], dev)
            res = {"rope_store_kv": rope_store_stats(msgl, pe, dev, iters=max(1, args.steps)),
                   "store_kv_chunk_4096_rows": store_chunk_stats(msgl, dev, iters=max(1, args.steps))}
        else:
            res = other_workloads(msgl, dev, ext_iters=max(1, args.steps),
                                  dec_iters=max(1, args.steps), only=args.only)
        if args.copy_calibration:
            src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        print(json.dumps(res), flush=True)
        return
    log("building workloads on the device")
    wl_dec = config_llama3_8b_decode(device=dev)
    wl_ext = config_radix_shared_extend(device=dev)
    pd = Prepared(wl_dec, wl_dec.phases[0], dev)
    pe = Prepared(wl_ext, wl_ext.phases[0], dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        run_store(msgl, pd)
        if ev is not None:
            ev[1].record()
        run_decode(msgl, pd)
        if ev is not None:
            ev[2].record()
        run_store(msgl, pe)
        if ev is not None:
            ev[3].record()
        run_extend(msgl, pe)
        if ev is not None:
            ev[4].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(4)] for ev in events])  # ms
    st_dec_ms, dec_ms, st_ext_ms, ext_ms = per.mean(axis=0)
    dec_med = float(np.median(per[:, 1]))
    ext_med = float(np.median(per[:, 3]))

    # decode after reading a 1 GiB buffer: the 256 MB MALL and the L2s then
    # hold none of the pool (the flush is a read, so it leaves no dirty
    # lines whose write-back would be charged to the decode)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.cold_iters):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run_decode(msgl, pd)
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    cold_ms = float(np.median(cold))

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 512 MiB device copies")
        del src, dst

    ph_d, ph_e = wl_dec.phases[0], wl_ext.phases[0]
    dbytes = decode_bytes(wl_dec, ph_d)
    eflops = extend_flops(wl_ext, ph_e)
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9
    ext_tflops = eflops / (ext_ms * 1e-3) / 1e12
    sb_dec = store_bytes(wl_dec, ph_d.num_tokens)
    sb_ext = store_bytes(wl_ext, ph_e.num_tokens)

    alloc = mixed = rope_stats = graph_stats = others = ceilings = store_chunk = tp_share = None
    if not args.step_only:
        log("measured ceilings (copy, read, bf16 GEMM)")
        ceilings = measured_ceilings(dev)
        log("device-side page allocation")
        alloc = {"decode_step": alloc_stats(msgl, pd, dev), "extend_step": alloc_stats(msgl, pe, dev)}
        log("mixed decode + extend batch")
        mixed = mixed_stats(msgl, dev)
        log("fused rotary embedding + store_kv (extend rows)")
        rope_stats = rope_store_stats(msgl, pe, dev)
        log("store_kv of a 4096-row chunk")
        store_chunk = store_chunk_stats(msgl, dev)
        log("decode graph vs eager calls (small batch)")
        graph_stats = graph_vs_eager(msgl, dev)
        log("chunked 32k prefill and the Qwen3-30B-A3B-geometry decode")
        others = other_workloads(msgl, dev)
        log("one GPU's share of Llama-3-8B at tensor parallelism 8")
        tp_share = tp_share_stats(msgl, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl_dec, ph_d, wl_ext, ph_e, args.cpu_budget)

    result = {
        "metric": "decode paged-attn KV GB/s + extend TFLOP/s on 1 MI355X (frac. of roofline)",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("llama3-8b-geometry decode: 32q/8kv d128 ps16 B64 L~U[512,4096] "
                         "(sum L 154680) store_kv+decode; + radix-shared extend: 16 x "
                         "(prefix 2048 shared + 512 new) store_kv+extend"),
            "decode_batch": ph_d.batch,
            "decode_sum_seq_len": int(ph_d.seq_lens.sum()),
            "extend_batch": ph_e.batch,
            "extend_tokens": ph_e.num_tokens,
            "page_size": wl_dec.page_size,
            "num_qo_heads": wl_dec.num_qo_heads,
            "num_kv_heads": wl_dec.num_kv_heads,
            "head_dim": wl_dec.head_dim,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "msgl_paged_decode (balanced-range decode + merge)",
            "achieved": round(dec_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode"),
            "algorithmic_bytes_per_launch": dbytes,
            "avg_launch_us": round(dec_ms * 1e3, 3),
            "median_launch_us": round(dec_med * 1e3, 3),
            "cold_mall_median_us": round(cold_ms * 1e3, 3),
            "cold_mall_GBs": round(dbytes / (cold_ms * 1e-3) / 1e9, 2),
            "measured_ceiling": None if ceilings is None else {
                "copy_GBs": ceilings["copy_512MiB_GBs"],
                "read_GBs": ceilings["read_1GiB_GBs"],
                "frac_of_copy": round(dec_gbs / ceilings["copy_512MiB_GBs"], 4),
                "frac_of_read": round(dec_gbs / ceilings["read_1GiB_GBs"], 4)},
        },
        "roofline_extend": {
            "bound": "mfma",
            "kernel": "msgl_paged_extend",
            "achieved": round(ext_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ext_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("extend"),
            "algorithmic_flops_per_launch": eflops,
            "avg_launch_us": round(ext_ms * 1e3, 3),
            "median_launch_us": round(ext_med * 1e3, 3),
            "measured_ceiling": None if ceilings is None else {
                "bf16_gemm_TFLOPs": ceilings["bf16_gemm_8192_TFLOPs"],
                "frac_of_gemm": round(ext_tflops / ceilings["bf16_gemm_8192_TFLOPs"], 4)},
        },
        "store_kv": {
            "decode_rows": ph_d.num_tokens,
            "decode_avg_us": round(st_dec_ms * 1e3, 3),
            "decode_GBs": round(sb_dec / (st_dec_ms * 1e-3) / 1e9, 2),
            "extend_rows": ph_e.num_tokens,
            "extend_avg_us": round(st_ext_ms * 1e3, 3),
            "extend_GBs": round(sb_ext / (st_ext_ms * 1e-3) / 1e9, 2),
            "chunk_4096_rows": store_chunk,
        },
        "extend_tflops": round(ext_tflops, 2),
        "decode_graph": graph_stats,
        "rope_store_kv": rope_stats,
        "alloc_pages": alloc,
        "mixed_batch": mixed,
        "other_workloads": others,
        "tp8_share": tp_share,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
