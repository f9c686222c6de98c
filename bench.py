"""Throughput of the attention hot path on one MI355X.

One step runs every stage of the path once on resident synthetic inputs:
  1. causal GQA prefill, Hq=32, Hkv=8, D=128, S=4096, bf16 (the workload the
     headline TFLOP/s is quoted on);
  2. paged split-KV decode + combine, 64 sequences with contexts uniform in
     [512, 4096], shuffled 16-token pages, Hq=32, Hkv=8, D=128;
  3. long-context split-KV decode + combine, B=1, Hq=16, Hkv=4, D=256,
     131072 cached tokens.
`value` is the prefill TFLOP/s (algorithmic causal FLOPs / prefill time);
the decodes are reported as KV-read GB/s in the same JSON line. Each kernel
call is bracketed by HIP events on the stream it runs on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "attention TFLOP/s (prefill); decode KV-read GB/s; % of MI355X roofline"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "attention_attn_fwd_03_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key: str, launches_bytes_alg: float):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(kernel_key)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(prefill_case, min_seconds: float = 10.0, max_reps: int = 8):
    """The fp64 oracle timed on the host cores on a bounded sample of the
    prefill workload: the whole causal GQA problem (all query heads), run
    until at least `min_seconds` of CPU time have accumulated."""
    import oracle
    from attention_attn_fwd_03_amd import accounting
    q, k, v = prefill_case.as_f64()
    H, Hkv = prefill_case.num_q_heads, prefill_case.num_kv_heads
    reps, t_total = 0, 0.0
    while reps < max_reps and (reps == 0 or t_total < min_seconds):
        t0 = time.perf_counter()
        oracle.attention_dense(q, k, v, prefill_case.cu_seqlens, H, Hkv, prefill_case.scale, True)
        t_total += time.perf_counter() - t0
        reps += 1
    fl = accounting.prefill_flops(prefill_case.seqlens, H, prefill_case.head_dim, True) * reps
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    return {"value": fl / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the causal GQA prefill S={prefill_case.total_tokens}, Hq={H}, Hkv={Hkv}, "
                      f"D={prefill_case.head_dim} (all heads), {reps} run(s), {t_total:.1f} s; fp64 numpy "
                      f"materialized form; host has {len(os.sched_getaffinity(0))} usable cores"}


def sweep_splits(torch, mi, dev):
    """Paged decode time for split counts 1, 2, 4, ..., 256 and for the
    library's own plan (num_splits = 0) on synthetic caches (seeded
    device-side normals, shuffled 16-token pages), for the two decode shapes
    and batch 1-128, contexts 1K-64K (fixed, and uniform in [ctx/8, ctx])."""
    import statistics
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rng = torch.Generator().manual_seed(1)

    def make(lens, Hq, Hkv, D):
        pages = [(L + 15) // 16 for L in lens]
        tot, mp = sum(pages), max(pages)
        kc = torch.randn((tot, 16, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn((tot, 16, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        perm = torch.randperm(tot, generator=g, device=dev).to(torch.int32)
        bt = torch.full((len(lens), mp), -1, dtype=torch.int32, device=dev)
        o = 0
        for b, n in enumerate(pages):
            bt[b, :n] = perm[o:o + n]
            o += n
        q = torch.randn((len(lens), Hq, D), generator=g, device=dev).to(torch.bfloat16)
        return q, kc, vc, bt, torch.tensor(lens, dtype=torch.int32, device=dev)

    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)

    def time_it(args, S, scale):
        # per-call events; a working set below 512 MB (twice the last-level
        # cache) is evicted by a 512 MB read before each call, outside the
        # events, so its K/V come from HBM
        cold = 4 * args[1].numel() < 512e6
        for _ in range(3):
            mi.attn_decode_paged(*args, scale=scale, num_splits=S)
        torch.cuda.synchronize()
        evs = []
        for i in range(40):
            if cold:
                flush.max()   # read-only: leaves no dirty lines behind
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            mi.attn_decode_paged(*args, scale=scale, num_splits=S)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return statistics.median([a.elapsed_time(b) * 1e3 for a, b in evs])

    # the grid of batch x context, plus launches around the plan's size
    # threshold (batch x table width between 2^16 and 2^19 tokens)
    grid = [(B, ctx) for B in (1, 4, 16, 64) for ctx in (1024, 4096, 16384, 65536) if B * ctx <= 1 << 20]
    grid += [(8, 16384), (8, 32768), (16, 8192), (32, 4096), (32, 8192), (64, 2048), (64, 3072), (128, 2048)]
    for Hq, Hkv, D in ((32, 8, 128), (16, 4, 256)):
        for B, ctx in grid:
            for var in (False, True):
                if var and B == 1:
                    continue
                lens = [ctx] * B if not var else [int(x) for x in torch.randint(ctx // 8, ctx + 1, (B,),
                                                                                    generator=rng)]
                args = make(lens, Hq, Hkv, D)
                pol = mi.decode_pick_splits(B, Hkv, max(lens))
                cand = sorted({1, 2, 4, 8, 16, 32, 64, 128, 256, pol})
                res = {S: round(time_it(args, S, D ** -0.5), 1) for S in cand if S <= (max(lens) + 15) // 16}
                lib = round(time_it(args, 0, D ** -0.5), 1)   # the library's own plan
                best = min(res, key=res.get)
                by = 4 * sum(lens) * Hkv * D
                print(json.dumps({"shape": {"Hq": Hq, "Hkv": Hkv, "D": D}, "B": B, "ctx": ctx,
                                  "table_tokens": B * ((max(lens) + 15) // 16) * 16,
                                  "lengths": "uniform [ctx/8, ctx]" if var else "fixed", "policy": pol,
                                  "us_policy": res.get(pol), "us_library": lib,
                                  "fastest": best, "us_fastest": res[best],
                                  "GB/s_fastest": round(by / res[best] / 1e3, 1), "us_by_splits": res}),
                      flush=True)
                del args
                torch.cuda.empty_cache()


def numerics_timing(torch, mi, dev, bf16, i32, steps: int, warmup: int):
    """Time the decode's numerics variants (split records, rounding points,
    round-robin tiles) beside the fast path on the paged-decode and
    long-context workloads; one JSON line per variant."""
    import synth
    from attention_attn_fwd_03_amd import accounting

    R = mi
    for case in (synth.config3(seed=0, tail="zero"), synth.config4(ctx=131072, seed=0),
                 synth.config4(ctx=32768, seed=0)):
        args = (bf16(case.q), bf16(case.k_cache), bf16(case.v_cache), i32(case.block_table), i32(case.seq_lens))
        pol = mi.decode_pick_splits(case.batch, case.num_kv_heads, case.max_pages * 16)
        n_tiles8 = -(-case.max_pages // 8)
        variants = [("fast path (attn_decode_paged)", None, pol, 0),
                    ("LSE record", R.RECORD_LSE, pol, 0),
                    ("fp32 numerators", R.RECORD_NUMERATOR_F32, pol, 0),
                    ("bf16 normalised + rounded l, 16-page tiles round robin",
                     R.RECORD_NORMALIZED_BF16 | R.NUMERICS_ROUNDED_NORMALIZER, pol, 16),
                    ("bf16 numerators, ordered merge, one group per 8 pages", R.RECORD_NUMERATOR_BF16,
                     n_tiles8, 8),
                    ("LSE record, fp16 P", R.RECORD_LSE | R.NUMERICS_P_FP16, pol, 0)]
        by = accounting.decode_bytes(case.seq_lens, case.num_q_heads, case.num_kv_heads, case.head_dim)
        base = None
        for label, numerics, S, tp in variants:
            if numerics is None:
                def f():
                    mi.attn_decode_paged(*args, scale=case.scale, num_splits=S)
            else:
                def f():
                    mi.attn_decode_paged_numerics(*args, scale=case.scale, num_splits=S, numerics=numerics,
                                                  tile_pages=tp)
            for _ in range(warmup):
                f()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                f()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            base = base or us
            print(json.dumps({"numerics": label, "workload": case.name, "splits": S, "tile_pages": tp,
                              "us": round(us, 2), "GB/s": round(by / us / 1e3, 1),
                              "frac_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                              "time_vs_fast_path": round(us / base, 3)}), flush=True)
        del args
        torch.cuda.empty_cache()


def mfma_peak(torch, dev, iters: int = 2000):
    """Matrix-core rate of this chip: back-to-back 32x32x16 bf16 MFMAs on
    register operands (libmiattn_peak.so), over 1-16 independent accumulator
    chains and 1, 2 or 4 workgroups of four waves per compute unit; one JSON
    line per cell, then the best rate beside the published dense peak."""
    import ctypes
    from attention_attn_fwd_03_amd.build import PEAK_LIB
    lib = ctypes.CDLL(PEAK_LIB)
    lib.miattn_probe_mfma_peak.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p]
    lib.miattn_probe_mfma_peak.restype = ctypes.c_int
    # bf16 operands near 1.0 (bit patterns 0x3f80 + small offsets): finite sums
    seed = (torch.arange(32, dtype=torch.int32, device=dev) + 0x3F80).contiguous()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    best = None
    for chains in (1, 2, 4, 8, 16):
        for blocks in (256, 512, 1024):
            out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

            def run(n):
                rc = lib.miattn_probe_mfma_peak(ctypes.c_void_p(seed.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                                blocks, n, chains, st)
                assert rc == 0, rc
            t_end = time.perf_counter() + 0.2   # settle the clock under this load
            while time.perf_counter() < t_end:
                run(iters)
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run(iters)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            tf = blocks * 4 * iters * 16 * 32768 / (ms * 1e-3) / 1e12
            cell = {"probe": "mfma_f32_32x32x16_bf16, register operands", "chains": chains,
                    "workgroups": blocks, "waves_per_simd": blocks // 256, "ms": round(ms, 4),
                    "TFLOP/s": round(tf, 1), "frac_of_2500": round(tf / PEAK_BF16_TFLOPS, 4)}
            print(json.dumps(cell), flush=True)
            if best is None or tf > best["TFLOP/s"]:
                best = cell
    print(json.dumps({"mfma_peak_best": best, "published_dense_bf16_TFLOP/s": PEAK_BF16_TFLOPS}), flush=True)


def cells(torch, mi, dev, bf16, i32, f32, oracle_too: bool):
    """Every cell of the measurement table, one op per cell: 10 warmups, then
    each call bracketed by its own HIP events (median and min reported). Cells
    whose working set is below 512 MB (twice the 256 MB last-level cache) get a
    512 MB read of a scratch buffer before each timed call, outside the
    events, so their inputs come from HBM (a read, not a write: written lines
    would still be draining to HBM during the timed call). With `oracle_too`, the fp64 oracle
    is timed on the host on a bounded sample of each workload."""
    import statistics
    import oracle
    import synth
    from attention_attn_fwd_03_amd import accounting
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)

    def timed(f, n, cold):
        for _ in range(10):
            f()
        torch.cuda.synchronize()
        evs = []
        for i in range(n):
            if cold:
                flush.max()   # read-only: leaves no dirty lines behind
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        return statistics.median(us), min(us)

    def oracle_time(fn, work, unit, sample, min_s=2.0):
        reps, tot = 0, 0.0
        while reps == 0 or (tot < min_s and reps < 5):
            t0 = time.perf_counter()
            fn()
            tot += time.perf_counter() - t0
            reps += 1
        return {"value": work * reps / tot / (1e12 if unit == "TFLOP/s" else 1e9), "unit": unit,
                "sample": sample, "reps": reps, "s": round(tot, 2)}

    def emit(d):
        print(json.dumps(d), flush=True)

    # config 1: dense fp32, one head, 256 tokens, non-causal (latency)
    c1 = synth.config1(0)
    a1 = (f32(c1.q), f32(c1.k), f32(c1.v), i32(c1.cu_seqlens))

    def f1():
        mi.attn_fwd(*a1, c1.max_seqlen, scale=c1.scale, causal=False)
    warm, _ = timed(f1, 200, False)
    cold, mn = timed(f1, 200, True)
    d = {"cell": "config1 fp32 dense S=256 D=64", "us_median_warm": round(warm, 2), "us_median_cold": round(cold, 2),
         "us_min_cold": round(mn, 2), "bound": "latency"}
    if oracle_too:
        q, k, v = c1.as_f64()
        d["oracle"] = oracle_time(lambda: oracle.attention_dense(q, k, v, c1.cu_seqlens, 1, 1, c1.scale, False),
                                  accounting.prefill_flops(c1.seqlens, 1, 64, False), "TFLOP/s", "whole workload")
    emit(d)

    # config 2: causal GQA prefill at S = 1024, 2048, 4096
    for S in (1024, 2048, 4096):
        c = synth.config2(S=S, seed=0)
        a = (bf16(c.q), bf16(c.k), bf16(c.v), i32(c.cu_seqlens))
        o = torch.empty_like(a[0])
        lse = torch.empty((32, S), dtype=torch.float32, device=dev)

        def f():
            mi.attn_fwd(*a, c.max_seqlen, scale=c.scale, causal=True, out=o, lse=lse)
        med, mn = timed(f, 50, True)
        fl = accounting.prefill_flops(c.seqlens, 32, 128, True)
        emit({"cell": f"config2 causal GQA prefill S={S}", "us_median": round(med, 2), "us_min": round(mn, 2),
              "TFLOP/s": round(fl / med / 1e6, 1), "frac_mfma": round(fl / med / 1e6 / PEAK_BF16_TFLOPS, 4),
              "flushed": True})
        del a, o, lse

    # config 3: paged decode, 64 sequences
    c3 = synth.config3(seed=0, tail="zero")
    a3 = (bf16(c3.q), bf16(c3.k_cache), bf16(c3.v_cache), i32(c3.block_table), i32(c3.seq_lens))
    by3 = accounting.decode_bytes(c3.seq_lens, 32, 8, 128)
    for S in (0, 1, 2, 4, 8, 16, 32):
        med, mn = timed(lambda: mi.attn_decode_paged(*a3, scale=c3.scale, num_splits=S), 200, False)
        emit({"cell": f"config3 paged decode B=64 splits={S or 'library plan'}", "us_median": round(med, 2),
              "us_min": round(mn, 2), "GB/s": round(by3 / med / 1e3, 1),
              "frac_hbm": round(by3 / med / 1e3 / PEAK_HBM_GBS, 4), "working_set_MB": round(by3 / 1e6, 1),
              "flushed": False})
    if oracle_too:
        q, kc, vc = c3.as_f64()
        emit({"cell": "config3 oracle", "oracle": oracle_time(
            lambda: oracle.decode_dense(q, kc, vc, c3.block_table, c3.seq_lens, c3.scale), by3, "GB/s",
            "whole workload (64 sequences, all heads)")})
        del q, kc, vc
    del a3

    # config 4: long decode, contexts 16K-128K x split counts
    for ctx in (16384, 32768, 65536, 131072):
        c = synth.config4(ctx=ctx, seed=0)
        a = (bf16(c.q), bf16(c.k_cache), bf16(c.v_cache), i32(c.block_table), i32(c.seq_lens))
        by = accounting.decode_bytes(c.seq_lens, 16, 4, 256)
        cold = by < 512e6
        for S in (1, 16, 64, 256, 0):
            med, mn = timed(lambda: mi.attn_decode_paged(*a, scale=c.scale, num_splits=S), 200, cold)
            emit({"cell": f"config4 long decode ctx={ctx} splits={S or 'policy'}", "us_median": round(med, 2),
                  "us_min": round(mn, 2), "GB/s": round(by / med / 1e3, 1),
                  "frac_hbm": round(by / med / 1e3 / PEAK_HBM_GBS, 4), "working_set_MB": round(by / 1e6, 1),
                  "flushed": cold})
        if oracle_too and ctx == 131072:
            q, kc, vc = c.as_f64()
            emit({"cell": "config4 oracle ctx=131072", "oracle": oracle_time(
                lambda: oracle.decode_dense(q, kc, vc, c.block_table, c.seq_lens, c.scale), by, "GB/s",
                "whole workload (128K tokens, 16 heads)")})
            del q, kc, vc
        del a
        torch.cuda.empty_cache()

    # config 5: varlen causal prefill, head_dim 256
    c5 = synth.config5(seed=0)
    a5 = (bf16(c5.q), bf16(c5.k), bf16(c5.v), i32(c5.cu_seqlens))
    o5 = torch.empty_like(a5[0])
    l5 = torch.empty((16, c5.total_tokens), dtype=torch.float32, device=dev)
    med, mn = timed(lambda: mi.attn_fwd(*a5, c5.max_seqlen, scale=c5.scale, causal=True, out=o5, lse=l5), 20,
                    False)
    fl5 = accounting.prefill_flops(c5.seqlens, 16, 256, True)
    emit({"cell": "config5 varlen causal prefill D=256", "us_median": round(med, 2), "us_min": round(mn, 2),
          "TFLOP/s": round(fl5 / med / 1e6, 1), "frac_mfma": round(fl5 / med / 1e6 / PEAK_BF16_TFLOPS, 4),
          "flushed": False})
    if oracle_too:
        # the longest sequence alone (all 16 heads)
        b = int(np.argmax(c5.seqlens))
        s0, s1 = int(c5.cu_seqlens[b]), int(c5.cu_seqlens[b + 1])
        q, k, v = c5.as_f64()
        q, k, v = q[s0:s1], k[s0:s1], v[s0:s1]
        emit({"cell": "config5 oracle", "oracle": oracle_time(
            lambda: oracle.attention_dense(q, k, v, np.array([0, s1 - s0]), 16, 4, c5.scale, True),
            accounting.prefill_flops([s1 - s0], 16, 256, True), "TFLOP/s",
            f"the longest sequence ({s1 - s0} tokens), all 16 heads", min_s=1.0)})
    # the backward of the same varlen head_dim-256 problem (forward outputs once)
    mi.attn_fwd(*a5, c5.max_seqlen, scale=c5.scale, causal=True, out=o5, lse=l5)
    do5 = bf16(synth.output_gradient(9, 0, c5.total_tokens, 16, 256))
    med, mn = timed(lambda: mi.attn_bwd(a5[0], a5[1], a5[2], o5, l5, do5, a5[3], c5.max_seqlen, scale=c5.scale,
                                        causal=True), 10, False)
    fb5 = accounting.backward_flops(c5.seqlens, 16, 256, True)
    emit({"cell": "config5 varlen causal backward D=256", "us_median": round(med, 2), "us_min": round(mn, 2),
          "TFLOP/s": round(fb5 / med / 1e6, 1), "frac_mfma": round(fb5 / med / 1e6 / PEAK_BF16_TFLOPS, 4),
          "flushed": False})
    del a5, o5, l5, do5


# kernels whose HBM traffic the counter summary records: key -> (stage run by
# --only, kernel-name substrings of one launch)
TRAFFIC_KERNELS = {
    "prefill_causal_gqa_s4096": ("prefill", ["miattn_prefill_pp_kernel"]),
    "decode_paged_b64": ("decode", ["miattn_decode_split_kernel", "miattn_combine_kernel"]),
    "decode_long_ctx131072": ("long", ["miattn_decode_split_kernel", "miattn_combine_kernel"]),
    "chunked_prefill_8x1024": ("chunked", ["miattn_prefill_fwd_kernel"]),
    "varlen_prefill_d256": ("varlen", ["miattn_prefill_pair_kernel", "miattn_bf16_to_f16_kernel"]),
    "backward_causal_gqa_s4096": ("backward", ["miattn_bwd_prep_kernel", "miattn_bwd_dkdv_pair_kernel",
                                               "miattn_bwd_dq_kernel"]),
}


def summarize_counters(root: str):
    """Turn rocprofv3 --pmc runs into profiles/hbm_traffic.json.

    `root` holds one rocprofv3 output directory per (stage, counter), named
    `<stage>_FETCH_SIZE` / `<stage>_WRITE_SIZE`, for every stage named in
    TRAFFIC_KERNELS and for copy (--only copy, a 1 GiB device copy). Counter
    values are KiB per dispatch; each is scaled by (true bytes / counter
    bytes) of the copy, which reads and writes exactly 1 GiB."""
    import csv
    import glob
    import sqlite3

    def per_dispatch(stage, counter):
        """median over dispatches of each kernel's counter value (rocprofv3
        writes a rocpd SQLite database, or CSV with --output-format csv)"""
        d = os.path.join(root, f"{stage}_{counter}")
        vals = {}
        for fn in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            con = sqlite3.connect(fn)
            for name, disp, v in con.execute(
                    "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?",
                    (counter,)):
                vals[(name, disp)] = vals.get((name, disp), 0.0) + float(v)   # sum over instances
            con.close()
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        key = (r["Kernel_Name"], r.get("Dispatch_Id", ""))
                        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        by_kernel = {}
        for (name, _), v in vals.items():
            by_kernel.setdefault(name, []).append(v)
        return {n: float(np.median(v)) for n, v in by_kernel.items()}

    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = per_dispatch("copy", counter)
        kib = max(d.values())   # the copy kernel is the dispatch with the most traffic
        cal[counter] = (1 << 30) / (kib * 1024.0)
    out = {"counter_unit": "KiB per dispatch", "calibration_1GiB_copy": cal,
           "source_hash": kernel_source_hash(), "kernels": {}}
    for key, (stage, names) in TRAFFIC_KERNELS.items():
        rec = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = per_dispatch(stage, counter)
            kib = sum(v for n, v in d.items() if any(s in n for s in names))
            rec[counter] = {"raw_kib": kib, "bytes": kib * 1024.0 * cal[counter]}
        rec["hbm_bytes_per_launch"] = rec["FETCH_SIZE"]["bytes"] + rec["WRITE_SIZE"]["bytes"]
        rec["source_hash"] = out["source_hash"]
        out["kernels"][key] = rec
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed steps for this long before the warmup steps: the GPU clock ramps up "
                         "over the first few hundred milliseconds of sustained load")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-splits", type=int, default=0, help="0 = library policy")
    ap.add_argument("--long-splits", type=int, default=0, help="0 = library policy")
    ap.add_argument("--long-ctx", type=int, default=131072,
                    help="context of the long decode (only with --only long: the step keeps 131072)")
    ap.add_argument("--flush-each", action="store_true",
                    help="with --only: read a 512 MB scratch buffer before every call, so inputs below the "
                         "last-level cache come from HBM (the printed mean then includes the reads; per-kernel "
                         "times come from a kernel trace)")
    ap.add_argument("--only", choices=["prefill", "decode", "long", "chunked", "backward", "varlen", "copy"],
                    default=None,
                    help="profiling aid: run just one stage (or a 1 GiB device copy used to calibrate "
                         "the HBM byte counters) for --steps iterations and print its mean time")
    ap.add_argument("--sweep-splits", action="store_true",
                    help="time paged decode over split counts on a grid of batch sizes and contexts and print "
                         "the library policy's pick beside the fastest (one JSON line per cell)")
    ap.add_argument("--graph", action="store_true",
                    help="the step (prefill + paged decode + long decode) captured once in a HIP graph: "
                         "time per step replayed against the same calls made eagerly on the same stream")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="measure the matrix cores' sustained bf16 rate with a register-operand probe")
    ap.add_argument("--cells", action="store_true",
                    help="time every workload cell (one op per cell, per-call events, cache flush below 512 MB)")
    ap.add_argument("--cells-oracle", action="store_true",
                    help="with --cells: also time the fp64 oracle on a bounded sample of each workload")
    ap.add_argument("--numerics", action="store_true",
                    help="time the decode numerics variants beside the fast path (one JSON line each)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="write profiles/hbm_traffic.json from rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a design note, "
                                   "not implemented", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.long_ctx != 131072 and args.only != "long":
        ap.error("--long-ctx changes the long decode's context; use it with --only long")
    if args.flush_each and args.only is None:
        ap.error("--flush-each applies to --only runs")

    import torch
    import attention_attn_fwd_03_amd as mi
    import synth
    from attention_attn_fwd_03_amd import accounting

    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if args.sweep_splits:
        sweep_splits(torch, mi, dev)
        return
    if args.mfma_peak:
        mfma_peak(torch, dev)
        return
    if args.cells:
        cells(torch, mi, dev, bf16, i32, f32, args.cells_oracle)
        return

    if args.numerics:
        numerics_timing(torch, mi, dev, bf16, i32, args.steps, args.warmup)
        return

    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "ms": dt * 1e3,
                          "GB/s": 2 * n / dt / 1e9}), flush=True)
        return

    print("[bench] generating inputs", file=sys.stderr, flush=True)
    want = {"prefill", "decode", "long", "chunked", "backward", "varlen"} if args.only is None else {args.only}
    if args.graph:
        want = {"prefill", "decode", "long"}
    P = Dd = Ld = None
    pc = synth.config2(S=4096, seed=0)
    if "prefill" in want or "backward" in want:
        P = dict(q=bf16(pc.q), k=bf16(pc.k), v=bf16(pc.v), cu=i32(pc.cu_seqlens))
        P["o"] = torch.empty_like(P["q"])
        P["lse"] = torch.empty((pc.num_q_heads, pc.total_tokens), dtype=torch.float32, device=dev)
    if "backward" in want:
        # the same causal GQA problem: forward outputs once, then the backward
        # on a seeded upstream gradient
        mi.attn_fwd(P["q"], P["k"], P["v"], P["cu"], pc.max_seqlen, scale=pc.scale, causal=True,
                    out=P["o"], lse=P["lse"])
        P["do"] = bf16(synth.output_gradient(9, 0, pc.total_tokens, pc.num_q_heads, pc.head_dim))
        P["dq"] = torch.empty_like(P["q"])
        P["dk"] = torch.empty_like(P["k"])
        P["dv"] = torch.empty_like(P["v"])
    dc = synth.config3(seed=0, tail="zero") if "decode" in want else None
    if dc is not None:
        Dd = dict(q=bf16(dc.q), kc=bf16(dc.k_cache), vc=bf16(dc.v_cache), bt=i32(dc.block_table),
                  sl=i32(dc.seq_lens))
        Dd["o"] = torch.empty_like(Dd["q"])
        Dd["lse"] = torch.empty((dc.batch, dc.num_q_heads), dtype=torch.float32, device=dev)
        # 0 = the library's policy (length-proportional groups where it splits)
        dsplits = args.decode_splits
    lc = synth.config4(ctx=args.long_ctx, seed=0) if "long" in want else None
    if lc is not None:
        Ld = dict(q=bf16(lc.q), kc=bf16(lc.k_cache), vc=bf16(lc.v_cache), bt=i32(lc.block_table),
                  sl=i32(lc.seq_lens))
        Ld["o"] = torch.empty_like(Ld["q"])
        Ld["lse"] = torch.empty((lc.batch, lc.num_q_heads), dtype=torch.float32, device=dev)
        lsplits = args.long_splits

    cc = synth.config6(seed=0, tail="zero") if "chunked" in want else None
    if cc is not None:
        Cd = dict(q=bf16(cc.q), kc=bf16(cc.k_cache), vc=bf16(cc.v_cache), bt=i32(cc.block_table),
                  cu=i32(cc.cu_seqlens_q), sk=i32(cc.seq_lens_k))
        Cd["o"] = torch.empty_like(Cd["q"])
        Cd["lse"] = torch.empty((cc.num_q_heads, cc.total_q), dtype=torch.float32, device=dev)

    def chunked():
        mi.attn_fwd_paged(Cd["q"], Cd["kc"], Cd["vc"], Cd["bt"], Cd["cu"], Cd["sk"], cc.max_seqlen_q,
                          scale=cc.scale, causal=True, out=Cd["o"], lse=Cd["lse"])

    vc5 = synth.config5(seed=0) if "varlen" in want else None
    if vc5 is not None:
        V5 = dict(q=bf16(vc5.q), k=bf16(vc5.k), v=bf16(vc5.v), cu=i32(vc5.cu_seqlens))
        V5["o"] = torch.empty_like(V5["q"])
        V5["lse"] = torch.empty((vc5.num_q_heads, vc5.total_tokens), dtype=torch.float32, device=dev)

    def varlen():
        mi.attn_fwd(V5["q"], V5["k"], V5["v"], V5["cu"], vc5.max_seqlen, scale=vc5.scale, causal=True,
                    out=V5["o"], lse=V5["lse"])

    def backward():
        mi.attn_bwd(P["q"], P["k"], P["v"], P["o"], P["lse"], P["do"], P["cu"], pc.max_seqlen, scale=pc.scale,
                    causal=True, dq=P["dq"], dk=P["dk"], dv=P["dv"])

    def prefill():
        mi.attn_fwd(P["q"], P["k"], P["v"], P["cu"], pc.max_seqlen, scale=pc.scale, causal=True,
                    out=P["o"], lse=P["lse"])

    def decode():
        mi.attn_decode_paged(Dd["q"], Dd["kc"], Dd["vc"], Dd["bt"], Dd["sl"], scale=dc.scale,
                             num_splits=dsplits, out=Dd["o"], lse=Dd["lse"])

    def long_decode():
        mi.attn_decode_paged(Ld["q"], Ld["kc"], Ld["vc"], Ld["bt"], Ld["sl"], scale=lc.scale,
                             num_splits=lsplits, out=Ld["o"], lse=Ld["lse"])

    def settle(fns):
        # untimed: run the work until the clocks have settled (bounded queue)
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        n = 0
        while time.perf_counter() < t_end:
            for fn in fns:
                fn()
            n += 1
            if n % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    stages = [prefill, decode, long_decode]
    if args.only is not None:
        f = {"prefill": prefill, "decode": decode, "long": long_decode, "chunked": chunked,
             "backward": backward, "varlen": varlen}[args.only]
        if args.flush_each:
            flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
            f_run = f

            def f():
                flush.max()   # read-only: leaves no dirty lines behind
                f_run()
        settle([f])
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "ms": e0.elapsed_time(e1) / args.steps}), flush=True)
        return
    if args.graph:
        # the library's per-stream buffers are made by the eager calls on the
        # capturing stream; the graph then replays the same kernels on it
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            settle(stages)
            for _ in range(args.warmup):
                for f in stages:
                    f()
        gs.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            for f in stages:
                f()
        res = {}
        for mode in ("eager", "graph", "eager", "graph"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(gs):
                e0.record(gs)
                for _ in range(args.steps):
                    if mode == "graph":
                        graph.replay()
                    else:
                        for f in stages:
                            f()
                e1.record(gs)
            gs.synchronize()
            res[mode] = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"graph": True, "stages": "prefill S=4096 + paged decode B=64 + long decode "
                          f"ctx={args.long_ctx}", "steps": args.steps, "eager_ms_per_step": round(res["eager"], 4),
                          "graph_ms_per_step": round(res["graph"], 4)}), flush=True)
        return
    print(f"[bench] settle {args.settle_ms:.0f} ms, warmup {args.warmup}", file=sys.stderr, flush=True)
    settle(stages)
    for _ in range(args.warmup):
        for f in stages:
            f()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, f in enumerate(stages):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(stages))] for s in range(args.steps)])
    t_pre, t_dec, t_long = (float(np.mean(per[:, i])) * 1e-3 for i in range(3))
    step_ms = float(np.mean(per.sum(axis=1)))

    # chunked prefill (a row beyond the step): timed on its own after the step
    for _ in range(args.warmup):
        chunked()
    ce0 = torch.cuda.Event(enable_timing=True)
    ce1 = torch.cuda.Event(enable_timing=True)
    ce0.record(stream)
    for _ in range(args.steps):
        chunked()
    ce1.record(stream)
    torch.cuda.synchronize()
    t_chunk = ce0.elapsed_time(ce1) / args.steps * 1e-3
    # backward of the prefill workload (beside the step as well)
    for _ in range(args.warmup):
        backward()
    be0 = torch.cuda.Event(enable_timing=True)
    be1 = torch.cuda.Event(enable_timing=True)
    be0.record(stream)
    for _ in range(args.steps):
        backward()
    be1.record(stream)
    torch.cuda.synchronize()
    t_bwd = be0.elapsed_time(be1) / args.steps * 1e-3
    # varlen packed causal prefill at head_dim 256 (beside the step as well)
    for _ in range(args.warmup):
        varlen()
    ve0 = torch.cuda.Event(enable_timing=True)
    ve1 = torch.cuda.Event(enable_timing=True)
    ve0.record(stream)
    for _ in range(args.steps):
        varlen()
    ve1.record(stream)
    torch.cuda.synchronize()
    t_var = ve0.elapsed_time(ve1) / args.steps * 1e-3
    fl_var = accounting.prefill_flops(vc5.seqlens, vc5.num_q_heads, vc5.head_dim, True)
    by_var = accounting.prefill_bytes(vc5.total_tokens, vc5.num_q_heads, vc5.num_kv_heads, vc5.head_dim)
    fl_bwd = accounting.backward_flops(pc.seqlens, pc.num_q_heads, pc.head_dim, True)
    by_bwd = accounting.backward_bytes(pc.total_tokens, pc.num_q_heads, pc.num_kv_heads, pc.head_dim)

    fl_chunk = accounting.chunked_prefill_flops(cc.q_lens, cc.seq_lens_k, cc.num_q_heads, cc.head_dim, True)
    by_chunk = accounting.chunked_prefill_bytes(cc.q_lens, cc.seq_lens_k, cc.num_q_heads, cc.num_kv_heads,
                                                cc.head_dim)

    fl_pre = accounting.prefill_flops(pc.seqlens, pc.num_q_heads, pc.head_dim, True)
    tflops = fl_pre / t_pre / 1e12
    by_dec = accounting.decode_bytes(dc.seq_lens, dc.num_q_heads, dc.num_kv_heads, dc.head_dim)
    by_long = accounting.decode_bytes(lc.seq_lens, lc.num_q_heads, lc.num_kv_heads, lc.head_dim)
    gbs_dec = by_dec / t_dec / 1e9
    gbs_long = by_long / t_long / 1e9

    traffic = traffic_from_profile("prefill_causal_gqa_s4096", accounting.prefill_bytes(4096, 32, 8, 128))
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), rounded to bf16)",
        "config": {
            "workload": "causal GQA prefill Hq=32 Hkv=8 D=128 S=4096 + paged decode B=64 ctx U[512,4096] "
                        "shuffled 16-token pages + long decode B=1 Hq=16 Hkv=4 D=256 ctx=131072 (one step); "
                        "chunked prefill 8 chunks x 1024 after prefixes U[0,6144] and the prefill's backward "
                        "reported beside it",
            "prefill": {"S": 4096, "Hq": 32, "Hkv": 8, "D": 128, "causal": True, "ms": round(t_pre * 1e3, 4),
                        "algorithmic_gflop": round(fl_pre / 1e9, 3)},
            "decode_paged": {"B": dc.batch, "tokens": int(dc.seq_lens.sum()),
                             "splits": dsplits or "library policy: about 256 groups, each sequence's count "
                                                  "proportional to its length",
                             "ms": round(t_dec * 1e3, 4), "GB/s": round(gbs_dec, 1),
                             "frac_hbm": round(gbs_dec / PEAK_HBM_GBS, 4), "algorithmic_MB": round(by_dec / 1e6, 2),
                             "traffic": traffic_from_profile("decode_paged_b64", by_dec)},
            "decode_long": {"ctx": 131072, "splits": lsplits or "library policy: 256 groups",
                            "ms": round(t_long * 1e3, 4),
                            "GB/s": round(gbs_long, 1), "frac_hbm": round(gbs_long / PEAK_HBM_GBS, 4),
                            "algorithmic_MB": round(by_long / 1e6, 2)},
            "chunked_prefill": {"chunks": len(cc.q_lens), "chunk": cc.q_lens[0],
                                "cached_tokens": int(cc.seq_lens_k.sum()), "Hq": 32, "Hkv": 8, "D": 128,
                                "causal": True, "ms": round(t_chunk * 1e3, 4),
                                "TFLOP/s": round(fl_chunk / t_chunk / 1e12, 2),
                                "frac_mfma": round(fl_chunk / t_chunk / 1e12 / PEAK_BF16_TFLOPS, 4),
                                "algorithmic_gflop": round(fl_chunk / 1e9, 3),
                                "algorithmic_MB": round(by_chunk / 1e6, 2),
                                "traffic": traffic_from_profile("chunked_prefill_8x1024", by_chunk),
                                "timing": "its own loop of --steps calls after the step loop"},
            "backward": {"S": 4096, "Hq": 32, "Hkv": 8, "D": 128, "causal": True, "ms": round(t_bwd * 1e3, 4),
                         "TFLOP/s": round(fl_bwd / t_bwd / 1e12, 2),
                         "frac_mfma": round(fl_bwd / t_bwd / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_gflop": round(fl_bwd / 1e9, 3),
                         "algorithmic_MB": round(by_bwd / 1e6, 2),
                         "traffic": traffic_from_profile("backward_causal_gqa_s4096", by_bwd),
                         "work": "5 products per admissible pair (2.5x the forward)",
                         "timing": "its own loop of --steps calls after the step loop"},
            "varlen_prefill_d256": {"seqlens": [int(x) for x in vc5.seqlens], "Hq": 16, "Hkv": 4, "D": 256,
                                    "causal": True, "ms": round(t_var * 1e3, 4),
                                    "TFLOP/s": round(fl_var / t_var / 1e12, 2),
                                    "frac_mfma": round(fl_var / t_var / 1e12 / PEAK_BF16_TFLOPS, 4),
                                    "algorithmic_gflop": round(fl_var / 1e9, 3),
                                    "algorithmic_MB": round(by_var / 1e6, 2),
                                    "traffic": traffic_from_profile("varlen_prefill_d256", by_var),
                                    "timing": "its own loop of --steps calls after the step loop"},
            "wall_s": round(wall, 4),
        },
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "miattn_prefill_pp_kernel<128, 2, true>",
                     "per_launch_work": f"{fl_pre:.6g} FLOP"},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs_long, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs_long / PEAK_HBM_GBS, 4),
                            "traffic": traffic_from_profile("decode_long_ctx131072", by_long),
                            "kernel": "miattn_decode_split_kernel<256, false, false, false> + miattn_combine_kernel",
                            "per_launch_work": f"{by_long:.6g} B"},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(pc)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
