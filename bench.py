"""Benchmark of the masked-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one pass of the hot path over one batch of synthetic input:
  1. mzattn_fwd_execute on the packed-guidance workload: one row of 2848
     tokens ([2048 conditional | 800 unconditional] segments,
     block-diagonal, positions restarting at 0), Hq 16 / Hkv 8, head_dim
     128, bf16, RoPE base 1e6 on every head: the rotation of K, then the
     attention kernel.  The layout prepasses (mzattn_fwd_plan: RoPE table,
     segment key ranges and positions) depend on the segment ids alone and
     run once before timing, as in a sampling loop over one layout; their
     time is reported beside the step;
  2. mzattn_decode on the static-cache step: batch 2, one query, Hq 16 /
     Hkv 2, head_dim 128, 8192-position cache fully filled (L = 8192), bf16,
     full span, reading one of 32 rotating cache copies so the step sees
     cold HBM (537 MB > the 256 MB Infinity Cache).

Inputs are resident in HBM before timing starts.  Prints one JSON line:
``value`` is the live TFLOP/s of the forward execute (K rotation +
attention) on the packed workload (the headline), timed with HIP events
around the whole execute in the odd timed steps; ``roofline`` that of the
attention kernel alone, timed with an event between the two launches in
the even steps; ``decode`` the static-cache step's HBM GB/s, each against
MI355X's published peaks, and ``cpu_baseline`` the fp64 oracle timed on
the host for full packed-workload calls (with the F5-style layer, the
padded pair and the decode step beside it).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "masked-attn TFLOP/s & % MFMA peak; static-cache decode HBM GB/s & % peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def live_pairs_packed():
    from masked_bidirectional_attention_amd import workloads as W
    return 16 * (W.QWEN_S ** 2 + W.QWEN_UNCOND ** 2)


def fwd_flops():
    """4 * D per live (query, key) pair: 2 for Q.K^T and 2 for P.V."""
    return 4 * 128 * live_pairs_packed()


# live flops of the F5-style layer: B 2 x H 16 x 1500 queries, row 0 sees
# 1500 keys and row 1 1200, 4 * D (64) per live pair
F5_GFLOP = 4 * 64 * 16 * 1500 * (1500 + 1200) / 1e9


def decode_bytes(L=8192, span=8192):
    """K and V rows of the live keys (B 2 x Hkv 2 x L x D 128 x 2 bytes x 2),
    the mask bytes in the span (2 rows), q and o (2 x 16 x 128 x 2 each)."""
    return 2 * 2 * L * 128 * 2 * 2 + 2 * span + 2 * (2 * 16 * 128 * 2)


def kernel_source_hash():
    """Hash of the kernel sources; counter-derived traffic is reported only
    while it matches the hash recorded with the counters."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "masked_bidirectional_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def append_bytes(L):
    """The append step at fill L: K and V rows of the L cached keys and of
    the new one read (B 2 x Hkv 2 x (L + 1) x D 128 x 2 bytes x 2), the new
    K/V rows written, q and o (2 x 16 x 128 x 2 each); no mask."""
    return 2 * 2 * (L + 1) * 128 * 2 * 2 + 2 * 2 * 128 * 2 * 2 + 2 * (2 * 16 * 128 * 2)


COPY_BYTES = 64 * 1024 * 1024


def pmc_workload():
    """A short run for rocprofv3 --pmc: a plain copy of known size (the
    counter calibration), then the forward execute of the timed workload,
    the attention kernel on dense 2048-token rows and the decode step of the
    timed workload, three launches each."""
    import torch
    import masked_bidirectional_attention_amd as mz
    from masked_bidirectional_attention_amd import workloads as W
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    c3 = W.qwen_cfg_packed()
    seg = c3.seg_q.to(dev)
    fwd = mz.FwdCall(c3.q.to(dev), c3.k.to(dev), c3.v.to(dev), seg_q=seg, seg_k=seg, rope_base=c3.rope_base)
    c4 = W.vox_decode(8192)
    dq, dmask = c4.q.to(dev), c4.mask.to(dev)
    copies = [(c4.k_cache.to(dev), c4.v_cache.to(dev)) for _ in range(3)]
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    fwd.plan()
    for _ in range(3):
        fwd.execute()
    torch.cuda.synchronize()
    # dense rows, every work-group the same length (B 2, 2048 tokens, Hq 16
    # / Hkv 8, no mask, no RoPE): the per-step figures without load imbalance
    g = torch.Generator().manual_seed(5)
    qd, kd, vd = (torch.randn(2, h, 2048, 128, generator=g).to(torch.bfloat16).to(dev) for h in (16, 8, 8))
    dense = mz.FwdCall(qd, kd, vd)
    dense.plan()
    for _ in range(3):
        dense.attend()
    torch.cuda.synchronize()
    for kc, vc in copies:
        mz.mzattn_decode(dq, kc, vc, span=8192, mask=dmask, scale=c4.scale)
    torch.cuda.synchronize()
    print("pmc workload done", flush=True)


# (key, kernel-name pattern): the packed workload's attention kernel is the
# segment-kind instance, the dense rows' the no-mask one
TRAFFIC_KERNELS = (("fwd_mfma_kernel", "fwd_mfma_kernel<mz::BF16, 128, 2,"),
                   ("fwd_mfma_kernel_dense", "fwd_mfma_kernel<mz::BF16, 128, 0,"),
                   ("k_rotate16_kernel", "k_rotate16_kernel"),
                   ("decode_mfma_kernel", "decode_mfma_kernel"), ("decode_merge16_kernel", "decode_merge16_kernel"))
SIMDS = 1024  # 256 compute units x 4 SIMDs
XCDS = 8


def _counter_rows(d):
    """(kernel name, counter name, value) of every counter_collection.csv
    row under a rocprofv3 output directory (one row per dispatch and
    counter)."""
    import csv
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    for r in csv.DictReader(f):
                        yield r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])


def counters_from(d):
    """Per-dispatch means of the counters of one rocprofv3 --pmc run of
    pmc_workload, per kernel of the timed path, with the MFMA busy share
    (MFMA-busy SIMD cycles over GPU-active cycles times the SIMD count), the
    LDS bank-conflict share of LDS-active cycles, and the flop the MFMA ops
    counter implies (512 per op)."""
    acc = {}
    for kname, cname, v in _counter_rows(d):
        for key, pat in TRAFFIC_KERNELS:
            if pat in kname:
                acc.setdefault(key, {}).setdefault(cname, []).append(v)
    # launch durations of the same run (its kernel trace)
    import csv
    dur = {}
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("kernel_trace.csv"):
                with open(os.path.join(root, fn)) as f:
                    for r in csv.DictReader(f):
                        for key, pat in TRAFFIC_KERNELS:
                            if pat in r["Kernel_Name"]:
                                dur.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {"source_hash": kernel_source_hash(), "xcds": XCDS, "simds": SIMDS}
    for key, cs in acc.items():
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        e = {c: round(v, 1) for c, v in m.items()}
        e["dispatches"] = max(len(v) for v in cs.values())
        if dur.get(key):
            e["avg_duration_us"] = round(sum(dur[key]) / len(dur[key]) / 1e3, 2)
        # GRBM_GUI_ACTIVE comes summed over the XCDs: per-XCD active cycles
        gui = m.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        if gui and dur.get(key):
            e["gui_cycles_per_ns"] = round(gui / (sum(dur[key]) / len(dur[key])), 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and gui:
            e["mfma_busy_pct"] = round(100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS), 2)
        if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_LDS_IDX_ACTIVE"):
            e["lds_bank_conflict_pct"] = round(100.0 * m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"], 3)
        mops = sum(m.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16"))
        if mops:
            e["mfma_gflop"] = round(mops * 512 / 1e9, 3)
        out[key] = e
    return out


def traffic_from(fetch_dir, write_dir):
    """HBM bytes per launch from two rocprofv3 --pmc runs of pmc_workload
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each divided by the
    factor the same counter shows for the copy kernel of known size."""
    def per_kernel(d, counter):
        vals = {}
        for kname, cname, v in _counter_rows(d):
            if cname == counter:
                vals.setdefault(kname, []).append(v)
        return vals

    out = {"source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copy = [v for k, vs in vals.items() if "copy" in k.lower() or "elementwise" in k.lower() for v in vs]
        if not copy:
            raise SystemExit(f"no copy kernel found for {counter} in {d}")
        factor = max(copy) * 1024.0 / COPY_BYTES
        out[counter.lower() + "_factor"] = round(factor, 4)
        for key, pat in TRAFFIC_KERNELS:
            vs = [v for k, v_ in vals.items() if pat in k for v in v_]
            if vs:
                out.setdefault(key, {})[counter.lower() + "_bytes"] = round(sum(vs) / len(vs) * 1024.0 / factor)
    for key, _ in TRAFFIC_KERNELS:
        if key in out and "fetch_size_bytes" in out[key] and "write_size_bytes" in out[key]:
            out[key]["bytes"] = out[key]["fetch_size_bytes"] + out[key]["write_size_bytes"]
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The fp64 numpy oracle (never tuned for speed) on the host, on a
    bounded sample of the packed-guidance workload: the full forward with
    every BLAS thread (nproc) and a 2-head slice single-threaded, each the
    median of 3 timed runs, scaled to live TFLOP/s; and the other
    configurations (F5-style layer, padded pair, decode step at L 8192)
    whole with every thread, median of 3, in s per call."""
    import statistics
    import threadpoolctl
    from masked_bidirectional_attention_amd import workloads as W
    from oracle import mzref

    c = W.qwen_cfg_packed()
    bq, bk, bv = W.to_bits(c.q), W.to_bits(c.k), W.to_bits(c.v)
    seg = c.seg_q.numpy()

    def run(heads):
        t0 = time.perf_counter()
        mzref.mzref_fwd(c.dtype, bq, bk, bv, rope_base=c.rope_base, mask_kind="segment", seg_q=seg, seg_k=seg,
                        heads=heads)
        return time.perf_counter() - t0

    nproc = os.cpu_count() or 1
    with threadpoolctl.threadpool_limits(limits=nproc, user_api="blas"):
        threads = max([i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                       if i.get("user_api") == "blas"] or [nproc])
        multi = statistics.median(run(None) for _ in range(3))
    sub = [0, 9]   # one head of each K/V pair kind: heads 0 and 9 read K/V heads 0 and 4
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
        single = statistics.median(run(sub) for _ in range(3))
    f_full = fwd_flops()
    f_sub = f_full * len(sub) / 16
    # the other configurations, whole, with every BLAS thread, median of 3
    others = {}
    with threadpoolctl.threadpool_limits(limits=nproc, user_api="blas"):
        c1 = W.f5_dit_layer()
        c2 = W.qwen_cfg_padded()
        for name, cf, gflop in (("f5_dit_layer", c1, F5_GFLOP), ("qwen_padded", c2, fwd_flops() / 1e9)):
            args = (cf.dtype, W.to_bits(cf.q), W.to_bits(cf.k), W.to_bits(cf.v))
            kw = dict(scale=cf.scale, rope_base=cf.rope_base, pe_attn_head=cf.pe_attn_head, mask_kind=cf.mask_kind,
                      mask=cf.mask.numpy())

            def run_cfg():
                t0 = time.perf_counter()
                mzref.mzref_fwd(*args, **kw)
                return time.perf_counter() - t0
            sec = statistics.median(run_cfg() for _ in range(3))
            others[name] = {"s_per_call": round(sec, 3), "TFLOP/s": round(gflop / sec / 1e3, 4)}
        c4 = W.vox_decode(8192)
        dargs = (c4.dtype, W.to_bits(c4.q), W.to_bits(c4.k_cache), W.to_bits(c4.v_cache))

        def run_dec():
            t0 = time.perf_counter()
            mzref.mzref_decode(*dargs, span=8192, mask=c4.mask.numpy(), scale=c4.scale)
            return time.perf_counter() - t0
        sec = statistics.median(run_dec() for _ in range(3))
        others["vox_decode_L8192"] = {"s_per_call": round(sec, 4), "GB/s": round(decode_bytes() / sec / 1e9, 2)}
    return {
        "value": f_full / multi / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"packed-guidance forward (16 heads, 2848 tokens, {f_full / 1e9:.2f} live GFLOP) through the fp64 "
                  f"numpy oracle with {threads} BLAS threads: median of 3 runs {multi:.2f} s",
        "single_thread": {"value": f_sub / single / 1e12, "unit": "TFLOP/s", "cores": 1,
                          "sample": f"heads {sub} of the same forward ({f_sub / 1e9:.2f} live GFLOP), one BLAS "
                                    f"thread: median of 3 runs {single:.2f} s"},
        "other_configs": others,
        "nproc": nproc,
        "cpu_model": _cpu_model(),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cache-copies", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM traffic per launch (from rocprofv3 --pmc), if present")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run the short counter workload (under rocprofv3 --pmc) and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output dirs into traffic JSON on stdout and exit")
    ap.add_argument("--counters-from", metavar="PMC_DIR",
                    help="per-kernel counter means of one rocprofv3 --pmc output dir as JSON on stdout, and exit")
    a = ap.parse_args(argv)
    if a.traffic_from:
        print(json.dumps(traffic_from(*a.traffic_from), indent=1))
        return 0
    if a.counters_from:
        print(json.dumps(counters_from(a.counters_from), indent=1))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    if a.pmc_workload:
        pmc_workload()
        return 0

    import torch
    import masked_bidirectional_attention_amd as mz
    from masked_bidirectional_attention_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    info = mz.mzattn_device_info(0)

    # ---- inputs resident in HBM
    c3 = W.qwen_cfg_packed()
    fq, fk, fv = c3.q.to(dev), c3.k.to(dev), c3.v.to(dev)
    seg = c3.seg_q.to(dev)
    fwd = mz.FwdCall(fq, fk, fv, seg_q=seg, seg_k=seg, rope_base=c3.rope_base)

    c4 = W.vox_decode(8192)
    dq, dmask = c4.q.to(dev), c4.mask.to(dev)
    kc0, vc0 = c4.k_cache.to(dev), c4.v_cache.to(dev)
    copies = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(max(0, a.cache_copies - 1))]
    dec = mz.DecodeCall(dq, kc0, vc0, span=8192, mask=dmask, scale=c4.scale)
    torch.cuda.synchronize()
    print(f"[bench] device {props.name} {info['arch']}, {info['compute_units']} CUs, peak engine clock "
          f"{info['clock_mhz']:.0f} MHz; inputs resident", file=sys.stderr, flush=True)

    # the layout prepasses, once (they depend on the segment ids alone)
    fwd.plan()

    # Timed steps alternate: in even steps an event between the K pass and
    # the attention kernel times the attention kernel alone (the roofline
    # figure); in odd steps nothing sits between the two launches, which
    # times the execute as a sampling loop runs it (an event between two
    # launches holds the second until the first has drained: several us).
    def step(i, evs=None, split=False):
        if evs:
            evs[0].record()
        fwd.rotate_k()
        if evs and split:
            evs[1].record()
        fwd.attend()
        if evs:
            evs[2].record()
        dec.set_cache(*copies[i % len(copies)])
        dec()
        if evs:
            evs[3].record()

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup {a.warmup} steps done", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, evs[i], split=i % 2 == 0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    split_evs = evs[0::2]
    whole_evs = evs[1::2] or split_evs
    rot_ms = sum(e[0].elapsed_time(e[1]) for e in split_evs) / len(split_evs)
    att_ms = sum(e[1].elapsed_time(e[2]) for e in split_evs) / len(split_evs)
    exe_split_ms = sum(e[0].elapsed_time(e[2]) for e in split_evs) / len(split_evs)
    exe_ms = sum(e[0].elapsed_time(e[2]) for e in whole_evs) / len(whole_evs)
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / a.steps
    # the execute without an event between its two launches (100 back to
    # back), reported beside the timed region's
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(100):
        fwd.execute()
    e1.record()
    torch.cuda.synchronize()
    exe_b2b_ms = e0.elapsed_time(e1) / 100
    # the attention kernel alone, 100 launches back to back: the dispatch of
    # each overlaps the end of the one before, so this is the figure to set
    # beside the kernel trace's average duration (the events around one
    # launch in the timed steps also hold its dispatch)
    e0.record()
    for _ in range(100):
        fwd.attend()
    e1.record()
    torch.cuda.synchronize()
    att_b2b_ms = e0.elapsed_time(e1) / 100
    print(f"[bench] timed {a.steps} steps: {wall / a.steps * 1e3:.3f} ms/step, forward execute "
          f"{exe_ms * 1e3:.1f} us ({exe_split_ms * 1e3:.1f} with an event between: K rotation {rot_ms * 1e3:.1f}, "
          f"attention kernel {att_ms * 1e3:.1f}; {exe_b2b_ms * 1e3:.1f} back to back), decode {dec_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    # the layout prepasses, timed apart
    torch.cuda.synchronize()
    e0.record()
    for _ in range(50):
        fwd.plan()
    e1.record()
    torch.cuda.synchronize()
    plan_us = e0.elapsed_time(e1) / 50 * 1e3

    tflops = fwd_flops() / (exe_ms * 1e-3) / 1e12
    att_tflops = fwd_flops() / (att_ms * 1e-3) / 1e12
    gbs = decode_bytes() / (dec_ms * 1e-3) / 1e9

    # ---- the decode step at other cache fills (reported, not the headline):
    # the same cold cache copies under the mask of fill L, at the full span
    # and at the span rounded up to 256
    by_fill = []
    for L in (257, 1024, 3100, 8192):
        mask_l = torch.zeros_like(dmask)
        mask_l[..., :L] = True
        for span in sorted({8192, W.ceil256(L)}, reverse=True):
            # eager (events around each call, host launch included) and as a
            # replayed graph of 8 calls over 8 cold cache copies (GPU time)
            dl = mz.DecodeCall(dq, kc0, vc0, span=span, mask=mask_l, scale=c4.scale)
            n = 50
            for i in range(5):
                dl.set_cache(*copies[i % len(copies)])
                dl()
            torch.cuda.synchronize()
            tot = 0.0
            for i in range(n):
                dl.set_cache(*copies[i % len(copies)])
                e0.record()
                dl()
                e1.record()
                torch.cuda.synchronize()
                tot += e0.elapsed_time(e1)
            us = tot / n * 1e3
            gs = torch.cuda.Stream()
            gcalls = [mz.DecodeCall(dq, kc, vc, span=span, mask=mask_l, scale=c4.scale, stream=gs)
                      for kc, vc in copies[:8]]
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                for c_ in gcalls:
                    c_()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(6):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            gus = e0.elapsed_time(e1) / (6 * 8) * 1e3
            del g
            by_fill.append({"fill": L, "span": span, "us": round(us, 2), "graph_us": round(gus, 2),
                            "GB/s": round(decode_bytes(L, span) / (us * 1e-6) / 1e9, 1),
                            "GB/s_graph": round(decode_bytes(L, span) / (gus * 1e-6) / 1e9, 1),
                            "algorithmic_mb": round(decode_bytes(L, span) / 1e6, 3)})
    # ---- what one launch that moves the decode step's bytes costs here: a
    # plain device copy of half of them (8.4 MB read, 8.4 MB written) from 32
    # rotating cold sources, eager (events around each launch) and as a
    # replayed graph of 8 copies; the decode step is two dependent launches
    half = decode_bytes() // 2 // 2
    fsrc = [torch.empty(half, dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(32)]
    fdst = torch.empty(half, dtype=torch.bfloat16, device=dev)
    for i in range(5):
        fdst.copy_(fsrc[i])
    torch.cuda.synchronize()
    tot = 0.0
    nfl = 64
    for i in range(nfl):
        e0.record()
        fdst.copy_(fsrc[i % 32])
        e1.record()
        torch.cuda.synchronize()
        tot += e0.elapsed_time(e1)
    floor_us = tot / nfl * 1e3
    gs = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for i in range(8):
            fdst.copy_(fsrc[8 + i])
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(6):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    floor_graph_us = e0.elapsed_time(e1) / (6 * 8) * 1e3
    del g, fsrc, fdst
    floor = {"what": "one torch device copy moving the decode step's 16.81 MB (half read, half written), "
                     "cold sources; the decode step itself is two dependent launches",
             "us": round(floor_us, 2), "graph_us": round(floor_graph_us, 2),
             "GB/s": round(decode_bytes() / (floor_us * 1e-6) / 1e9, 1),
             "GB/s_graph": round(decode_bytes() / (floor_graph_us * 1e-6) / 1e9, 1)}

    # ---- causal prefill (reported, not the headline): the same kernel under
    # the causal kind, K rotation + attention per call, layout planned once
    cp = W.vox_prefill_causal()
    cpf = mz.FwdCall(cp.q.to(dev), cp.k.to(dev), cp.v.to(dev), causal=True, rope_base=cp.rope_base,
                     scale=cp.scale)
    cpf.plan()
    for _ in range(5):
        cpf.execute()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(50):
        cpf.execute()
    e1.record()
    torch.cuda.synchronize()
    cp_us = e0.elapsed_time(e1) / 50 * 1e3
    B_, Hq_, S_ = cp.q.shape[0], cp.q.shape[1], cp.q.shape[2]
    cp_gflop = 4 * 128 * B_ * Hq_ * S_ * (S_ + 1) / 2 / 1e9
    causal = {"workload": f"causal prefill: B {B_}, {S_} tokens, Hq 16 / Hkv 2, D 128, bf16, RoPE base 1e4",
              "execute_us": round(cp_us, 2), "live_gflop": round(cp_gflop, 3),
              "TFLOP/s": round(cp_gflop / cp_us * 1e3, 1),
              "frac": round(cp_gflop / cp_us * 1e3 / PEAK_BF16_TFLOPS, 4)}

    # ---- the other two forward workloads of the configuration list
    # (reported beside the headline): the F5-style DiT layer (fp16, D 64,
    # RoPE on head 0 only, row 1's last 300 keys masked) and the padded
    # Qwen-shaped CFG pair (bf16, materialized 4-D bool mask).  Execute =
    # K pass + attention kernel, layout planned once; attention_us: the
    # attention kernel alone (events around back-to-back launches).
    def time_fwd(case, gflop, peak, n=50):
        kw = dict(scale=case.scale, rope_base=case.rope_base, pe_attn_head=case.pe_attn_head)
        if case.mask_kind == W.MASK_BOOL:
            kw["mask"] = case.mask.to(dev)
        call = mz.FwdCall(case.q.to(dev), case.k.to(dev), case.v.to(dev), **kw)
        call.plan()
        for _ in range(5):
            call.execute()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            call.execute()
        e1.record()
        torch.cuda.synchronize()
        exe = e0.elapsed_time(e1) / n * 1e3
        call.rotate_k()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            call.attend()
        e1.record()
        torch.cuda.synchronize()
        att = e0.elapsed_time(e1) / n * 1e3
        return {"execute_us": round(exe, 2), "attention_us": round(att, 2), "live_gflop": round(gflop, 3),
                "TFLOP/s": round(gflop / exe * 1e3, 1), "frac": round(gflop / exe * 1e3 / peak, 4),
                "attention_TFLOP/s": round(gflop / att * 1e3, 1),
                "attention_frac": round(gflop / att * 1e3 / peak, 4)}

    f5 = W.f5_dit_layer()
    f5_gflop = F5_GFLOP
    other_fwd = {
        "f5_dit_layer": {"workload": "F5-style DiT layer: B 2 (CFG), H 16, S 1500, D 64, fp16, RoPE base 1e4 on "
                                     "head 0 only, row 1 keys 1200-1499 masked ([2,1,1,1500] bool)",
                         **time_fwd(f5, f5_gflop, PEAK_BF16_TFLOPS)},
        "qwen_padded": {"workload": "padded Qwen-shaped CFG pair: B 2, S 2048, Hq 16 / Hkv 8, D 128, bf16, RoPE "
                                    "base 1e6, [2,1,2048,2048] bool mask (row 1: 800 x 800 live)",
                        **time_fwd(W.qwen_cfg_padded(), fwd_flops() / 1e9, PEAK_BF16_TFLOPS)},
    }

    # ---- the packed workload with q / k RMSNorm before RoPE (reported, not
    # the headline): execute = K pass (normalise + rotate) + attention kernel
    gen_n = torch.Generator().manual_seed(3)
    wq = (1.0 + 0.1 * torch.randn(128, generator=gen_n)).to(torch.bfloat16).to(dev)
    wk = (1.0 + 0.1 * torch.randn(128, generator=gen_n)).to(torch.bfloat16).to(dev)
    fn = mz.FwdCall(fq, fk, fv, seg_q=seg, seg_k=seg, rope_base=c3.rope_base, q_norm_weight=wq, k_norm_weight=wk)
    fn.plan()
    for _ in range(5):
        fn.execute()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(50):
        fn.execute()
    e1.record()
    torch.cuda.synchronize()
    norm_us = e0.elapsed_time(e1) / 50 * 1e3
    qk_norm = {"workload": "packed-guidance workload with q / k RMSNorm before RoPE", "execute_us": round(norm_us, 2),
               "TFLOP/s": round(fwd_flops() / (norm_us * 1e-6) / 1e12, 1)}

    # ---- short bidirectional sequences (reported, not the headline): the
    # latency of one forward execute (K rotation + attention) for a CFG
    # pair, Hq 16 / Hkv 2, D 128, bf16, RoPE, no mask, the shape class of a
    # local DiT / encoder step run many times per generated patch
    short = []
    for S in (16, 64, 128, 256):
        gs_ = torch.Generator().manual_seed(S)
        sq = torch.randn(2, 16, S, 128, generator=gs_).to(torch.bfloat16).to(dev)
        sk = torch.randn(2, 2, S, 128, generator=gs_).to(torch.bfloat16).to(dev)
        sv = torch.randn(2, 2, S, 128, generator=gs_).to(torch.bfloat16).to(dev)
        sc_ = mz.FwdCall(sq, sk, sv, rope_base=1e4)
        sc_.plan()
        for _ in range(10):
            sc_.execute()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(100):
            sc_.execute()
        e1.record()
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) / 100 * 1e3
        # the same execute recorded 20 times in one graph (GPU time without
        # the host's launch path)
        gs = torch.cuda.Stream()
        gc_ = mz.FwdCall(sq, sk, sv, rope_base=1e4, stream=gs)
        with torch.cuda.stream(gs):
            gc_.plan()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for _ in range(20):
                gc_.execute()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) / 200 * 1e3
        del g
        short.append({"seq": S, "execute_us": round(eager, 2), "graph_us": round(graph_us, 2),
                      "launches": 1 if S <= 64 else 2})

    # ---- the append step (reported, not the headline): the static-cache
    # step that reads the filled length on the device, rotates q and the new
    # key, writes the new K/V rows into the cache and attends keys
    # j <= len; eagerly and as a replayed HIP graph.  The cache copies rotate
    # as above; the length stays fixed so every call writes the same rows.
    gen = torch.Generator().manual_seed(4)
    aq = torch.randn(2, 16, 1, 128, generator=gen).to(torch.bfloat16).to(dev)
    akn = torch.randn(2, 2, 1, 128, generator=gen).to(torch.bfloat16).to(dev)
    avn = torch.randn(2, 2, 1, 128, generator=gen).to(torch.bfloat16).to(dev)
    append = []
    for L in (256, 1023, 3099, 8191):
        length = torch.full((2,), L, dtype=torch.int32, device=dev)
        calls = [mz.DecodeAppendCall(aq, akn, avn, kc, vc, length, rope_base=1e4, scale=c4.scale)
                 for kc, vc in copies[:8]]
        for i in range(16):
            calls[i % 8]()
        torch.cuda.synchronize()
        n = 48
        tot = 0.0
        for i in range(n):
            e0.record()
            calls[i % 8]()
            e1.record()
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        eager_us = tot / n * 1e3
        # the same step as a graph: 8 steps (one per cache copy) per replay
        gs = torch.cuda.Stream()
        gcalls = [mz.DecodeAppendCall(aq, akn, avn, kc, vc, length, rope_base=1e4, scale=c4.scale, stream=gs)
                  for kc, vc in copies[:8]]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for c_ in gcalls:
                c_()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(6):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) / (6 * 8) * 1e3
        nbytes = append_bytes(L)
        append.append({"filled": L, "eager_us": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
                       "GB/s_graph": round(nbytes / (graph_us * 1e-6) / 1e9, 1),
                       "algorithmic_mb": round(nbytes / 1e6, 3)})
        del g

    traffic = {}
    if os.path.exists(a.traffic):
        with open(a.traffic) as f:
            traffic = json.load(f)
        if traffic.get("source_hash") != kernel_source_hash():
            traffic = {}  # the kernels changed since the counters were taken
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "packed-guidance bidirectional attention: 1 row x 2848 tokens "
                        "[2048 cond | 800 uncond] block-diagonal, Hq 16 / Hkv 8, D 128, RoPE base 1e6",
            "decode_workload": "static-cache step: B 2, 1 query, Hq 16 / Hkv 2, D 128, "
                               "cache 8192 filled 8192, full span, 32 rotating cache copies (cold HBM)",
            "global_batch": 1,
            "seq_len": 2848,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "fwd_mfma_kernel<bf16,128>",
            "bound": "mfma",
            "achieved": round(att_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": (traffic.get("fwd_mfma_kernel") or {}).get("bytes"),
            "kernel_us": round(att_ms * 1e3, 2),
            "algorithmic_gflop": round(fwd_flops() / 1e9, 3),
        },
        "forward": {
            "execute_us": round(exe_ms * 1e3, 2),
            "execute_us_with_event_between": round(exe_split_ms * 1e3, 2),
            "k_rotation_us": round(rot_ms * 1e3, 2),
            "attention_us": round(att_ms * 1e3, 2),
            "execute_us_back_to_back": round(exe_b2b_ms * 1e3, 2),
            "attention_us_back_to_back": round(att_b2b_ms * 1e3, 2),
            "plan_us_once_per_layout": round(plan_us, 2),
        },
        "decode": {
            "value": round(gbs, 1),
            "unit": "GB/s",
            "roofline": {
                "kernel": "whole decode call: decode_mfma_kernel<bf16,128,1> + decode_merge16_kernel<bf16,128>",
                "bound": "hbm",
                "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": (traffic.get("decode_mfma_kernel") or {}).get("bytes"),
                "kernel_us": round(dec_ms * 1e3, 2),
                "algorithmic_mb": round(decode_bytes() / 1e6, 3),
            },
            "by_fill": by_fill,
            "one_launch_copy_floor": floor,
        },
        "other_forward": other_fwd,
        "causal_prefill": causal,
        "qk_norm": qk_norm,
        "short_bidirectional": {"workload": "B 2 (CFG), Hq 16 / Hkv 2, D 128, bf16, RoPE base 1e4, no mask; "
                                            "execute_us: events around 100 eager executes (host launch path "
                                            "included); graph_us: 20 executes replayed as one graph",
                                "by_seq": short},
        "decode_append": {"workload": "append step: B 2, 1 new token, Hq 16 / Hkv 2, D 128, bf16, cache 8192, "
                                      "length on the device, RoPE base 1e4 on q and the new key",
                          "by_fill": append},
        "device": {"name": props.name, "arch": info["arch"], "compute_units": info["compute_units"],
                   "peak_engine_clock_mhz": info["clock_mhz"], "memory_clock_mhz": info["mem_clock_mhz"]},
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
