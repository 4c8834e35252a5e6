#!/usr/bin/env python3
"""Benchmark of the int4 group-quantized decode GEMM on one MI355X.

One step is one pass of the whole hot path over the 70B-class MLP
up-projection (K=8192, N=28672, 4-bit codes, group 128 along K):
    wq_gemm(X[B], codes) for B = 1, 2, 4, 8, 16, 32, 64   decode-step products
    wq_quantize_pack(W)                      fp16 weights -> codes + fp16 headers
Each kernel works on its own copy from a pool of packed weights larger than
1 GiB (two fp16 weight copies for the quantizer), so no call finds its inputs
in the 256 MB Infinity Cache or the L2: every call streams from HBM.  Inputs
are resident in HBM before timing starts.

Printed: one JSON line whose value is the metric, the products' algorithmic
bytes per second over B = 1..64 (GB/s, timed inside the K timed steps with
events on the library's stream); the quantizer as its own kernel entry; the
roofline of the dominant product with its duration measured by HIP events on
the stream it runs on; every kernel's fraction of the vendor peak and of the
read rate the load-only probe measured; and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--steps 20] [--warmup 5] [--no-cpu]
    python bench.py --workload gemv_k896_n4864_g32 | mlp7b_up_k4096_n11008_g128   # other configs (table lines)
    python bench.py --sweep        # batch sweep across the ridge (K=N=8192), table only
    python bench.py --decode-set   # 7B-class decode step (224 products, B=32), table only
    python bench.py --kv           # decode attention over an int4 KV cache, table only
    python bench.py --ceiling      # load-only probe read rates (and plain torch rates), table only
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for int4 group-quant decode GEMM at B=1..64"
WORKLOAD = "mlp70b_up_k8192_n28672_g128"
METRIC_BATCHES = (1, 2, 4, 8, 16, 32, 64)   # the metric's batch range on the headline workload
POOL_BYTES = 1 << 30          # packed-weight pool, >= 4x the 256 MB Infinity Cache


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=WORKLOAD)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--sweep", action="store_true", help="batch sweep on K=N=8192 (table)")
    p.add_argument("--decode-set", action="store_true",
                   help="7B-class decode step, 224 products at B=32 (table)")
    p.add_argument("--kv", action="store_true",
                   help="decode attention over an int4 KV cache, 1024 heads x 4096 tokens "
                        "(a 7B-class model's whole cache; table line)")
    p.add_argument("--format", choices=["nf4", "offset"], default=None,
                   help="another weight format on the step's workload: NF4 at blocks of 64, or "
                        "the float-offset variant at the workload's group and --bits; quantize + "
                        "product at --batches (default 1) (table line)")
    p.add_argument("--ceiling", action="store_true",
                   help="what plain torch kernels read and copy on this GPU over 1 GiB buffers "
                        "(context for the roofline fractions; table line)")
    p.add_argument("--path", default="auto", choices=["auto", "gemv", "mfma"])
    p.add_argument("--bits", type=int, default=0,
                   help="code width of the step (default: the workload's, 4); 2 and 3 take "
                        "the bit-stream GEMV at B = 1 and past 32, the matrix cores between")
    p.add_argument("--batches", default="",
                   help="comma-separated batch sizes of the step (default: the workload's)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after timing, copy this many MiB device-to-device once (a "
                        "known-size kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc counter CSVs into profiles/traffic_*.txt "
                        "(with --copy-calibration-mib as used in those runs)")
    p.add_argument("--traffic-match", nargs=2, action="append", metavar=("TAG_SUFFIX", "NAME_FRAGMENT"),
                   help="write the summary of wq_gemm_b<TAG_SUFFIX> (or wq_quantize_pack) from "
                        "the kernel whose name holds NAME_FRAGMENT")
    p.add_argument("--fetch-cmd", default="", help="command line of the FETCH_SIZE run (recorded)")
    p.add_argument("--write-cmd", default="", help="command line of the WRITE_SIZE run (recorded)")
    return p.parse_args()


def kernel_entry(name, nbytes, flops, ms_list, bound="hbm"):
    from bit_weight_only_wq_amd import roofline as rl
    ms = sum(ms_list) / len(ms_list)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    e = {"kernel": name, "avg_us": round(ms * 1e3, 3), "bytes": int(nbytes),
         "achieved_GBps": round(gbs, 1), "frac_hbm": round(gbs * 1e9 / rl.MI355X_HBM_BYTES_PER_S, 4)}
    if flops:
        e["TFLOPs"] = round(tflops, 2)
        e["frac_mfma_f16"] = round(tflops * 1e12 / rl.MI355X_FP16_MFMA_FLOPS, 4)
    e["bound"] = bound
    return e


# Sources each kernel family is built from: a traffic summary stays valid only
# while these files are unchanged.
KERNEL_SOURCES = {
    "gemv": ["wq_gemv.hip", "wq_device.h"],
    "mfma": ["wq_gemm_mfma.hip", "wq_mfma_dq.h", "wq_device.h"],
    "xr": ["wq_gemm_xr.hip", "wq_device.h"],
    "qs": ["wq_gemm_qs.hip", "wq_device.h"],
    "q4": ["wq_gemm_q4.hip", "wq_device.h"],
    "ts": ["wq_gemm_ts.hip", "wq_device.h"],
    "sk": ["wq_gemm_sk.hip", "wq_device.h"],
    "kw": ["wq_gemm_kw.hip", "wq_mfma_dq.h", "wq_nf4_levels.h", "wq_device.h"],
    "quantize": ["wq_quantize.hip", "wq_device.h"],
    "kv_attn": ["wq_kv.hip", "wq_device.h"],
    "kv_quantize": ["wq_kv.hip", "wq_device.h"],
}
KV_WORKLOAD = "kv_decode_7b_ctx4096"
KV_SHAPE = (1024, 4096, 128, 128)   # heads (32 layers x 32), tokens, head dim, block
# rocprofv3 kernel-name fragment of each family.
KERNEL_NAMES = {"gemv": "gemv_", "mfma": "gemm_mfma_kernel", "xr": "gemm_xr_kernel", "qs": "gemm_qs_kernel",
                "q4": "gemm_q4_kernel", "ts": "gemm_ts_kernel", "sk": "gemm_sk_kernel", "kw": "gemm_kw_kernel",
                "quantize": "quantize_"}


def sources_sha256(files):
    import hashlib
    src = os.path.join(ROOT, "bit_weight_only_wq_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode() + b"\0")
        h.update(open(os.path.join(src, f), "rb").read())
    return h.hexdigest()


def traffic_path(kernel_tag):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")


def read_traffic(kernel_tag):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current sources of that kernel (else None)."""
    path = traffic_path(kernel_tag)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    files = vals.get("sources", "").split()
    if not files or vals.get("sources_sha256") != sources_sha256(files):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_mfma_counters(workload, path=None):
    """Per batch size, the matrix-core busy share of the product kernel from a
    committed rocprofv3 counter summary, if it was taken on the current
    sources of those kernels (else {})."""
    import re
    path = path or os.path.join(ROOT, "profiles", f"mfma_counters_wq_gemm_{workload}.txt")
    if not os.path.exists(path):
        return {}
    files, sha, cur, out = [], None, None, {}
    for line in open(path):
        if line.startswith("sources:"):
            files = line.split(":", 1)[1].split()
        elif line.startswith("sources_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith("["):
            m = re.search(r"B = ([0-9, ]+), grid", line)
            cur = [int(v) for v in m.group(1).split(",")] if m else None
        elif "mfma_busy_frac:" in line and cur:
            frac = float(line.rsplit("mfma_busy_frac:", 1)[1].split()[0])
            for B in cur:
                out[B] = frac
    if not files or sha != sources_sha256(files):
        return {}
    return out


def traffic_from(fetch_csv, write_csv, copy_mib):
    """Per-launch HBM bytes of each wq kernel from two rocprofv3 --pmc CSVs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for the calibration kernel, an elementwise pass that reads
    and writes copy_mib MiB: factor = known bytes / counted bytes.
    """
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals[(r["Kernel_Name"], r["Grid_Size"])].append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in vals.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    known = copy_mib * (1 << 20)

    def calib(vals):
        # The calibration kernel: torch's elementwise multiply (not a fill).
        cands = [v for k, v in vals.items() if "wq::" not in k[0] and "Unary" in k[0]]
        return known / max(cands) if cands and max(cands) > 0 else None

    fr, wr = calib(fetch), calib(write)
    if fr is None or wr is None:
        raise SystemExit("calibration kernel not found in the counter CSVs")
    out = {}
    for key in set(fetch) | set(write):
        if "wq::" in key[0]:
            out[key] = (fetch.get(key, 0.0) * fr, write.get(key, 0.0) * wr)
    return out, fr, wr


def write_summary(args, tag, workload, fam, name, f, w, fr, wr, algo):
    path = traffic_path(f"{tag}_{workload}")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic per launch of {tag} on {workload}\n")
        fh.write(f"# kernel: {name}\n")
        fh.write(f"# fetch: {args.fetch_cmd}\n# write: {args.write_cmd}\n")
        fh.write("# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over launches) "
                 "scaled by known/counted bytes of a torch elementwise multiply "
                 f"over {args.copy_calibration_mib} MiB\n")
        fh.write(f"fetch_scale: {fr:.6f}\nwrite_scale: {wr:.6f}\n")
        fh.write(f"fetch_bytes_per_launch: {f:.0f}\nwrite_bytes_per_launch: {w:.0f}\n")
        fh.write(f"hbm_bytes_per_launch: {f + w:.0f}\n")
        fh.write(f"algorithmic_bytes_per_launch: {algo}\n")
        fh.write(f"traffic_over_algorithmic: {(f + w) / algo:.4f}\n")
        fh.write(f"sources: {' '.join(KERNEL_SOURCES[fam])}\n")
        fh.write(f"sources_sha256: {sources_sha256(KERNEL_SOURCES[fam])}\n")
    print("wrote", os.path.relpath(path, ROOT))


def write_traffic_summaries(args):
    """Print every wq kernel's calibrated traffic and write one summary file
    per kernel family and grid size under profiles/."""
    import bit_weight_only_wq_amd.roofline as rl
    import wq_inputs
    out, fr, wr = traffic_from(args.traffic_from[0], args.traffic_from[1], args.copy_calibration_mib)
    if args.kv:
        H, T, D, G = KV_SHAPE
        for (name, grid), (f, w) in sorted(out.items()):
            print(f"{name[:100]} grid={grid}: fetch {f / 1e6:.2f} MB, write {w / 1e6:.2f} MB")
            if "kv_attn_kernel" in name:
                write_summary(args, "wq_kv_attention", KV_WORKLOAD, "kv_attn", name, f, w, fr, wr,
                              rl.kv_attention_bytes(H, T, D))
            elif "kv_quantize_kernel" in name:
                write_summary(args, "wq_kv_quantize_block", KV_WORKLOAD, "kv_quantize", name, f, w, fr, wr,
                              rl.kv_append_bytes(H, G, D))
        return
    cfg = wq_inputs.WORKLOADS[args.workload]
    N, K, G, bits = cfg["N"], cfg["K"], cfg["group"], cfg["bits"]
    batches = [b for b in cfg["batches"] if b <= 64] or [1]
    for (name, grid), (f, w) in sorted(out.items()):
        print(f"{name[:100]} grid={grid}: fetch {f / 1e6:.2f} MB, write {w / 1e6:.2f} MB")
    for fam, frag in KERNEL_NAMES.items():
        hits = [(k, v) for k, v in out.items() if frag in k[0]]
        if fam == "quantize":
            tags = [("wq_quantize_pack", rl.quantize_bytes(N, K, G, bits))]
        else:
            tags = [(f"wq_gemm_b{B}", rl.gemm_bytes(B, N, K, G, bits)) for B in batches]
        for tag, algo in tags:
            # A family's launches at one batch size share one kernel instance;
            # match the summary to a batch by the kernel name's batch tile.
            for (name, grid), (f, w) in hits:
                if not args.traffic_match or not any(m in name and tag.endswith(t)
                                                     for t, m in args.traffic_match):
                    continue
                write_summary(args, tag, args.workload, fam, name, f, w, fr, wr, algo)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(name, batches, bits=0):
    """The oracle as it stands, timed on this host: quantize/pack and the
    double-precision product (at every batch of the step), each on a row
    sample of the workload, on all the cores the process may use and on one.
    Rates are algorithmic GB/s of the sample (the unit of `value`); `value`
    is the product's rate on all cores."""
    import oracle
    import wq_inputs
    from bit_weight_only_wq_amd import roofline as rl
    cfg = wq_inputs.WORKLOADS[name]
    K, G = cfg["K"], cfg["group"]
    bits = bits or cfg["bits"]
    oracle.build(force=False)
    all_cores = len(os.sched_getaffinity(0))

    def timed(fn, min_s):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return dt / reps, reps

    out = {}
    # Sample sizes keep each of the four timings to a few seconds.
    plan = {"all": (all_cores, min(cfg["N"], 8192), min(cfg["N"], 2048)),
            "one": (1, min(cfg["N"], 1024), min(cfg["N"], 128))}
    Wall, X = wq_inputs.workload_arrays(name, rows=max(p[1] for p in plan.values()))
    for tag, (threads, q_rows, g_rows) in plan.items():
        oracle.set_num_threads(threads)
        W = Wall[:q_rows]
        tq, rq = timed(lambda: oracle.quantize(W, G, bits), 2.0)
        c, s, z = oracle.quantize(W[:g_rows], G, bits)
        tg, rg = timed(lambda: [oracle.gemm(X[:B], c, s, z, g_rows, K, G, bits) for B in batches], 3.0)
        gb = sum(rl.gemm_bytes(B, g_rows, K, G, bits) for B in batches)
        out[tag] = {"threads": threads,
                    "quantize_pack": {"rows": q_rows, "s": round(tq, 4), "reps": rq,
                                      "GBps": round(rl.quantize_bytes(q_rows, K, G, bits) / tq / 1e9, 4)},
                    "gemm": {"rows": g_rows, "batches": list(batches), "s": round(tg, 4), "reps": rg,
                             "GBps": round(gb / tg / 1e9, 4)}}
    oracle.set_num_threads(all_cores)
    return {"value": out["all"]["gemm"]["GBps"], "unit": "GB/s", "cores": all_cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"rows of {name}: quantize/pack of {plan['all'][1]} rows and the double-precision "
                      f"product at B={','.join(map(str, batches))} of {plan['all'][2]} rows on "
                      f"{all_cores} threads; {plan['one'][1]} and {plan['one'][2]} rows on 1 thread",
            "breakdown": out}


def run_step_bench(args):
    import torch

    import bit_weight_only_wq_amd as wq
    import wq_inputs
    from bit_weight_only_wq_amd import roofline as rl

    cfg = wq_inputs.WORKLOADS[args.workload]
    N, K, G, bits = cfg["N"], cfg["K"], cfg["group"], cfg["bits"]
    bits = args.bits or bits
    # The headline workload runs the metric's batch range; the others their own.
    batches = list(METRIC_BATCHES) if args.workload == WORKLOAD else [b for b in cfg["batches"] if b <= 64]
    if args.batches:
        batches = [int(b) for b in args.batches.split(",")]
    dev = torch.device("cuda:0")
    Wn, Xn = wq_inputs.workload_arrays(args.workload)
    Wd = [torch.from_numpy(Wn).to(dev) for _ in range(2)]
    Xd = torch.from_numpy(Xn).to(dev)
    Xb = {B: Xd[:B].contiguous() for B in batches}
    Yb = {B: torch.empty((B, N), dtype=torch.float16, device=dev) for B in batches}
    slot_bytes = rl.packed_bytes(N, K, G, bits)
    P = max(len(batches) + 3, -(-POOL_BYTES // slot_bytes))
    P = max(P, 2 * len(batches) + 3)
    pool = [wq.quantize_pack(Wd[0], G, bits) for _ in range(P)]
    # One caller-owned workspace serves every product of the step (they run
    # one after another on the stream).
    ws_bytes = max(wq.gemm_workspace_bytes(B, K, N, G, bits, args.path) for B in batches)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_ptr = ws.data_ptr() if ws_bytes else None
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    nb = len(batches)
    # The timed loop calls the C ABI directly with precomputed pointers, so
    # host-side overhead stays far below the kernels' duration.
    lib = wq.load()
    hs = stream.cuda_stream
    path_id = {"auto": wq.WQ_PATH_AUTO, "gemv": wq.WQ_PATH_GEMV, "mfma": wq.WQ_PATH_MFMA}[args.path]
    slot_ptrs = [(c.data_ptr(), s.data_ptr(), z.data_ptr()) for c, s, z in pool]
    w_ptrs = [w.data_ptr() for w in Wd]
    xy = {B: (Xb[B].data_ptr(), Yb[B].data_ptr()) for B in batches}

    def gemm(j, B, slot):
        c, s, z = slot_ptrs[slot % P]
        st = lib.wq_gemm_ex(xy[B][0], c, s, z, xy[B][1], B, K, N, G, bits, path_id, ws_ptr, ws_bytes, hs)
        if st:
            wq.check(st, "wq_gemm")

    def quant(i, slot):
        c, s, z = slot_ptrs[slot % P]
        st = lib.wq_quantize_pack(w_ptrs[i % 2], N, K, G, bits, c, s, z, hs)
        if st:
            wq.check(st, "wq_quantize_pack")

    def step(i, ev=None):
        # Products first, each on its own pool slot; then the quantizer writes a
        # slot that is next read two steps later (>1 GB of traffic in between).
        # ev: optional events (before the products, after them, after quantize).
        if ev:
            ev[0].record(stream)
        for j, B in enumerate(batches):
            gemm(j, B, nb * i + j)
        if ev:
            ev[1].record(stream)
        quant(i, nb * i + 2 * nb + 1)
        if ev:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back.  Events on the stream the
    # library launches on split each step into its products and its quantize.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = evs[0][0].elapsed_time(evs[-1][2])
    ms_step = ms_total / args.steps
    ms_gemm = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_quant = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    # Per kernel: each product (and the quantizer) launched `steps` times back
    # to back, every launch on another pool slot, bracketed by one pair of
    # events on the library's stream; average duration per launch.
    def burst(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        fn(0)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i + 1)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    per = {B: burst(lambda i, j=j, B=B: gemm(j, B, i)) for j, B in enumerate(batches)}
    per_q = burst(lambda i: quant(i, i + nb))

    gemm_bytes = sum(rl.gemm_bytes(B, N, K, G, bits) for B in batches)
    gemm_flops = sum(rl.gemm_flops(B, N, K) for B in batches)
    q_bytes = rl.quantize_bytes(N, K, G, bits)
    kernels = {}
    for B in batches:
        kernels[f"wq_gemm_B{B}"] = kernel_entry(
            f"wq_gemm B={B}", rl.gemm_bytes(B, N, K, G, bits), rl.gemm_flops(B, N, K), [per[B]])
    kernels["wq_quantize_pack"] = kernel_entry("wq_quantize_pack", q_bytes, 0, [per_q])
    ceiling = read_ceiling()
    if ceiling:
        for e in kernels.values():
            e["frac_measured_read_ceiling"] = round(e["achieved_GBps"] / ceiling["GBps"], 4)

    busy = read_mfma_counters(args.workload) if bits == cfg["bits"] else {}
    for B in batches:
        if B in busy:
            kernels[f"wq_gemm_B{B}"]["mfma_busy_frac"] = busy[B]
    # The dominant product (longest launch) carries the roofline object.
    Bd = max(batches, key=lambda B: per[B])
    head = kernels[f"wq_gemm_B{Bd}"]
    traffic = read_traffic(f"wq_gemm_b{Bd}_{args.workload}") if bits == cfg["bits"] else None
    roof = {"kernel": head["kernel"], "bound": "hbm", "achieved": head["achieved_GBps"],
            "peak": rl.MI355X_HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
            "frac": round(head["achieved_GBps"] * 1e9 / rl.MI355X_HBM_BYTES_PER_S, 4),
            "traffic": traffic, "avg_us": head["avg_us"], "bytes_per_launch": head["bytes"]}
    if Bd in busy:
        roof["mfma_busy_frac"] = busy[Bd]
    if ceiling:
        roof["measured_read_ceiling_GBps"] = ceiling["GBps"]
        roof["frac_measured_read_ceiling"] = round(head["achieved_GBps"] / ceiling["GBps"], 4)

    value = gemm_bytes / (ms_gemm * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "N": N, "K": K, "group": G, "bits": bits,
                   "batches": batches, "path": args.path,
                   "step": "wq_gemm at B=" + ",".join(map(str, batches)) + " + wq_quantize_pack",
                   "value": "algorithmic bytes of the step's products / their time inside the timed steps",
                   "gemm_bytes_per_step": int(gemm_bytes), "quantize_bytes_per_step": int(q_bytes),
                   "workspace_bytes": int(ws_bytes), "pool_slots": P, "wall_s": round(wall, 4)},
        "frac_hbm_peak": round(value * 1e9 / rl.MI355X_HBM_BYTES_PER_S, 4),
        "ms_gemm_per_step": round(ms_gemm, 4),
        "ms_quantize_per_step": round(ms_quant, 4),
        "gemm_TFLOPs": round(gemm_flops / (ms_gemm * 1e-3) / 1e12, 2),
        "step_GBps_with_quantize": round((gemm_bytes + q_bytes) / (ms_step * 1e-3) / 1e9, 1),
        "roofline": roof,
        "kernels": kernels,
    }
    if ceiling:
        out["frac_measured_read_ceiling"] = round(value / ceiling["GBps"], 4)
        out["measured_read_ceiling"] = ceiling
    del pool, Wd
    torch.cuda.empty_cache()
    return out, batches


def read_ceiling():
    """The load-only probe's best read rate (one 1 KB piece of one row per
    load instruction), from the committed summary
    profiles/hbm_read_ceiling_probe.txt (None if absent)."""
    path = os.path.join(ROOT, "profiles", "hbm_read_ceiling_probe.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    try:
        return {"GBps": float(vals["best_GBps"]), "shape": vals.get("best_shape", ""),
                "source": "profiles/hbm_read_ceiling_probe.txt"}
    except (KeyError, ValueError):
        return None


def run_sweep(args):
    import torch

    import bit_weight_only_wq_amd as wq
    import wq_inputs
    from bit_weight_only_wq_amd import roofline as rl

    name = "ridge_sweep_k8192_n8192_g128"
    cfg = wq_inputs.WORKLOADS[name]
    N, K, G, bits = cfg["N"], cfg["K"], cfg["group"], cfg["bits"]
    dev = torch.device("cuda:0")
    Wn, Xn = wq_inputs.workload_arrays(name)
    W = torch.from_numpy(Wn).to(dev)
    X = torch.from_numpy(Xn).to(dev)
    P = -(-POOL_BYTES // rl.packed_bytes(N, K, G, bits)) + 1
    pool = [wq.quantize_pack(W, G, bits) for _ in range(P)]
    ws = torch.empty(max(16, max(wq.gemm_workspace_bytes(B, K, N, G, bits, p) for B in cfg["batches"]
                                 for p in ("gemv", "mfma") if not (p == "gemv" and B > 8))),
                     dtype=torch.uint8, device=dev)
    rows = []
    for B in cfg["batches"]:
        for path in ("gemv", "mfma"):
            if path == "gemv" and B > 8:
                continue
            Xb = X[:B].contiguous()
            Y = torch.empty((B, N), dtype=torch.float16, device=dev)
            for i in range(3):
                c, s, z = pool[i % P]
                wq.gemm(Xb, c, s, z, N=N, K=K, group=G, bits=bits, path=path, out=Y, workspace=ws)
            torch.cuda.synchronize()
            reps = 30
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                c, s, z = pool[i % P]
                wq.gemm(Xb, c, s, z, N=N, K=K, group=G, bits=bits, path=path, out=Y, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            nbytes = rl.gemm_bytes(B, N, K, G, bits)
            fl = rl.gemm_flops(B, N, K)
            model = rl.roofline_time_s(nbytes, fl) * 1e3
            rows.append({"B": B, "path": path, "us": round(ms * 1e3, 2),
                         "GBps": round(nbytes / ms / 1e6, 1),
                         "TFLOPs": round(fl / ms / 1e9, 2),
                         "intensity_2B_over_w": round(rl.intensity(B, rl.bytes_per_weight(bits, G)), 1),
                         "roofline_us": round(model * 1e3, 2)})
            print(json.dumps(rows[-1]), flush=True)
    return rows


def run_decode_set(args):
    """The 7B-class decode step: 32 layers x (q, k, v, o, gate, up, down) at
    B = 32, int4 group 128 and 8-bit per-channel.  Every matrix has its own
    packed weights in HBM (3.4 GB at int4, 6.5 GB at 8 bits), so nothing is
    served from a cache; weights are drawn on the GPU, N(0, 0.02), fp16.
    The step is timed as one wq_gemm_grouped call per layer (the headline)
    and as one wq_gemm call per matrix, each eagerly and from a HIP graph."""
    import torch

    import bit_weight_only_wq_amd as wq
    import wq_inputs
    from bit_weight_only_wq_amd import roofline as rl

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    B = wq_inputs.DECODE_SET_BATCH
    out = []
    for bits, label in ((4, "int4 g128"), (8, "int8 per-channel")):
        mats = []
        for layer in range(wq_inputs.DECODE_SET_LAYERS):
            for _, N, K in wq_inputs.DECODE_SET_SHAPES:
                G = 128 if bits == 4 else K
                W = (torch.randn((N, K), generator=gen, device=dev) * wq_inputs.DECODE_SET_SIGMA).half()
                mats.append((N, K, G) + tuple(wq.quantize_pack(W, G, bits)))
                del W
        Xs = {K: torch.randn((B, K), generator=gen, device=dev).half()
              for K in {k for _, _, k in wq_inputs.DECODE_SET_SHAPES}}
        # One output per matrix of a layer (grouped products need distinct
        # outputs); layers reuse them in stream order.
        per_layer = len(wq_inputs.DECODE_SET_SHAPES)
        Ys = [torch.empty((B, N), dtype=torch.float16, device=dev)
              for _, N, _ in wq_inputs.DECODE_SET_SHAPES]
        torch.cuda.synchronize()

        lib = wq.load()
        stream = torch.cuda.current_stream(dev)
        hs = stream.cuda_stream
        calls = [(Xs[K].data_ptr(), c.data_ptr(), s.data_ptr(), z.data_ptr(),
                  Ys[i % per_layer].data_ptr(), B, K, N, G)
                 for i, (N, K, G, c, s, z) in enumerate(mats)]
        from bit_weight_only_wq_amd._lib import GemmItem
        layers = []
        for l0 in range(0, len(calls), per_layer):
            arr = (GemmItem * per_layer)()
            for j, (x, c, s, z, y, b, k, n, g) in enumerate(calls[l0:l0 + per_layer]):
                arr[j] = GemmItem(x, c, s, z, y, b, k, n, g, bits)
            layers.append(arr)

        # One caller workspace, sized for the largest call, serves every call
        # of the step (they run one after another on the stream).
        import ctypes
        need = 0
        for arr in layers:
            n = ctypes.c_size_t(0)
            wq.check(lib.wq_gemm_grouped_workspace_size(arr, per_layer, ctypes.byref(n)), "workspace size")
            need = max(need, n.value)
        for N, K, G, *_ in mats[:per_layer]:
            need = max(need, wq.gemm_workspace_bytes(B, K, N, G, bits))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        ws_ptr = ws.data_ptr() if need else None

        def single_on(h):
            for x, c, s, z, y, b, k, n, g in calls:
                st = lib.wq_gemm_ex(x, c, s, z, y, b, k, n, g, bits, 0, ws_ptr, need, h)
                if st:
                    wq.check(st, "wq_gemm")

        def grouped_on(h):
            for arr in layers:
                st = lib.wq_gemm_grouped(arr, per_layer, ws_ptr, need, h)
                if st:
                    wq.check(st, "wq_gemm_grouped")

        def timed(fn, reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        def graph_ms(step_on):
            # Replayed from a HIP graph: no host launch gaps.  The calls
            # allocate nothing, so capture records kernels only.
            cap = torch.cuda.Stream()
            torch.cuda.synchronize()
            with torch.cuda.stream(cap):
                step_on(cap.cuda_stream)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=cap):
                step_on(cap.cuda_stream)
            graph.replay()
            return timed(graph.replay, 5)

        for _ in range(2):
            single_on(hs)
            grouped_on(hs)
        ms_single_eager = timed(lambda: single_on(hs), 5)
        ms_eager = timed(lambda: grouped_on(hs), 5)
        ms_single = graph_ms(single_on)
        ms = graph_ms(grouped_on)
        nbytes = sum(rl.gemm_bytes(B, N, K, G, bits) for N, K, G, *_ in mats)
        flops = sum(rl.gemm_flops(B, N, K) for N, K, *_ in mats)
        row = {"decode_set": label, "matrices": len(mats), "B": B, "ms_per_step": round(ms, 4),
               "ms_per_step_eager": round(ms_eager, 4),
               "ms_per_step_one_call_per_matrix": round(ms_single, 4),
               "ms_per_step_one_call_per_matrix_eager": round(ms_single_eager, 4),
               "GBps": round(nbytes / ms / 1e6, 1), "TFLOPs": round(flops / ms / 1e9, 2),
               "bytes_per_step": int(nbytes)}
        print(json.dumps(row), flush=True)
        out.append(row)
        del mats
        torch.cuda.empty_cache()
    return out


def run_kv(args):
    """Decode attention over the int4 KV cache of a 7B-class model (32 layers x
    32 heads of dimension 128) at 4096 tokens: every head's cache read once
    per step.  Two caches alternate (1.1 GB, beyond the 256 MB Infinity
    Cache); inputs are drawn on the GPU, K with one hot channel."""
    import torch

    import bit_weight_only_wq_amd as wq
    from bit_weight_only_wq_amd import roofline as rl

    H, T, D, G = KV_SHAPE
    nb = T // G
    gen = torch.Generator(device="cuda").manual_seed(0)
    caches = []
    for _ in range(2):
        cache = wq.KVCache(H, nb)
        for j in range(nb):
            Kb = torch.randn((H, G, D), generator=gen, device="cuda")
            Kb[:, :, 3] *= 8.0
            wq.kv_quantize_block(Kb.half(), torch.randn((H, G, D), generator=gen, device="cuda").half(),
                                 cache, j)
        caches.append(cache)
    q = torch.randn((H, D), generator=gen, device="cuda").half()
    lens = torch.full((H,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((H, D), dtype=torch.float16, device="cuda")
    Kb = torch.randn((H, G, D), generator=gen, device="cuda").half()
    Vb = torch.randn((H, G, D), generator=gen, device="cuda").half()
    stream = torch.cuda.current_stream()

    def burst(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    import ctypes
    n = ctypes.c_size_t(0)
    desc = caches[0].descriptor()
    wq.check(wq.load().wq_kv_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "wq_kv_workspace_size")
    ws = torch.empty(max(16, n.value), dtype=torch.uint8, device="cuda")
    ms_attn = burst(lambda i: wq.kv_attention(q, caches[i % 2], lens, out=out, workspace=ws), args.steps)
    ms_app = burst(lambda i: wq.kv_quantize_block(Kb, Vb, caches[i % 2], i % nb), args.steps)
    b_attn = rl.kv_attention_bytes(H, T, D)
    b_app = rl.kv_append_bytes(H, G, D)
    gbs = b_attn / (ms_attn * 1e-3) / 1e9
    row = {
        "metric": "decode attention over an int4 KV cache (GB/s of cache read)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "ms_per_step": round(ms_attn, 4), "higher_is_better": True, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": KV_WORKLOAD, "heads": H, "tokens": T, "head_dim": D,
                   "group": G, "bits": 4},
        "roofline": {"kernel": "kv_attn_kernel + kv_combine_kernel", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": rl.MI355X_HBM_BYTES_PER_S / 1e9,
                     "unit": "GB/s", "frac": round(gbs * 1e9 / rl.MI355X_HBM_BYTES_PER_S, 4),
                     "traffic": read_traffic(f"wq_kv_attention_{KV_WORKLOAD}"),
                     "bytes_per_launch": int(b_attn), "avg_us": round(ms_attn * 1e3, 2)},
        "kernels": {
            "kv_attention": {"avg_us": round(ms_attn * 1e3, 2), "bytes": int(b_attn),
                             "achieved_GBps": round(gbs, 1)},
            "kv_quantize_block": {"avg_us": round(ms_app * 1e3, 2), "bytes": int(b_app),
                                  "achieved_GBps": round(b_app / (ms_app * 1e-3) / 1e9, 1)},
        },
    }
    print(json.dumps(row), flush=True)
    return row


def run_format(args):
    """Another weight format on the step's workload: NF4 at blocks of 64 (the
    block the NF4 paragraph of "Gör inference billig" uses), or the
    float-offset variant of "Quantization & inference optimisation"
    ("Quantization") at the workload's group.  GPU quantize and the format's
    GEMV, each timed as a burst of launches rotating over >= 1 GiB of packed
    copies."""
    import torch

    import bit_weight_only_wq_amd as wq
    import wq_inputs
    from bit_weight_only_wq_amd import roofline as rl

    cfg = wq_inputs.WORKLOADS[args.workload]
    fmt = args.format
    N, K = cfg["N"], cfg["K"]
    G = 64 if fmt == "nf4" else cfg["group"]
    bits = 4 if fmt == "nf4" else (args.bits or cfg["bits"])
    batches = [int(b) for b in args.batches.split(",")] if args.batches else [1]
    Wn, Xn = wq_inputs.workload_arrays(args.workload)
    W = torch.from_numpy(Wn).cuda()
    X = torch.from_numpy(Xn).cuda()
    hdr = 2 if fmt == "nf4" else 4                    # fp16 scale (+ fp16 minimum) per group
    packed = N * K * bits // 8 + hdr * N * (K // G)
    P = max(3, -(-POOL_BYTES // packed))
    pool = [wq.quantize_pack(W, G, bits, scheme=fmt) for _ in range(P)]
    stream = torch.cuda.current_stream()

    def product(Xb, slot, Y):
        c, s, m = slot
        if fmt == "nf4":
            return wq.gemm_nf4(Xb, c, s, N=N, K=K, group=G, out=Y)
        return wq.gemm_offset(Xb, c, s, m, N=N, K=K, group=G, bits=bits, out=Y)

    def burst(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    kernels = {}
    for B in batches:
        Xb = X[:B].contiguous()
        Y = torch.empty((B, N), dtype=torch.float16, device="cuda")
        ms = burst(lambda i: product(Xb, pool[i % P], Y), args.steps)
        nbytes = packed + 2 * B * K + 2 * B * N
        kernels[f"wq_gemm_{fmt}_B{B}"] = {"avg_us": round(ms * 1e3, 2), "bytes": nbytes,
                                          "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    outs = [tuple(torch.empty_like(t) for t in pool[0]) for _ in range(2)]
    ms_q = burst(lambda i: wq.quantize_pack(W, G, bits, out=outs[i % 2], scheme=fmt), args.steps)
    qb = 2 * N * K + packed
    kernels[f"wq_quantize_pack_{fmt}"] = {"avg_us": round(ms_q * 1e3, 2), "bytes": qb,
                                          "achieved_GBps": round(qb / (ms_q * 1e-3) / 1e9, 1)}
    head = kernels[f"wq_gemm_{fmt}_B{batches[0]}"]
    row = {"metric": f"{fmt} decode product, achieved HBM GB/s", "value": head["achieved_GBps"], "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "ms_per_step": round(head["avg_us"] / 1e3, 5),
           "higher_is_better": True, "dtype": "f16", "data": "synthetic",
           "config": {"workload": args.workload, "N": N, "K": K, "group": G, "bits": bits, "format": fmt,
                      "batches": batches},
           "roofline": {"bound": "hbm", "achieved": head["achieved_GBps"],
                        "peak": rl.MI355X_HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
                        "frac": round(head["achieved_GBps"] * 1e9 / rl.MI355X_HBM_BYTES_PER_S, 4)},
           "kernels": kernels}
    print(json.dumps(row), flush=True)
    return row


def main():
    args = parse()
    if args.traffic_from:
        write_traffic_summaries(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.ceiling:
        run_ceiling(args)
        return
    if args.sweep:
        run_sweep(args)
        return
    if args.decode_set:
        run_decode_set(args)
        return
    if args.kv:
        run_kv(args)
        calibration_copy(args)
        return
    if args.format:
        run_format(args)
        return
    out, batches = run_step_bench(args)
    calibration_copy(args)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.workload, batches, args.bits)
    print(json.dumps(out), flush=True)


def probe_ceiling(shapes=None, reps=20, log=True):
    """Read rates of the load-only probe (libwq_probe.so) over the packed codes
    of the 70B-class up-projection (28672 rows x 4096 bytes), eight distinct
    buffers in rotation (940 MB, beyond the 256 MB Infinity Cache).  Each shape
    is (lanes per row, loads in flight per wave, walk order, non-temporal,
    workgroups per compute unit); returns one row per shape."""
    import torch

    from bit_weight_only_wq_amd import probe

    rows, row_bytes = 28672, 4096
    nbuf = 8
    bufs = [torch.empty(rows * row_bytes, dtype=torch.uint8, device="cuda:0") for _ in range(nbuf)]
    for i, b in enumerate(bufs):
        b.fill_(i + 1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    hs = stream.cuda_stream
    if shapes is None:
        shapes = ([(64, D, o, 1, bpc) for D in (2, 4) for o in (0, 1) for bpc in (1, 2, 4)] +
                  [(L, D, o, nt, bpc) for L in (32, 16, 8, 4) for D in (4, 8) for o in (0, 1, 2)
                   for nt in (1, 0) for bpc in (2, 4)])
    out = []
    for L, D, o, nt, bpc in shapes:
        def call(i):
            probe.read(bufs[i % nbuf].data_ptr(), rows, row_bytes, L, D, o, nt, bpc, sink.data_ptr(), hs)
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        row = {"lanes_per_row": L, "depth": D, "order": o, "nontemporal": nt, "blocks_per_cu": bpc,
               "us": round(us, 2), "GBps": round(rows * row_bytes / us / 1e3, 1)}
        if log:
            print(json.dumps(row), flush=True)
        out.append(row)
    del bufs
    torch.cuda.empty_cache()
    return out


def run_ceiling(args):
    """Reachable HBM read rates on this GPU, as context for the roofline
    fractions (peak 8 TB/s): the hand-written load-only probe in the access
    shapes of the product kernels (one 1 KB piece of one row per load
    instruction, as the GEMVs read; 64 to 256 bytes of each of 4 to 16 rows,
    as the matrix-core kernels read), plus plain torch read / copy / fill
    kernels over 1 GiB buffers for comparison."""
    import torch
    rows = probe_ceiling(reps=max(args.steps, 10))
    best = {}
    for r in rows:
        L = r["lanes_per_row"]
        if L not in best or r["GBps"] > best[L]["GBps"]:
            best[L] = r
    n = 1 << 29                                  # fp16 elements: 1 GiB
    src = [torch.ones(n, dtype=torch.float16, device="cuda:0") for _ in range(2)]
    dst = torch.empty(n, dtype=torch.float16, device="cuda:0")

    def timed(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps      # us per call

    reps = max(args.steps // 2, 5)
    read_us = timed(lambda i: torch.sum(src[i % 2], dtype=torch.float32), reps)
    copy_us = timed(lambda i: dst.copy_(src[i % 2]), reps)
    write_us = timed(lambda i: dst.fill_(float(i % 3)), reps)
    nbytes = n * 2
    row = {"table": "hbm ceiling", "probe_bytes": 28672 * 4096,
           "probe_best_by_lanes_per_row": {str(k): v for k, v in sorted(best.items())},
           "torch_read": {"kernel": "torch.sum (fp16 -> fp32)", "us": round(read_us, 2),
                          "GBps": round(nbytes / read_us / 1e3, 1)},
           "torch_copy": {"kernel": "Tensor.copy_", "us": round(copy_us, 2),
                          "GBps": round(2 * nbytes / copy_us / 1e3, 1)},
           "torch_write": {"kernel": "Tensor.fill_", "us": round(write_us, 2),
                           "GBps": round(nbytes / write_us / 1e3, 1)},
           "peak_GBps": 8000.0}
    print(json.dumps(row), flush=True)
    return row


def calibration_copy(args):
    if args.copy_calibration_mib:
        import torch
        # An elementwise kernel (not a DMA copy, which the counters do not see)
        # that reads and writes exactly copy_calibration_mib MiB each.
        a = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda:0")
        a.fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 3, out=b)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
