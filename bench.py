#!/usr/bin/env python3
"""Throughput of one simulated Ulysses step on one MI355X.

A step is one pass of the whole per-rank hot path over one batch of synthetic
input, for every layer type of the workload: cu_seqlens/max_len rebuilt from
the gathered position_ids, pack of Q/K/V (sequence -> head shards, all P
simulated ranks), attention forward on every rank, unpack of O, pack of dO,
attention backward on every rank, unpack of dQ/dK/dV.  Inputs are resident
in HBM before the timed region starts.

``value`` is attention fwd+bwd TFLOP/s of the whole step: algorithmic FLOPs
(12*D per visible (query, key) pair per query head: 4*D forward, 8*D
backward; recompute not counted, masked pairs not counted) divided by the
wall time of the step, all P ranks together.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd+bwd TFLOP/s per rank share (% bf16 MFMA peak); a2a pack GB/s"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
DEFAULT_WORKLOAD = 5         # S=131072 causal, GQA 28/4, D=128, P=4 (the largest)


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_digest():
    """sha256 over the kernel sources and the build flags: HBM traffic taken with
    rocprofv3 counters is reported only while this digest is unchanged."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "ulysses_sequence_attention_rank_amd")
    files = [os.path.join(pkg, "build.py")]
    csrc = os.path.join(pkg, "csrc")
    files += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_per_launch(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for
    the pack kernel's known bytes), or None if absent or taken on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get(kernel)
    return None if k is None else k["bytes_per_launch"]


def visible_pairs(doc_lengths, causal, wl, wr):
    """Unmasked (query, key) pairs per query head: keys in the query's document,
    j <= i if causal, i - j <= wl and j - i <= wr when those are >= 0."""
    import numpy as np
    total = 0
    for L in doc_lengths:
        t = np.arange(L, dtype=np.int64)
        lo = np.maximum(0, t - wl) if wl >= 0 else np.zeros_like(t)
        hi = np.full_like(t, L - 1)
        if causal:
            hi = np.minimum(hi, t)
        if wr >= 0:
            hi = np.minimum(hi, t + wr)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return total


def docs_of(inp):
    c = inp.case
    if inp.doc_lengths is not None:
        return list(inp.doc_lengths)
    return [c.S] * c.B


def kernel_credit(case, docs):
    """Algorithmic work credited to each kernel, per layer type and rank call:
    (unit, amount).  Attention: FLOPs (fwd QK^T and PV: 4D per pair; bwd: dP, dV
    and dK in the key-tile kernel: 6D, dQ in the query-tile kernel: 2D).
    Layout and scan kernels: bytes that must cross HBM."""
    D, hq = case.D, case.hq
    out = {}
    for v in case.variants:
        pairs = visible_pairs(docs, v.causal, v.window_left, v.window_right) * hq
        out[v.name] = {"attn_fwd": 4 * D * pairs, "attn_bwd_dkdv": 6 * D * pairs,
                       "attn_bwd_dq": 2 * D * pairs, "pairs": pairs}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5, 6],
                    help="which of the five simulated workloads (default: the S=131072 one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mlp", action="store_true", help="skip the sequence-tiled MLP measurement")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="query heads of rank 0 the CPU oracle baseline runs (default: all of "
                         "rank 0's heads, every layer, for the S<=4096 workloads; one KV group of "
                         "rank 0 for the S=32768 ones; none for the larger ones)")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="S > 32768: query rows (stratified) of the CPU oracle's subset baseline")
    ap.add_argument("--cpu-keys", type=int, default=1024,
                    help="S > 32768: last keys whose dK/dV the CPU oracle's subset baseline computes")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of a captured HIP graph of the step")
    ap.add_argument("--layer", default=None,
                    help="run only this layer type of the workload (e.g. swa128)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for counter collection: warm-up and --steps eager steps only, no other "
                         "measurement; prints a short JSON line")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the vendor-library bf16 GEMM and the matrix-core calibration "
                         "measured beside the step")
    ap.add_argument("--gemm-reference-only", action="store_true",
                    help="measure only the vendor-library bf16 GEMM (for counter collection) and "
                         "print its JSON object")
    ap.add_argument("--mfma-calibration-only", action="store_true",
                    help="run only the matrix-core calibration (for counter collection) and print "
                         "its JSON object")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="no GPU run: summarise rocprofv3 CSV output under DIR (trace/, sq/, "
                         "fetch/, write/ and commands.txt) of a run of this script on --workload "
                         "into profiles/, and record the measured HBM traffic per kernel")
    args = ap.parse_args()

    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary, args.workload)
        return

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the P Ulysses ranks are simulated in memory "
              f"on that GPU, so --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.gemm_reference_only:
        print(json.dumps(measure_gemm_reference(torch.device("cuda", 0))), flush=True)
        return
    if args.mfma_calibration_only:
        import ulysses_sequence_attention_rank_amd as uly_
        if not os.path.exists(uly_.lib_path()):
            from ulysses_sequence_attention_rank_amd import build
            build.build()
        print(json.dumps(measure_mfma_calibration(torch.device("cuda", 0))), flush=True)
        return

    import ulysses_sequence_attention_rank_amd as uly
    from ulysses_inputs import WORKLOADS, make_inputs, seq_shards
    from ulysses_sequence_attention_rank_amd import sim

    if not os.path.exists(uly.lib_path()):
        from ulysses_sequence_attention_rank_amd import build
        build.build()
    uly.load()

    case = WORKLOADS[args.workload]
    if args.layer is not None:
        import dataclasses
        keep = tuple(v for v in case.variants if v.name == args.layer)
        if not keep:
            raise SystemExit(f"workload {case.name} has no layer {args.layer!r}")
        case = dataclasses.replace(case, variants=keep)
    log(f"workload {args.workload} {case.name}: generating inputs")
    inp = make_inputs(case)
    dev = torch.device("cuda", 0)
    P = case.P
    b = sim.allocate(seq_shards(inp.q, P).to(dev), seq_shards(inp.k, P).to(dev),
                     seq_shards(inp.v, P).to(dev), seq_shards(inp.dout, P).to(dev),
                     seq_shards(inp.positions, P).to(dev),
                     None if inp.sink is None else inp.sink.to(dev))
    torch.cuda.synchronize()

    def step():
        for v in case.variants:
            sim.step(b, causal=v.causal, window_left=v.window_left, window_right=v.window_right)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_pass:
        log(f"profile pass: {args.steps} eager steps")
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": case.name, "layers": [v.name for v in case.variants],
                          "steps": args.steps}), flush=True)
        return

    # The whole step is captured once into a HIP graph and replayed: about 50
    # kernel launches per step, many of them a few microseconds long, so
    # launch gaps would otherwise dominate the small workloads.
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()

    log(f"timing {args.steps} steps ({'HIP graph' if graph is not None else 'eager'})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps

    # the same step with the permutation folded into the attention kernels'
    # addressing (fused layout): timed the same way
    def fused_step():
        for v in case.variants:
            sim.step(b, causal=v.causal, window_left=v.window_left, window_right=v.window_right,
                     fused=True)
    fused_step()
    fgraph = None
    if not args.no_graph:
        fgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fgraph):
            fused_step()
        for _ in range(args.warmup):
            fgraph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if fgraph is not None:
            fgraph.replay()
        else:
            fused_step()
    torch.cuda.synchronize()
    fused_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    del fgraph

    # per-kernel durations: the same steps launched eagerly, one layer type at
    # a time, each kernel bracketed by HIP events on the stream it runs on
    kern_layer = {}
    for v in case.variants:
        log(f"per-kernel timing over {args.steps} eager steps of the {v.name} layer")
        uly.profile_start(max_launches=64 * args.steps * P + 64)
        for _ in range(args.steps):
            sim.step(b, causal=v.causal, window_left=v.window_left, window_right=v.window_right)
        torch.cuda.synchronize()
        uly.profile_stop()
        kern_layer[v.name] = uly.profile_report()
    kern = {}
    for rep in kern_layer.values():
        for name, (cnt, tot, mn, mx) in rep.items():
            c0 = kern.get(name, (0, 0.0, float("inf"), 0.0))
            kern[name] = (c0[0] + cnt, c0[1] + tot, min(c0[2], mn), max(c0[3], mx))

    docs = docs_of(inp)
    credit = kernel_credit(case, docs)
    layers = layer_figures(case, credit, kern_layer, args.steps)
    step_flops = sum(12 * case.D * credit[v.name]["pairs"] for v in case.variants) * P
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # per-kernel figures from the events recorded around each launch
    launches_per_step = {"attn_fwd": P * len(case.variants), "attn_bwd_dkdv": P * len(case.variants),
                         "attn_bwd_dq": P * len(case.variants)}
    rows = {}
    for name, (cnt, tot, mn, mx) in kern.items():
        rows[name] = {"launches": cnt, "avg_ms": tot / cnt, "total_ms_per_step": tot / args.steps}
    attn_credit = {k: sum(credit[v.name][k] for v in case.variants) * P * args.steps
                   for k in ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq")}
    for k, fl in attn_credit.items():
        if k in kern:
            rows[k]["tflops"] = fl / (kern[k][1] * 1e-3) / 1e12
            rows[k]["frac_of_peak"] = rows[k]["tflops"] / PEAK_BF16_TFLOPS
            # what the kernel's products compute per visible pair (masked
            # parts of diagonal tiles not counted): credited / executed
            cr, ex = EXECUTED_PER_PAIR[k]
            rows[k]["executed_flop_per_pair"] = f"{ex}*D (credited {cr}*D)"
            rows[k]["executed_tflops"] = rows[k]["tflops"] * ex / cr
    # layout permutation inside the step (every element read once and written
    # once; the step's buffers may sit in the Infinity Cache)
    elem_q = case.B * case.S * case.Hq * case.D
    elem_kv = case.B * case.S * case.Hkv * case.D
    pack_bytes = 2 * 2 * (2 * elem_q + 2 * elem_kv)   # Q, dO (Hq) and K, V (Hkv), per layer
    unpack_bytes = 2 * 2 * (2 * elem_q + 2 * elem_kv)  # O, dQ (Hq) and dK, dV (Hkv)
    if case.Hkv < case.P:
        # K and V are read once and written P / Hkv times over (replicated); dK, dV
        # are summed by their own kernel, so only O and dQ are unpacked
        elem_rep = case.P * case.B * case.S * case.D
        pack_bytes = 2 * (2 * 2 * elem_q + 2 * (elem_kv + elem_rep))
        unpack_bytes = 2 * 2 * 2 * elem_q
    nl = len(case.variants) * args.steps
    if "a2a_pack" in kern:
        rows["a2a_pack"]["gbps"] = pack_bytes * nl / (kern["a2a_pack"][1] * 1e-3) / 1e9
    if "a2a_unpack" in kern:
        rows["a2a_unpack"]["gbps"] = unpack_bytes * nl / (kern["a2a_unpack"][1] * 1e-3) / 1e9
    if case.Hkv < case.P:  # replicated KV heads: Q, K, V are not one permutation launch
        perm = {"tensors": "in-step figures (replicated KV heads)",
                "pack_gbps": round(rows.get("a2a_pack", {}).get("gbps", 0.0), 1),
                "unpack_gbps": round(rows.get("a2a_unpack", {}).get("gbps", 0.0), 1)}
    else:
        perm = measure_permutation(case, b, dev)
    attn_ms = sum(v[1] for k, v in kern.items() if k.startswith("attn_"))
    attn_tflops = step_flops * args.steps / (attn_ms * 1e-3) / 1e12

    # roofline of the kernel that takes the most time in the step
    dom = max(("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"), key=lambda k: kern.get(k, (0, 0))[1])
    per_launch_flops = attn_credit[dom] / kern[dom][0]
    achieved = per_launch_flops / (kern[dom][1] / kern[dom][0] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_per_launch(case.name, dom),
                "flops_per_launch": per_launch_flops,
                "avg_launch_ms": round(kern[dom][1] / kern[dom][0], 5)}

    ring = measure_ring(case, b, credit) if case.Hkv >= case.P else None
    mlp = None if args.no_mlp else measure_tiled_mlp(dev)
    gemm_ref = None if args.no_gemm_reference else measure_gemm_reference(dev)
    mfma_cal = None if args.no_gemm_reference else measure_mfma_calibration(dev)

    cpu = None
    if not args.no_cpu_baseline:
        if args.cpu_heads is not None:
            cpu = cpu_baseline(inp, ranks=[0], n_heads=args.cpu_heads)
        elif case.S <= 4096:
            cpu = cpu_baseline(inp, ranks=[0], n_heads=case.Hq // P)
        elif case.S <= 32768:
            cpu = cpu_baseline(inp, ranks=[0], n_heads=case.Hq // case.Hkv)
        else:
            cpu = cpu_baseline_subset(inp, n_rows=args.cpu_rows, n_keys=args.cpu_keys)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "precision": ("bf16 inputs and outputs; forward products bf16 MFMA, backward products fp16 "
                      "MFMA on exact power-of-two-scaled fp16 copies; fp32 accumulation"),
        "data": "synthetic",
        "config": {"workload": case.name, "P": P, "B": case.B, "S": case.S, "Hq": case.Hq,
                   "Hkv": case.Hkv, "D": case.D, "layers": [v.name for v in case.variants],
                   "sink": case.sink, "packed_docs": len(docs) if inp.doc_lengths else None},
        "execution": "hip_graph" if graph is not None else "eager",
        "device": device_info(dev),
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fa_convention": {"value": round(value * 14 / 12, 2),
                          "note": "the same step credited 14*D per pair (backward = 2.5 x forward, "
                                  "its recompute of QK^T included); not the reported value"},
        "fused_layout": {"ms_per_step": round(fused_ms, 4),
                         "value": round(step_flops / (fused_ms * 1e-3) / 1e12, 2),
                         "note": "attention reads Q/K/V and writes O/dQ/dK/dV in the sequence "
                                 "shards in place: no pack/unpack launches"},
        "attn_tflops": round(attn_tflops, 2),
        "pack_gbps": perm["pack_gbps"],
        "pack_frac_of_hbm": round(perm["pack_gbps"] / PEAK_HBM_GBPS, 4),
        "unpack_gbps": perm["unpack_gbps"],
        "permutation": perm,
        "layers": layers,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for k, r in rows.items()},
        "ring_inner_step": ring,
        "tiled_mlp": mlp,
        "gemm_reference": gemm_ref,
        "mfma_calibration": mfma_cal,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if cpu is not None:
        cpu.update(host_cpus())
        cpu["gpu_over_cpu"] = round(value / cpu["value"], 1) if cpu["value"] else None
    print(json.dumps(line), flush=True)


def host_cpus():
    """Logical CPUs, those this process may run on, and physical cores (distinct
    (package, core) pairs in /proc/cpuinfo) of the host."""
    out = {"logical_cpus": os.cpu_count()}
    try:
        out["usable_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        pairs, phys = set(), None
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("physical id"):
                    phys = ln.split(":")[1].strip()
                elif ln.startswith("core id"):
                    pairs.add((phys, ln.split(":")[1].strip()))
        if pairs:
            out["physical_cores"] = len(pairs)
    except OSError:
        pass
    return out


def device_info(dev):
    """The GPU as the runtime reports it: name, architecture, compute units
    and peak shader clock (hipDeviceGetAttribute), and the dense bf16 MFMA
    peak those give at 4096 FLOP per clock per CU (32x32x16 products, one per
    32 clocks on each of a CU's four SIMDs)."""
    import ctypes

    import torch
    p = torch.cuda.get_device_properties(dev)
    out = {"name": p.name, "arch": p.gcnArchName, "cus": p.multi_processor_count,
           "hbm_gib": round(p.total_memory / 2 ** 30, 1)}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (kHz) and hipDeviceAttributeMultiprocessorCount
        # of hip_runtime_api.h; the second must agree with torch's count
        if (hip.hipDeviceGetAttribute(ctypes.byref(val), 63, dev.index or 0) == 0
                and val.value == p.multi_processor_count
                and hip.hipDeviceGetAttribute(ctypes.byref(val), 5, dev.index or 0) == 0):
            out["peak_sclk_mhz"] = val.value // 1000
            out["peak_bf16_tflops"] = round(p.multi_processor_count * val.value * 1e3 * 4096 / 1e12, 1)
    except OSError:
        pass
    return out


# (credited, executed) multiples of D per visible pair: the forward's QK^T
# and PV; dK/dV recomputes QK^T; dQ recomputes QK^T and dP
EXECUTED_PER_PAIR = {"attn_fwd": (4, 4), "attn_bwd_dkdv": (6, 8), "attn_bwd_dq": (2, 6)}

ATTN_KERNELS = ("attn_fwd", "attn_fwd_merge", "attn_bwd_stats", "attn_bwd_prep", "attn_bwd_dkdv",
                "attn_bwd_dkdv_reduce", "attn_bwd_dq", "attn_bwd_dq_reduce", "attn_bwd_dsink")


def layer_figures(case, credit, kern_layer, steps):
    """Per layer type: the attention kernels' time per rank call (forward and
    backward, every launch of the attention calls), the credited TFLOP/s, and
    for a sliding-window layer, whose arithmetic intensity is below the ridge,
    the compulsory HBM bytes against the 8 TB/s peak: each rank call must read
    q, k, v and write O and LSE (forward), read q, k, v, O, dO, LSE and write
    dQ, dK, dV (backward)."""
    P, B, S, D, hq, hkv = case.P, case.B, case.S, case.D, case.hq, case.hkv
    qb, kvb, lseb = B * S * hq * D * 2, B * S * hkv * D * 2, B * S * hq * 4
    out = {}
    for v in case.variants:
        rep = kern_layer[v.name]
        calls = P * steps
        attn_ms = sum(t for k, (c, t, _, _) in rep.items() if k in ATTN_KERNELS) / calls
        fl = 12 * D * credit[v.name]["pairs"]
        rec = {"ms_per_rank": round(attn_ms, 5),
               "tflops": round(fl / (attn_ms * 1e-3) / 1e12, 2),
               "frac_of_mfma_peak": round(fl / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "kernels_ms_per_rank": {k: round(t / calls, 5) for k, (c, t, _, _) in rep.items()
                                       if k in ATTN_KERNELS}}
        if v.window_left >= 0 or v.window_right >= 0:
            hbm = (qb + 2 * kvb + qb + lseb) + (qb + 2 * kvb + 2 * qb + lseb + qb + 2 * kvb)
            gbps = hbm / (attn_ms * 1e-3) / 1e9
            rec["hbm"] = {"bound": "hbm", "bytes_per_rank": hbm, "floor_ms": round(hbm / 8e12 * 1e3, 5),
                          "achieved_gbps": round(gbps, 1), "peak_gbps": PEAK_HBM_GBPS,
                          "frac": round(gbps / PEAK_HBM_GBPS, 4),
                          "flop_per_byte": round(fl / hbm, 1)}
        out[v.name] = rec
    return out


def measure_permutation(case, b, dev, launches=40):
    """HBM throughput of the layout permutation on its own: Q, K and V packed
    in one launch (and dQ, dK, dV unpacked in one), back to back, rotating over
    enough buffer sets that the 256 MB Infinity Cache cannot hold them; one
    HIP event pair around all launches."""
    import math

    import torch

    import ulysses_sequence_attention_rank_amd as uly
    P = case.P
    seq0 = [b.q_seq, b.k_seq, b.v_seq]
    set_bytes = sum(t.numel() * t.element_size() for t in seq0)  # read once, written once
    n_sets = max(1, math.ceil(1.5 * 2 ** 30 / (2 * set_bytes)))
    seqs = [seq0] + [[t.clone() for t in seq0] for _ in range(n_sets - 1)]
    heads = [[torch.empty((P, t.shape[1], t.shape[2] * P, t.shape[3] // P, t.shape[4]),
                          dtype=t.dtype, device=dev) for t in ss] for ss in seqs]
    out = {"tensors": "Q, K, V in one launch", "launches": launches, "buffer_sets": n_sets,
           "bytes_per_launch": 2 * set_bytes}
    for name, fn, src, dst in (("pack", uly.a2a_pack_multi_into, seqs, heads),
                               ("unpack", uly.a2a_unpack_multi_into, heads, seqs)):
        for i in range(n_sets):
            fn(src[i], dst[i], P)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(launches):
            fn(src[i % n_sets], dst[i % n_sets], P)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        out[f"{name}_us_per_launch"] = round(1e3 * ms, 2)
        out[f"{name}_gbps"] = round(2 * set_bytes / (ms * 1e-3) / 1e9, 1)
    del seqs[1:], heads
    torch.cuda.empty_cache()
    return out


def measure_ring(case, b, credit, chunks=4, reps=5):
    """Rank 0's forward as the inner step of a ring over KV chunks: attention
    against each of `chunks` equal KV chunks, merged exactly as they arrive,
    then finished (sink added, bf16 out), against the single forward over all
    keys; every layer type, HIP events around `reps` repetitions."""
    import torch

    import ulysses_sequence_attention_rank_amd as uly
    S, hq = case.S, case.hq
    if S % chunks:
        return None
    sk = None if b.sink is None else b.sink[:hq]
    q, k, v = b.q_head[0], b.k_head[0], b.v_head[0]
    cu = b.cu if case.doc_len_range else None
    n = b.n_seqs if case.doc_len_range else None
    Sk = S // chunks
    out = {"chunks": chunks, "layers": {}}
    for var in case.variants:
        kw = dict(causal=var.causal, window_left=var.window_left, window_right=var.window_right)
        parts = [(torch.empty((case.B, S, hq, case.D), dtype=torch.float32, device=q.device),
                  torch.empty((case.B, hq, S), dtype=torch.float32, device=q.device))
                 for _ in range(2)]
        acc_o, acc_l = (torch.empty_like(parts[0][0]), torch.empty_like(parts[0][1]))
        fin_o = torch.empty_like(q)
        fin_l = torch.empty_like(acc_l)

        def ring():
            for c in range(chunks):
                dst = (acc_o, acc_l) if c == 0 else parts[c % 2]
                uly.attn_fwd_chunk(q, k[:, c * Sk:(c + 1) * Sk], v[:, c * Sk:(c + 1) * Sk], c * Sk,
                                   cu_seqlens=cu, n_seqs=n, out=dst[0], lse=dst[1],
                                   workspace=b.workspace, **kw)
                if c:
                    uly.attn_merge(acc_o, acc_l, dst[0], dst[1])
            uly.attn_merge_finish(acc_o, acc_l, sink=sk, out=fin_o, lse=fin_l)

        def plain():
            uly.attn_fwd(q, k, v, sink=sk, cu_seqlens=cu, n_seqs=n, out=b.o_head[0], lse=b.lse[0],
                         workspace=b.workspace, **kw)
        res = {}
        for name, fn in (("ring", ring), ("single", plain)):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[f"{name}_ms"] = round(e0.elapsed_time(e1) / reps, 4)
        res["ring_fwd_tflops"] = round(credit[var.name]["attn_fwd"] / (res["ring_ms"] * 1e-3) / 1e12, 1)
        out["layers"][var.name] = res
    return out


def measure_gemm_reference(dev, n=16384, reps=20):
    """What this GPU sustains on a plain dense bf16 contraction in the same
    run: torch.matmul (the vendor BLAS) on n x n x n bf16 operands, fp32
    accumulation, timed with HIP events over `reps` products after three
    untimed ones.  Context for the attention kernels' figures (the chip's
    clock falls under sustained MFMA load); not part of the step."""
    import torch
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"kind": "torch.matmul bf16 (vendor BLAS)", "m": n, "n": n, "k": n, "reps": reps,
            "ms": round(ms, 4), "tflops": round(tflops, 1),
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def measure_mfma_calibration(dev, iters=160000, reps=2):
    """The library's matrix-core calibration: bf16 32x32x16 products with
    nothing else to do (operands pseudo-random and changing), then with 8 fp32
    FMAs beside each product, then with one and with both operands of each
    product read from LDS (1 and 2 KiB a product), then with 8 exp2 (and, to
    compare, 8 multiplies) beside each product; two waves per SIMD.  What
    the GPU sustains on products alone and fed through LDS, at the clock it
    settles at under each load.  Context only, not part of the step."""
    import torch

    import ulysses_sequence_attention_rank_amd as uly
    out = torch.empty(512 * 256, dtype=torch.float32, device=dev)
    res = {"kind": "bf16 32x32x16 MFMA, pseudo-random operands (library calibration)",
           "iters": iters}
    for name, mode in (("registers", 0), ("registers_8_fma_per_mfma", 1),
                       ("lds_1KiB_per_mfma", 2), ("lds_2KiB_per_mfma", 3),
                       ("registers_8_exp2_per_mfma", 4), ("registers_8_mul_per_mfma", 5)):
        uly.calibrate_mfma(iters // 10 // 8 * 8, mode, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = 0
        for _ in range(reps):
            flops += uly.calibrate_mfma(iters, mode, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        tflops = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms / reps, 3), "tflops": round(tflops, 1),
                     "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}
    return res


def measure_tiled_mlp(dev, T=32768, H=2048, I=8192, tile=8192, reps=3):
    """The sequence-tiled gated MLP of one rank: a Llama-3.2-1B-sized MLP
    (hidden 2048, intermediate 8192) over the 32768 tokens a rank holds in the
    S=131072, P=4 workload, in tiles of 8192 tokens.  Forward and backward
    timed apart with HIP events over `reps` repetitions each; credited FLOPs
    6 T H I (forward) and 12 T H I (backward; its recompute of the gate and up
    projections, 4 T H I, is not credited), against the bf16 dense peak."""
    import torch

    import ulysses_sequence_attention_rank_amd as uly
    from ulysses_inputs import make_mlp_inputs
    m = make_mlp_inputs(2026, T, H, I, device=dev)
    ws = torch.empty(uly.tiled_mlp_workspace_bytes(T, H, I, tile), dtype=torch.uint8, device=dev)
    y = torch.empty_like(m.x)
    dx = torch.empty_like(m.x)
    dwg = torch.empty((I, H), dtype=torch.float32, device=dev)
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((H, I), dtype=torch.float32, device=dev)
    fwd = lambda: uly.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, m.w_down, tile, y=y, workspace=ws)
    bwd = lambda: uly.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile, dx=dx, dw_gate=dwg,
                                    dw_up=dwu, dw_down=dwd, workspace=ws)
    out = {"workload": f"T{T}_H{H}_I{I}_tile{tile}", "T": T, "H": H, "I": I, "tile": tile}
    thi = float(T) * H * I
    for name, fn, credit in (("fwd", fwd, 6 * thi), ("bwd", bwd, 12 * thi)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{name}_ms"] = round(ms, 4)
        out[f"{name}_tflops"] = round(credit / (ms * 1e-3) / 1e12, 1)
    out["tflops"] = round(18 * thi / ((out["fwd_ms"] + out["bwd_ms"]) * 1e-3) / 1e12, 1)
    out["frac_of_peak"] = round(out["tflops"] / PEAK_BF16_TFLOPS, 4)
    # per-kernel times of one forward and one backward
    uly.profile_start()
    fwd()
    bwd()
    torch.cuda.synchronize()
    uly.profile_stop()
    rep = uly.profile_report()
    out["kernels"] = {k: {"launches": v[0], "total_ms": round(v[1], 4)} for k, v in rep.items()
                      if k.startswith("mlp")}
    return out


def _rocprof_name(full):
    """Short name of a kernel as rocprofv3 prints it, matching the names the
    library's per-kernel timer uses."""
    import re
    if "at::native" in full:
        return "torch (buffer fill)"
    if full.startswith("Cijk_"):
        return "gemm_reference (vendor BLAS)"
    if "calib_mfma_kernel" in full:
        return "mfma_calibration"
    m = re.search(r"uly::(\w+?)_kernel(<[^>]*>)?", full)
    if not m:
        return full
    name, targs = m.group(1), m.group(2) or ""
    if name == "permute":
        return "a2a_pack" if "true" in targs else "a2a_unpack"
    if name == "segments":
        return "cu_seqlens"
    if name in ("dq_reduce", "dkdv_reduce"):
        return "attn_bwd_" + name
    if name == "mlp_gemm":  # the tiled MLP's products, by operand layouts and epilogue
        return {"<false, false, 1>": "mlp_gate_up", "<false, false, 0>": "mlp_down",
                "<false, false, 2>": "mlp_bwd_gate_up", "<false, true, 3>": "mlp_bwd_gated",
                "<false, true, 0>": "mlp_bwd_dx", "<true, true, 4>": "mlp_bwd_dw"}.get(targs, name)
    if name in ("dsink_partial", "dsink_final"):
        return "attn_bwd_" + name
    return name


def alg_bytes_per_launch(case, kernel):
    """Compulsory HBM bytes of one launch of `kernel` on `case` (per rank call
    for the attention kernels; per launch averaged over the step's launches for
    the permutation): every operand read once and every result written once.
    None for kernels without a stated figure."""
    B, S, D, hq, hkv, P = case.B, case.S, case.D, case.hq, case.hkv, case.P
    qb, kvb, lseb = B * S * hq * D * 2, B * S * hkv * D * 2, B * S * hq * 4
    eq, ekv = B * S * case.Hq * D * 2, B * S * case.Hkv * D * 2
    return {
        # forward: q, k, v in; O, LSE out
        "attn_fwd": qb + 2 * kvb + qb + lseb,
        # fp16 copies of q, dO, k, v and LSE*log2e, -delta in; dK, dV out
        "attn_bwd_dkdv": 2 * qb + 2 * kvb + 2 * lseb + 2 * kvb,
        # the same in; dQ out
        "attn_bwd_dq": 2 * qb + 2 * kvb + 2 * lseb + qb,
        # dout, O, q, k, v, LSE in; -delta, LSE*log2e out
        "attn_bwd_stats": 3 * qb + 2 * kvb + 3 * lseb,
        # q, k, v, dout in, their fp16 copies out; -delta rescaled in place
        "attn_bwd_prep": 2 * (2 * qb + 2 * kvb) + 2 * lseb,
        # Q, K, V in one launch, then dO: each element read and written once
        "a2a_pack": (2 * (eq + 2 * ekv) + 2 * eq) // 2 if case.Hkv >= P else None,
        # O, then dQ, dK, dV in one launch
        "a2a_unpack": (2 * eq + 2 * (eq + 2 * ekv)) // 2 if case.Hkv >= P else None,
    }.get(kernel)


PEAK_CLOCK_GHZ = 2.4
CUS = 256
SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8


def rocprof_summary(d, workload):
    """Write profiles/<workload>_kernels.md from rocprofv3 CSV files under d and
    record per-launch HBM traffic in profiles/traffic.json.

    d/trace: --kernel-trace --stats of the benchmark command; d/<layer>/sq,
    d/<layer>/fetch, d/<layer>/write: counter passes of `--profile-pass
    --layer <layer>` runs (one layer type each); d/commands.txt: the commands.
    Per kernel: executed MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024
    SIMDs x cycles), at the nominal 2.4 GHz over the traced duration and at the
    clock the kernel ran at (GRBM_GUI_ACTIVE cycles over the dispatch, which
    the counter reports summed over the 8 XCDs);
    VALU and MFMA instructions; the LDS's busy fraction (SQ_LDS_IDX_ACTIVE, summed
    over the CUs) and bytes read from it per MFMA; HBM bytes (FETCH_SIZE, WRITE_SIZE scaled by the
    pack kernel's known bytes), GB/s, and their ratio to the compulsory bytes."""
    import collections
    import csv
    import glob
    import re
    from ulysses_inputs import WORKLOADS
    case = WORKLOADS[workload]

    def rows(sub, suffix):
        fs = sorted(glob.glob(os.path.join(d, sub, "**", f"*{suffix}"), recursive=True))
        if not fs:
            raise SystemExit(f"no *{suffix} under {os.path.join(d, sub)}")
        with open(fs[0]) as f:
            return list(csv.DictReader(f))

    def counters(sub):
        """Per kernel: each counter's average per dispatch, and the dispatches'
        average duration in that pass ("_us").  For GRBM_GUI_ACTIVE and the
        duration a kernel's first dispatch in the process is left out when
        there are others: its busy cycles also count the code object's first
        load."""
        agg = collections.defaultdict(lambda: collections.defaultdict(dict))
        for r in rows(sub, "counter_collection.csv"):
            k, disp = _rocprof_name(r["Kernel_Name"]), int(r["Dispatch_Id"])
            agg[k][disp][r["Counter_Name"]] = float(r["Counter_Value"])
            agg[k][disp]["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        out = {}
        for k, by_disp in agg.items():
            every = sorted(by_disp)
            out[k] = {}
            for c in {c for dd in every for c in by_disp[dd]}:
                ds = every[1:] if (c in ("GRBM_GUI_ACTIVE", "_us") and len(every) > 1) else every
                vals = [by_disp[dd][c] for dd in ds if c in by_disp[dd]]
                out[k][c] = sum(vals) / len(vals)
        return out

    # scale factors: every thread of the pack kernel reads and writes
    # kPermUnroll 16-byte vectors (grids are a whole number of blocks for
    # these shapes), so a dispatch moves Grid_Size * 16 * kPermUnroll bytes
    # each way; the constant is read from the kernel's source
    with open(os.path.join(ROOT, "ulysses_sequence_attention_rank_amd", "csrc", "permute.hip")) as f:
        m = re.search(r"constexpr int kPermUnroll = (\d+);", f.read())
    if m is None:
        raise SystemExit("kPermUnroll not found in permute.hip")
    pack_thread_bytes = 16 * int(m.group(1))

    def pack_scale(sub, counter):
        known = got = 0.0
        for r in rows(sub, "counter_collection.csv"):
            if _rocprof_name(r["Kernel_Name"]) == "a2a_pack" and r["Counter_Name"] == counter:
                known += float(r["Grid_Size"]) * pack_thread_bytes
                got += float(r["Counter_Value"]) * 1024
        return known / got

    def averages(sub):
        out = {}
        for r in rows(sub, "kernel_stats.csv"):
            out.setdefault(_rocprof_name(r["Name"]), float(r["AverageNs"]) / 1e3)
        return out

    stats = rows("trace", "kernel_stats.csv")
    avg_all = averages("trace")
    with open(os.path.join(d, "commands.txt")) as f:
        commands = [ln.rstrip() for ln in f if ln.strip()]

    per_layer = {}
    for v in case.variants:
        sub = v.name
        sq, fe, wr = counters(f"{sub}/sq"), counters(f"{sub}/fetch"), counters(f"{sub}/write")
        f_scale, w_scale = pack_scale(f"{sub}/fetch", "FETCH_SIZE"), pack_scale(f"{sub}/write", "WRITE_SIZE")
        # per-dispatch durations of this layer's counter pass are not the traced
        # ones (counters serialise dispatches); the traced average is used
        lay = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
        # durations: this layer type's own kernel trace where the workload has
        # several (one kernel name serves all of them), else the benchmark's
        lay["avg_us"] = (averages(f"{sub}/trace") if os.path.isdir(os.path.join(d, sub, "trace"))
                         else avg_all)
        for k in sorted(sq):
            if k.startswith("torch") or k.startswith("__amd"):
                continue
            rec = {"sq": sq[k]}
            if k in fe and k in wr:
                rec["fetch_kib"] = round(fe[k]["FETCH_SIZE"], 1)
                rec["write_kib"] = round(wr[k]["WRITE_SIZE"], 1)
                rec["bytes_per_launch"] = round(1024 * (fe[k]["FETCH_SIZE"] * f_scale +
                                                        wr[k]["WRITE_SIZE"] * w_scale))
            lay["kernels"][k] = rec
        per_layer[sub] = lay

    # traffic.json: per workload, per kernel, bytes per launch averaged over the layer types
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_sha256") != kernel_source_digest():
        rec = {"source_sha256": kernel_source_digest(), "workloads": {}}
    rec["note"] = ("HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                   "dispatch), each scaled by bytes/counter of the pack kernel in the same run; "
                   "averaged over the workload's layer types")
    wl_rec = {}
    for k in sorted({k for lay in per_layer.values() for k in lay["kernels"]}):
        vals = [lay["kernels"][k] for lay in per_layer.values() if "bytes_per_launch" in lay["kernels"].get(k, {})]
        if vals:
            wl_rec[k] = {"bytes_per_launch": round(sum(x["bytes_per_launch"] for x in vals) / len(vals)),
                         "fetch_kib": round(sum(x["fetch_kib"] for x in vals) / len(vals), 1),
                         "write_kib": round(sum(x["write_kib"] for x in vals) / len(vals), 1)}
    rec["workloads"][case.name] = wl_rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")

    out = os.path.join(PROFILES, f"{case.name}_kernels.md")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 per-kernel summary: simulated Ulysses step, workload {case.name}\n\n")
        f.write(f"P={case.P}, B={case.B}, S={case.S}, Hq/Hkv={case.Hq}/{case.Hkv}, D={case.D}, "
                f"layers {[v.name for v in case.variants]}, sink={case.sink}.\n\n")
        f.write("Commands (run from /tmp with TMPDIR=/tmp; R = repository root):\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        f.write("\n## kernel trace of the benchmark command (--kernel-trace --stats)\n\n")
        f.write("| kernel | short name | calls | avg us | total us | % |\n|---|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| `{r['Name']}` | {_rocprof_name(r['Name'])} | {r['Calls']} | "
                    f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                    f"{float(r['Percentage']):.1f} |\n")
        for lname, lay in per_layer.items():
            f.write(f"\n## layer `{lname}`: utilisation per kernel (counter passes of this layer type)\n\n")
            src = (f"a kernel trace of this layer type alone (`{lname}/trace`)"
                   if lay["avg_us"] is not avg_all else "the benchmark's kernel trace")
            f.write(f"Durations (avg us) from {src}.  "
                    "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles): over the traced "
                    "average duration at the nominal 2.4 GHz, and over GRBM_GUI_ACTIVE cycles (the "
                    "clock the dispatch ran at: GRBM_GUI_ACTIVE over the counter pass's own durations of "
                    "the same dispatches; each kernel's first dispatch left out; for dispatches of a few "
                    "tens of us the counter also takes in the dispatch's set-up, and the clock it gives "
                    "exceeds the chip's 2.4 GHz).  HBM bytes: FETCH_SIZE x "
                    f"{lay['fetch_scale']} + WRITE_SIZE x {lay['write_scale']} (KiB, scaled by the "
                    "pack kernel's known bytes).  Compulsory bytes: every operand read and every "
                    "result written once.\n\n")
            f.write("LDS busy = SQ_LDS_IDX_ACTIVE / (256 CUs x cycles at the run clock); LDS bytes "
                    "read = SQ_INSTS_LDS_LOAD_BANDWIDTH x 64.\n\n")
            f.write("| kernel | avg us | MFMA busy @2.4 GHz | MFMA busy @run clock | run clock GHz | "
                    "VALU / MFMA instr | LDS instr / MFMA | LDS busy | LDS bytes read / MFMA | "
                    "LDS bank conflicts | HBM MB/launch | "
                    "HBM GB/s | HBM / compulsory bytes |\n|" + "---|" * 13 + "\n")
            for k, r in lay["kernels"].items():
                sqk = r["sq"]
                us = lay["avg_us"].get(k)
                busy = sqk.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
                gui = sqk.get("GRBM_GUI_ACTIVE")
                mfma = sqk.get("SQ_INSTS_MFMA", 0.0)
                u_nom = busy / (SIMDS * us * 1e-6 * PEAK_CLOCK_GHZ * 1e9) if us else None
                # GRBM_GUI_ACTIVE reads the sum over the 8 XCDs' busy cycles
                u_run = busy / (SIMDS * gui / XCDS) if gui else None
                cus = sqk.get("_us")  # the same dispatches' own durations
                clk = gui / XCDS / (cus * 1e-6) / 1e9 if (gui and cus) else None
                lds_act, lds_rd = sqk.get("SQ_LDS_IDX_ACTIVE"), sqk.get("SQ_INSTS_LDS_LOAD_BANDWIDTH")
                u_lds = lds_act / (CUS * gui / XCDS) if (gui and lds_act is not None) else None
                rd_mfma = 64 * lds_rd / mfma if (mfma and lds_rd is not None) else None
                hbm = r.get("bytes_per_launch")
                alg = alg_bytes_per_launch(case, k)
                fmt = lambda x, p="{:.3f}": "" if x is None else p.format(x)
                f.write(f"| {k} | {fmt(us, '{:.1f}')} | {fmt(u_nom)} | {fmt(u_run)} | {fmt(clk, '{:.2f}')} | "
                        f"{fmt(sqk.get('SQ_INSTS_VALU', 0) / mfma if mfma else None, '{:.2f}')} | "
                        f"{fmt(sqk.get('SQ_INSTS_LDS', 0) / mfma if mfma else None, '{:.2f}')} | "
                        f"{fmt(u_lds)} | {fmt(rd_mfma, '{:.0f}')} | "
                        f"{sqk.get('SQ_LDS_BANK_CONFLICT', 0):.0f} | {fmt(hbm / 1e6 if hbm else None, '{:.1f}')} | "
                        f"{fmt(hbm / (us * 1e-6) / 1e9 if (hbm and us) else None, '{:.0f}')} | "
                        f"{fmt(hbm / alg if (hbm and alg) else None, '{:.2f}')} |\n")
            cols = sorted({c for r in lay["kernels"].values() for c in r["sq"] if not c.startswith("_")})
            f.write("\nRaw counters, average per dispatch:\n\n| kernel | " + " | ".join(cols) +
                    " | FETCH_SIZE KiB | WRITE_SIZE KiB |\n|" + "---|" * (len(cols) + 3) + "\n")
            for k, r in lay["kernels"].items():
                f.write(f"| {k} | " + " | ".join(f"{r['sq'].get(c, float('nan')):.0f}" for c in cols) +
                        f" | {r.get('fetch_kib', '')} | {r.get('write_kib', '')} |\n")
    print(open(out).read())


def _visible_counts(docs, S_total, causal, wl, wr, idx, keys_side):
    """Per flattened token in `idx`: visible keys of that query (keys_side False)
    or queries that see that key (keys_side True), under the mask rules."""
    import numpy as np
    starts = np.cumsum([0] + list(docs))
    out = []
    for t in idx:
        d = int(np.searchsorted(starts, t, side="right") - 1)
        lo, hi = int(starts[d]), int(starts[d + 1])
        if not keys_side:   # keys j visible to query t
            a, b = lo, hi
            if causal:
                b = min(b, t + 1)
            if wl >= 0:
                a = max(a, t - wl)
            if wr >= 0:
                b = min(b, t + wr + 1)
        else:               # queries i that see key t
            a, b = lo, hi
            if causal:
                a = max(a, t)
            if wl >= 0:
                b = min(b, t + wl + 1)
            if wr >= 0:
                a = max(a, t - wr)
        out.append(max(0, b - a))
    return out


def cpu_baseline_subset(inp, n_rows, n_keys):
    """The fp64 CPU oracle, as it stands, on a bounded sample of rank 0's share
    of a long workload: O, LSE and dQ of `n_rows` query rows stratified over the
    sequence (one seeded row in each of n_rows equal strata), and dK, dV of the
    last `n_keys` keys, for every query head of rank 0 and every layer type.
    Credited FLOPs: 6*D per visible pair on each side (forward 4*D + dQ 2*D
    for the rows; dP, dV, dK for the keys), as the GPU figure credits them;
    the oracle's recompute of the statistics of the rows a key needs is timed
    but not credited."""
    import oracle
    import torch
    from ulysses_inputs import seq_shards
    c = inp.case
    P, D, S, hq = c.P, c.D, c.S, c.hq
    kv_pack = oracle.pack_replicated if c.Hkv < P else oracle.pack
    qh = oracle.pack(seq_shards(inp.q, P))[0]
    kh, vh = kv_pack(seq_shards(inp.k, P))[0], kv_pack(seq_shards(inp.v, P))[0]
    dh = oracle.pack(seq_shards(inp.dout, P))[0]
    sk = None if inp.sink is None else inp.sink[:hq].contiguous()
    cu = None
    if inp.doc_lengths is not None:
        cu, _, _ = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    docs = docs_of(inp)
    T = c.B * S
    g = torch.Generator().manual_seed(4242)
    rows = [int(k * T // n_rows + torch.randint(0, max(1, T // n_rows), (1,), generator=g))
            for k in range(n_rows)]
    keys = list(range(T - n_keys, T))
    log(f"cpu baseline: oracle on rank 0 ({hq} query heads), {n_rows} stratified rows and the "
        f"last {n_keys} keys, {oracle.num_threads()} threads")
    flops = 0
    t0 = time.perf_counter()
    for v in c.variants:
        kw = dict(sink=sk, cu=cu, causal=v.causal, window_left=v.window_left,
                  window_right=v.window_right)
        oracle.attn_fwd(qh, kh, vh, rows=rows, **kw)
        oracle.attn_bwd(qh, kh, vh, dh, qrows=rows, want_dkdv=False, want_dsink=False, **kw)
        oracle.attn_bwd(qh, kh, vh, dh, krows=keys, want_dq=False, want_dsink=False, **kw)
        pr = sum(_visible_counts(docs, T, v.causal, v.window_left, v.window_right, rows, False))
        pk = sum(_visible_counts(docs, T, v.causal, v.window_left, v.window_right, keys, True))
        flops += 6 * D * (pr + pk) * hq
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2), "subset": True,
            "sample": (f"subset of rank 0's share (all {hq} query heads, layers "
                       f"{[v.name for v in c.variants]}): O, LSE and dQ of {n_rows} query rows "
                       f"stratified over S={S}, dK and dV of the last {n_keys} keys; fp64; "
                       f"{flops / 1e9:.1f} GFLOP credited at 6*D per visible pair and side")}


def cpu_baseline(inp, ranks, n_heads):
    """The fp64 CPU oracle, as it stands, on a bounded sample of the same workload:
    the first ``n_heads`` query heads (with their KV heads) of each rank in
    ``ranks``, full sequence, every layer type, forward and backward."""
    import oracle
    from ulysses_inputs import seq_shards
    c = inp.case
    P, D = c.P, c.D
    G = c.Hq // c.Hkv
    hq = c.Hq // P
    n_heads = min(hq, max(G, (n_heads // G) * G))
    nkv = max(1, n_heads // G)
    kv_pack = oracle.pack_replicated if c.Hkv < P else oracle.pack
    packed = [oracle.pack(seq_shards(inp.q, P)), kv_pack(seq_shards(inp.k, P)),
              kv_pack(seq_shards(inp.v, P)), oracle.pack(seq_shards(inp.dout, P))]
    cu = None
    if inp.doc_lengths is not None:
        cu, _, _ = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    docs = docs_of(inp)
    flops = 0
    log(f"cpu baseline: oracle on ranks {ranks}, {n_heads} query heads each, "
        f"{oracle.num_threads()} threads")
    t0 = time.perf_counter()
    for r in ranks:
        qh = packed[0][r][:, :, :n_heads].contiguous()
        kh = packed[1][r][:, :, :nkv].contiguous()
        vh = packed[2][r][:, :, :nkv].contiguous()
        dh = packed[3][r][:, :, :n_heads].contiguous()
        sk = None if inp.sink is None else inp.sink[r * (c.Hq // P):][:n_heads].contiguous()
        for v in c.variants:
            kw = dict(sink=sk, cu=cu, causal=v.causal, window_left=v.window_left,
                      window_right=v.window_right)
            oracle.attn_fwd(qh, kh, vh, **kw)
            oracle.attn_bwd(qh, kh, vh, dh, **kw)
            flops += 12 * D * visible_pairs(docs, v.causal, v.window_left, v.window_right) * n_heads
    dt = time.perf_counter() - t0
    whole = len(ranks) == P and n_heads == c.Hq // P
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": (f"{'the whole step: ' if whole else ''}ranks {ranks}, {n_heads} of "
                       f"{c.Hq // P} query heads each ({nkv} KV head(s)), full sequence S={c.S}, "
                       f"layers {[v.name for v in c.variants]}, attention fwd+bwd in fp64")}


if __name__ == "__main__":
    main()
