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
DEFAULT_WORKLOAD = 2         # S=4096, 12 heads, D=128, full + causal layers, P=2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5],
                    help="which of the five simulated workloads (default: the S=4096 one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=2,
                    help="query heads of rank 0 the CPU oracle baseline runs")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of a captured HIP graph of the step")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the P Ulysses ranks are simulated in memory "
              f"on that GPU, so --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import ulysses_sequence_attention_rank_amd as uly
    from ulysses_inputs import CONFIGS, make_inputs, seq_shards
    from ulysses_sequence_attention_rank_amd import sim

    if not os.path.exists(uly.lib_path()):
        from ulysses_sequence_attention_rank_amd import build
        build.build()
    uly.load()

    case = CONFIGS[args.workload]
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

    # per-kernel durations: the same steps launched eagerly, each kernel
    # bracketed by HIP events on the stream it runs on
    log(f"per-kernel timing over {args.steps} eager steps")
    uly.profile_start(max_launches=64 * args.steps * len(case.variants) * P + 64)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    uly.profile_stop()
    kern = uly.profile_report()

    docs = docs_of(inp)
    credit = kernel_credit(case, docs)
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
    # layout permutation: every element read once and written once
    elem_q = case.B * case.S * case.Hq * case.D
    elem_kv = case.B * case.S * case.Hkv * case.D
    pack_bytes = 2 * 2 * (2 * elem_q + 2 * elem_kv)   # Q, dO (Hq) and K, V (Hkv), per layer
    unpack_bytes = 2 * 2 * (2 * elem_q + 2 * elem_kv)  # O, dQ (Hq) and dK, dV (Hkv)
    nl = len(case.variants) * args.steps
    if "a2a_pack" in kern:
        rows["a2a_pack"]["gbps"] = pack_bytes * nl / (kern["a2a_pack"][1] * 1e-3) / 1e9
        rows["a2a_pack"]["frac_of_peak"] = rows["a2a_pack"]["gbps"] / PEAK_HBM_GBPS
    if "a2a_unpack" in kern:
        rows["a2a_unpack"]["gbps"] = unpack_bytes * nl / (kern["a2a_unpack"][1] * 1e-3) / 1e9
    attn_ms = sum(v[1] for k, v in kern.items() if k.startswith("attn_"))
    attn_tflops = step_flops * args.steps / (attn_ms * 1e-3) / 1e12

    # roofline of the kernel that takes the most time in the step
    dom = max(("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"), key=lambda k: kern.get(k, (0, 0))[1])
    per_launch_flops = attn_credit[dom] / kern[dom][0]
    achieved = per_launch_flops / (kern[dom][1] / kern[dom][0] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": per_launch_flops,
                "avg_launch_ms": round(kern[dom][1] / kern[dom][0], 5)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_heads)

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
        "data": "synthetic",
        "config": {"workload": case.name, "P": P, "B": case.B, "S": case.S, "Hq": case.Hq,
                   "Hkv": case.Hkv, "D": case.D, "layers": [v.name for v in case.variants],
                   "sink": case.sink, "packed_docs": len(docs) if inp.doc_lengths else None},
        "execution": "hip_graph" if graph is not None else "eager",
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "attn_tflops": round(attn_tflops, 2),
        "pack_gbps": round(rows.get("a2a_pack", {}).get("gbps", 0.0), 1),
        "pack_frac_of_hbm": round(rows.get("a2a_pack", {}).get("frac_of_peak", 0.0), 4),
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for k, r in rows.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(inp, n_heads):
    """The fp64 CPU oracle, as it stands, on a bounded sample of the same workload:
    rank 0's first ``n_heads`` query heads (with their KV heads), full sequence,
    every layer type, forward and backward."""
    import torch

    import oracle
    from ulysses_inputs import seq_shards
    c = inp.case
    P, D = c.P, c.D
    G = c.Hq // c.Hkv
    n_heads = max(G, (n_heads // G) * G)
    nkv = n_heads // G
    qh = oracle.pack(seq_shards(inp.q, P))[0][:, :, :n_heads].contiguous()
    kh = oracle.pack(seq_shards(inp.k, P))[0][:, :, :nkv].contiguous()
    vh = oracle.pack(seq_shards(inp.v, P))[0][:, :, :nkv].contiguous()
    dh = oracle.pack(seq_shards(inp.dout, P))[0][:, :, :n_heads].contiguous()
    sk = None if inp.sink is None else inp.sink[:n_heads].contiguous()
    cu = None
    if inp.doc_lengths is not None:
        cu, _, _ = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    docs = docs_of(inp)
    flops = 0
    log(f"cpu baseline: oracle on rank 0, {n_heads} query heads, {oracle.num_threads()} threads")
    t0 = time.perf_counter()
    for v in c.variants:
        kw = dict(sink=sk, cu=cu, causal=v.causal, window_left=v.window_left,
                  window_right=v.window_right)
        oracle.attn_fwd(qh, kh, vh, **kw)
        oracle.attn_bwd(qh, kh, vh, dh, **kw)
        flops += 12 * D * visible_pairs(docs, v.causal, v.window_left, v.window_right) * n_heads
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": (f"rank 0, {n_heads} of {c.hq} query heads ({nkv} KV head), full sequence "
                       f"S={c.S}, layers {[v.name for v in c.variants]}, fwd+bwd in fp64")}


if __name__ == "__main__":
    main()
