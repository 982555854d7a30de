"""Benchmark of the MoE verify step on one MI355X.

One step = one moe_verify_step call over one batch: 12 MoE layers (64 routed
top-6 + 2 shared SwiGLU experts), final RMSNorm, LM-head argmax over 129,280
rows and the accept rule.  Weights, hidden states and drafts are seeded
synthetic data resident in HBM before timing starts; drafts equal the
verifier's argmax (from an untimed pass) with the workload's probability.

Prints one JSON line.  Default workload: batch 1, K = 3 (4 token rows).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "committed tokens/s (12-layer MoE verify, K=3) + % of HBM/MFMA roofline"
# HBM bytes per b1_k3 verify step measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
# (scaled by a 1 GiB copy; profiles/verify_step_b1_k3_hbm_counters.txt) on the
# kernel sources with this digest; reported only while the sources match.
MEASURED_TRAFFIC = {"b1_k3": {"csrc_sha256_16": "f4f7933c369c1699", "bytes_per_step": 2.1783e9}}
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def step_bytes(dims, ids, T):
    """Algorithmic HBM bytes of one verify step: every routed expert hit at
    least once plus the shared experts, the router and norm vectors, the LM
    head, and the hidden rows in and out."""
    es = 2 if dims.dtype == "bf16" else 4
    d, F, E = dims.d_model, dims.d_ff, dims.n_routed
    expert = 3 * F * d * es
    distinct = [len(np.unique(ids[layer])) for layer in range(dims.n_layers)]
    total = sum(n + dims.n_shared for n in distinct) * expert
    total += dims.n_layers * (E * d + d) * es          # router + ffn norm
    total += dims.vocab * d * es + d * es              # LM head + final norm
    total += 2 * T * d * es                            # h in, h out
    return total, distinct


def csrc_digest():
    import glob
    import hashlib

    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "speculative_decode_verification_router_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b1_k3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-baseline-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time graph replays")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run device copies of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify step is sized for a single MI355X "
              "and multi-GPU runs are not part of this library", file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": args.steps}), flush=True)
        return 0

    from speculative_decode_verification_router_amd import binding as bd
    from speculative_decode_verification_router_amd import synth

    bd.load()
    wl = synth.WORKLOADS[args.workload]
    if wl.batch == 0:
        raise SystemExit(f"{wl.name} has no LM head / drafts; not a verify-step workload")
    dims = wl.dims
    B, K = wl.batch, wl.k_draft
    T = B * (K + 1)
    torch.cuda.set_device(0)
    print(f"[bench] generating {wl.name} weights", file=sys.stderr, flush=True)
    W = synth.workload_weights(wl, seed=args.seed)
    model = bd.DeviceModel(dims, W, max_tokens=T)
    h_np = synth.workload_hidden(wl, seed=args.seed)
    h = bd.to_device(h_np)

    # untimed pass: the argmax does not depend on the drafts
    zero = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    pre = bd.run_verify_step(model, h, zero, B, K, routing=True)
    torch.cuda.synchronize()
    g = bd.to_host(pre["argmax"]).reshape(B, K + 1)
    ids = bd.to_host(pre["topk_ids"])
    drafts_np = synth.make_drafts(g, wl.match_p, dims.vocab, seed=args.seed)
    drafts = bd.to_device(drafts_np)

    out = bd.run_verify_step(model, h, drafts, B, K)

    def step(stream):
        bd.moe_verify_step(model.cfg, model.weights, B, K, h, drafts, out["h_out"], out["argmax"],
                           out["n_accepted"], out["committed"], out["n_committed"], None,
                           model.ws, model.ws_bytes, stream)

    run = step
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                step(side)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream())
        run = lambda stream: graph.replay()  # noqa: E731
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        run(stream)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run(stream)
    t_enq = time.perf_counter() - t0
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    committed_per_step = int(bd.to_host(out["n_committed"]).sum())
    value = committed_per_step / (ms * 1e-3)

    nbytes, distinct = step_bytes(dims, ids, T)
    achieved = nbytes / (ms * 1e-3) / 1e9
    meas = MEASURED_TRAFFIC.get(wl.name)
    traffic = meas["bytes_per_step"] if meas and meas["csrc_sha256_16"] == csrc_digest() else None
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        "kernel": "whole verify step (12 x [route, gate_up, down] + final norm + lm_head + accept)",
        "algorithmic_bytes_per_step": int(nbytes),
        "distinct_experts_per_layer": distinct,
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, W, h_np, drafts_np, args.cpu_baseline_steps)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "committed tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; weights N(0,0.02), hidden N(0,1), drafts = argmax w.p. p)",
        "config": {"workload": wl.name, "batch": B, "k_draft": K, "tokens": T,
                   "layers": dims.n_layers, "d_model": dims.d_model, "d_ff": dims.d_ff,
                   "experts": f"{dims.n_routed} routed top-{dims.top_k} + {dims.n_shared} shared",
                   "vocab": dims.vocab, "match_p": wl.match_p,
                   "committed_per_step": committed_per_step},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 4),
        "host_enqueue_ms_per_step": round(t_enq / args.steps * 1e3, 4),
        "graph": bool(args.graph),
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(wl, W, h_np, drafts_np, steps):
    """The CPU oracle timed on a bounded sample of the same workload."""
    from oracle import moe_oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    committed = 0
    for _ in range(steps):
        r = O.verify_step(h_np, drafts_np, W, wl.dims)
        committed += int(np.sum(r["n_committed"]))
    dt = time.perf_counter() - t0
    return {"value": round(committed / dt, 3), "unit": "committed tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{steps} verify steps of {wl.name} (float64 numpy oracle, same inputs)",
            "s_per_step": round(dt / steps, 3)}


if __name__ == "__main__":
    sys.exit(main())
