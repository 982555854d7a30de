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
# HBM bytes per b1_k3 and c32_k3 verify step and per b1_k3 mtp_draft call,
# measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (scaled by a 1 GiB copy;
# profiles/verify_step_{b1,c32}_k3_hbm_counters.txt, profiles/mtp_draft_b1_k3_hbm_counters.txt)
# on the kernel sources whose code (comments aside) has this digest; reported
# only while the code matches.
MEASURED_TRAFFIC = {"b1_k3": {"csrc_sha256_16": "c7b7512a5d65c16d", "bytes_per_step": 2.1844e9},
                    "c32_k3": {"csrc_sha256_16": "c7b7512a5d65c16d", "bytes_per_step": 6.4241e9},
                    "b1_k3_draft": {"csrc_sha256_16": "c7b7512a5d65c16d", "bytes_per_step": 1.0586e9}}
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
    """Digest of the kernel sources' code: line comments, block comments and
    blank lines are left out, so an edit of comments alone keeps it."""
    import glob
    import hashlib
    import re

    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "speculative_decode_verification_router_amd", "csrc", "*"))):
        with open(p, encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
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
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the device-copy ceiling measurement (for profiler runs of the step alone)")
    ap.add_argument("--one-launch", action="store_true",
                    help="time moe_verify_step_one_launch (batches of up to 8 rows) instead of moe_verify_step")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time graph replays")
    ap.add_argument("--cpu-baseline-rows", type=int, default=8,
                    help="stack workloads: rows the oracle pushes through the stack")
    ap.add_argument("--loop", action="store_true",
                    help="run the decode loop (sequences until --loop-tokens committed each)")
    ap.add_argument("--loop-tokens", type=int, default=1085)
    ap.add_argument("--loop-lengths", choices=("equal", "mixed"), default="equal",
                    help="decode loop: every sequence commits --loop-tokens tokens, or a seeded uniform "
                         "draw from 1 .. 2 * loop-tokens - 1 (the same mean) per sequence")
    ap.add_argument("--draft", action="store_true",
                    help="time the FastMTP draft block (mtp_draft) for the workload's B and K")
    ap.add_argument("--choose-k", action="store_true",
                    help="time a draft + verify step for K = 0..3 and report the draft length "
                         "mv_choose_k picks across acceptance rates")
    ap.add_argument("--with-draft", action="store_true",
                    help="decode loop: also run the draft block's work in every step (timed); the verify "
                         "step still takes synthetic drafts of acceptance p, so this times drafting and "
                         "does not measure a speculative speedup")
    ap.add_argument("--adaptive-k", action="store_true",
                    help="decode loop: choose K per step with mv_choose_k from step costs measured per batch")
    ap.add_argument("--loop-sweep", action="store_true",
                    help="decode loop: fixed K = 0..3 and adaptive K at p = 0.4, 0.6, 0.8")
    ap.add_argument("--k-draft", type=int, default=None)
    ap.add_argument("--match-p", type=float, default=None)
    ap.add_argument("--cold", action="store_true",
                    help="verify step and stack: time each step alone after a 1 GiB cache scrub "
                         "and report the median")
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
    torch.cuda.set_device(0)
    print(f"[bench] generating {wl.name} weights", file=sys.stderr, flush=True)
    W = synth.workload_weights(wl, seed=args.seed)
    if wl.batch == 0:
        line = bench_stack(args, wl, W, bd, synth, torch)
    elif args.draft:
        line = bench_draft(args, wl, W, bd, synth, torch)
    elif args.choose_k:
        line = bench_choose_k(args, wl, W, bd, synth, torch)
    elif args.loop or args.loop_sweep:
        line = bench_loop(args, wl, W, bd, synth, torch)
    else:
        line = bench_verify(args, wl, W, bd, synth, torch)
    print(json.dumps(line), flush=True)
    return 0


def _cores():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


SCRUB_BYTES = 1 << 30


def _timed(run, stream, steps, warmup, torch, cold=False):
    """Warm up, then time `steps` calls of run(stream) with events on `stream`.

    cold: before every step a 1 GiB device copy (512 MiB read, 512 MiB
    written, outside the events) evicts the step's data from L2 and the 256 MB
    memory-side cache; each step is timed alone and the median is returned."""
    for _ in range(warmup):
        run(stream)
    if cold:
        src = torch.ones(SCRUB_BYTES // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for a, b in evs:
                dst.copy_(src)
                a.record(stream)
                run(stream)
                b.record(stream)
        t_enq = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return float(np.median([a.elapsed_time(b) for a, b in evs])), wall, t_enq
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        run(stream)
    t_enq = time.perf_counter() - t0
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall, t_enq


def _timing(args):
    if args.cold:
        return "cold: median of steps timed alone, each after a 1 GiB cache scrub"
    return "warm: back-to-back steps between two events"


def _header(args, wl):
    return {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": wl.dims.dtype}


def copy_ceiling(torch, mib=512, reps=10):
    """Device-to-device copy rate, GB/s of bytes read plus bytes written: the
    ceiling a streaming kernel of the same box can be held against (the copy
    reads and writes equal amounts; the verify step mostly reads)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def bench_verify(args, wl, W, bd, synth, torch):
    dims = wl.dims
    B, K = wl.batch, wl.k_draft
    T = B * (K + 1)
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

    entry = bd.moe_verify_step_one_launch if args.one_launch else bd.moe_verify_step

    def step(stream):
        entry(model.cfg, model.weights, B, K, h, drafts, out["h_out"], out["argmax"],
              out["n_accepted"], out["committed"], out["n_committed"], None,
              model.ws, model.ws_bytes, stream)

    run = step
    if args.graph and args.one_launch:
        raise SystemExit("--graph and --one-launch are separate measurements")
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
    ms, wall, t_enq = _timed(run, stream, args.steps, args.warmup, torch, cold=args.cold)
    timed_draw = int(bd.to_host(out["n_committed"]).sum())
    # the step's work does not depend on the draft values: committed tokens per
    # step are the mean over many seeded draws of the drafts, each through the
    # library's accept rule on the step's argmax
    draws = _mean_commits(bd, torch, g, wl.match_p, dims.vocab, args.seed, n=4096)
    committed_per_step = draws * B
    q = wl.match_p + (1 - wl.match_p) / dims.vocab
    closed = B * sum(q ** i for i in range(K + 1))
    value = committed_per_step / (ms * 1e-3)

    nbytes, distinct = step_bytes(dims, ids, T)
    achieved = nbytes / (ms * 1e-3) / 1e9
    meas = MEASURED_TRAFFIC.get(wl.name)
    traffic = meas["bytes_per_step"] if meas and meas["csrc_sha256_16"] == csrc_digest() else None
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        "kernel": "whole verify step (12 x [routing, expert FFN] + final norm + lm_head with the accept rule)",
        "algorithmic_bytes_per_step": int(nbytes),
        "distinct_experts_per_layer": distinct,
    }
    if not args.no_copy_ceiling:
        copy_gbs = copy_ceiling(torch)
        roofline.update({"copy_gbs": copy_gbs, "frac_of_copy": round(achieved / copy_gbs, 4)})
    status = bd.step_status(model)
    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, W, h_np, drafts_np, args.cpu_baseline_steps)
        parity = forced_parity(bd, torch, model, W, dims, h, B, K, pre, drafts_np, out)
    line = {"metric": METRIC, "value": round(value, 1), "unit": "committed tokens/s"}
    line.update(_header(args, wl))
    line.update({
        "ms_per_step": round(ms, 4),
        "data": "synthetic (seeded; weights N(0,0.02), hidden N(0,1), drafts = argmax w.p. p)",
        "config": {"workload": wl.name, "batch": B, "k_draft": K, "tokens": T,
                   "layers": dims.n_layers, "d_model": dims.d_model, "d_ff": dims.d_ff,
                   "experts": f"{dims.n_routed} routed top-{dims.top_k} + {dims.n_shared} shared",
                   "vocab": dims.vocab, "match_p": wl.match_p,
                   "committed_per_step": round(committed_per_step, 4),
                   "committed_per_step_basis": "mean over 4096 seeded draft draws on the step's argmax",
                   "committed_per_step_closed_form": round(closed, 4),
                   "committed_timed_draw": timed_draw},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "wait_status": status,
        "wall_s_timed_region": round(wall, 4),
        "host_enqueue_ms_per_step": round(t_enq / args.steps * 1e3, 4),
        "graph": bool(args.graph),
        "entry_point": "moe_verify_step_one_launch" if args.one_launch else "moe_verify_step",
        "timing": _timing(args),
    })
    return line


def stack_flops(dims, T):
    """Algorithmic flops of the MoE stack on T rows: router GEMV plus
    gate/up and down of the k routed and S shared experts per row."""
    d, F = dims.d_model, dims.d_ff
    per_row = 2 * d * dims.n_routed + (dims.top_k + dims.n_shared) * (2 * d * 2 * F + 2 * F * d)
    return dims.n_layers * T * per_row


def bench_stack(args, wl, W, bd, synth, torch):
    """Token batch through the 12-layer stack (no LM head): one step = one
    pass of every layer, each a moe_layer_forward call; MFMA-bound."""
    dims = wl.dims
    T = wl.tokens
    model = bd.DeviceModel(dims, W, max_tokens=T)
    h_np = synth.workload_hidden(wl, seed=args.seed)
    h0 = bd.to_device(h_np)
    h1 = torch.empty_like(h0)

    def step(stream):
        for layer in range(dims.n_layers):
            bd.moe_layer_forward(model.cfg, model.weights, layer, T, h0 if layer == 0 else h1, h1,
                                 None, None, None, model.ws, model.ws_bytes, stream)

    stream = torch.cuda.current_stream()
    ms, wall, t_enq = _timed(step, stream, args.steps, args.warmup, torch, cold=args.cold)
    flops = stack_flops(dims, T)
    achieved = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O

        rows = max(1, args.cpu_baseline_rows)
        t0 = time.perf_counter()
        O.forward_tokens(h_np[:rows], W, dims, lm_head=False)
        dt = time.perf_counter() - t0
        cpu = {"value": round(rows / dt, 3), "unit": "tokens/s", "cores": _cores(), "kind": "oracle",
               "sample": f"first {rows} of the {T} rows through all {dims.n_layers} layers "
                         "(float64 numpy oracle; rows are independent)",
               "s_per_row": round(dt / rows, 4)}
    line = {"metric": "tokens/s through the 12-layer MoE stack + % of bf16 MFMA peak",
            "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s"}
    line.update(_header(args, wl))
    line.update({
        "ms_per_step": round(ms, 4),
        "data": "synthetic (seeded; weights N(0,0.02), hidden N(0,1))",
        "config": {"workload": wl.name, "tokens": T, "layers": dims.n_layers,
                   "d_model": dims.d_model, "d_ff": dims.d_ff,
                   "experts": f"{dims.n_routed} routed top-{dims.top_k} + {dims.n_shared} shared"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "whole stack (12 x moe_layer_forward)",
                     "algorithmic_flops_per_step": flops},
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 4),
        "host_enqueue_ms_per_step": round(t_enq / args.steps * 1e3, 4),
        "timing": _timing(args),
    })
    return line


def _step_costs(bd, torch, model, mtp, dims, Bs, k_max, steps, warmup, seed, code):
    """Measured time (ms) of one decode-loop step for B sequences and K drafts,
    for B in Bs and K = 0..k_max: moe_verify_step over B (K + 1) rows, after
    the draft block's K positions when mtp is given."""
    from speculative_decode_verification_router_amd import synth

    B_max = max(Bs)
    h = bd.to_device(synth.make_hidden(dims, B_max * (k_max + 1), seed, code))
    tok = torch.zeros(B_max, dtype=torch.int32, device="cuda")
    d_out = torch.zeros(B_max * max(k_max, 1), dtype=torch.int32, device="cuda")
    outs = bd.run_verify_step(model, h, d_out, B_max, k_max)
    cost = {}
    for B in Bs:
        row = []
        for K in range(k_max + 1):
            T = B * (K + 1)
            first = torch.arange(B, device="cuda") * (K + 1)

            def step(stream, B=B, K=K, T=T, first=first):
                if mtp is not None and K:
                    bd.mtp_draft(model.cfg, model.weights, mtp.weights, B, K, h.index_select(0, first), tok[:B],
                                 d_out, None, mtp.ws, mtp.ws_bytes, stream)
                bd.moe_verify_step(model.cfg, model.weights, B, K, h[:T], d_out, outs["h_out"], outs["argmax"],
                                   outs["n_accepted"], outs["committed"], outs["n_committed"], None, model.ws,
                                   model.ws_bytes, stream)

            ms, _, _ = _timed(step, torch.cuda.current_stream(), steps, warmup, torch)
            row.append(ms)
        cost[B] = row
    return cost


def _run_loop_pair(bd, torch, synth, DL, model, dims, wl, h_start, B0, target, policy, k_max, p, seed, mtp):
    """Rehearse the loop (drafts drawn from each step's argmax), then replay
    the same steps timed on the host clock.  Returns (wall s, result)."""
    before = None
    if mtp is not None:
        B_first = torch.arange(B0, device="cuda")
        tok = torch.zeros(B0, dtype=torch.int32, device="cuda")
        d_scratch = torch.empty(B0 * 16, dtype=torch.int32, device="cuda")

        def before(B, K, h_in):
            # the draft block's work for this step, from each sequence's first row; its drafts
            # are computed and timed, but the verify step takes the planned synthetic ones
            if K:
                hsel = h_in.index_select(0, B_first[:B] * (K + 1))
                bd.mtp_draft(model.cfg, model.weights, mtp.weights, B, K, hsel, tok[:B], d_scratch, None,
                             mtp.ws, mtp.ws_bytes, None)

    def draw(step, g, seqs):
        return synth.make_drafts(g, p, dims.vocab, seed=seed, step=step, code=wl.code)

    reh = DL.run_loop(bd, model, h_start, B0, target, policy, k_max, draw_drafts=draw, before_verify=before)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = DL.run_loop(bd, model, h_start, B0, target, policy, k_max, plan=reh.steps, before_verify=before)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert len(res.steps) == len(reh.steps) and res.committed == reh.committed
    return wall, res


def bench_loop(args, wl, W, bd, synth, torch):
    """Decode loop: every sequence runs until it has committed `loop_tokens`
    tokens; each step's output hidden rows are the next step's input rows,
    finished sequences drop out (decode_loop.run_loop).  Drafts are drawn in
    an untimed rehearsal of the same loop (the argmax does not depend on the
    drafts); the timed replay includes the per-step host read of the commit
    counts.  --adaptive-k chooses K per step with mv_choose_k from step costs
    measured per batch size; --loop-sweep runs fixed K = 0..3 and adaptive K
    for p in {0.4, 0.6, 0.8}."""
    from speculative_decode_verification_router_amd import decode_loop as DL

    dims = wl.dims
    B0 = wl.batch
    target = args.loop_tokens
    if args.loop_lengths == "mixed":
        target = np.random.default_rng(args.seed + 17).integers(1, 2 * args.loop_tokens, B0)
    total_tokens = int(np.sum(np.broadcast_to(target, (B0,))))
    k_max = 3
    model = bd.DeviceModel(dims, W, max_tokens=B0 * (k_max + 1))
    h_np = synth.make_hidden(dims, B0 * (k_max + 1), args.seed, wl.code)
    h_start = bd.to_device(h_np)
    mtp = None
    if args.with_draft:
        mtp = bd.DeviceMtp(dims, synth.make_mtp_weights(dims, seed=args.seed, sigma=wl.weight_sigma),
                           max_rows=B0)
    need_costs = args.adaptive_k or args.loop_sweep
    Bs = sorted({1, 2, 4, 8, 16, B0})
    cost = _step_costs(bd, torch, model, mtp, dims, Bs, k_max, 20, 3, args.seed, wl.code) if need_costs else None

    def one(K, p, adaptive):
        q = p + (1 - p) / dims.vocab
        policy = DL.AdaptiveK(bd, q, cost) if adaptive else DL.FixedK(K)
        print(f"[bench] loop {'adaptive K' if adaptive else f'K={K}'}, p={p}", file=sys.stderr, flush=True)
        wall, res = _run_loop_pair(bd, torch, synth, DL, model, dims, wl, h_start, B0, target, policy, k_max, p,
                                   args.seed, mtp)
        row = {"k": "adaptive" if adaptive else K, "p": p, "verify_steps": len(res.steps),
               "committed_tok_s": round(res.committed / wall, 1), "ms_per_step": round(wall / len(res.steps) * 1e3, 4),
               "committed_per_seq_step": round(res.per_seq_step, 4), "rows_verified": res.rows,
               "steps_per_k": {str(k): v for k, v in sorted(res.k_hist.items())}, "wall_s": round(wall, 4)}
        if cost is not None:
            pred = sum(DL.AdaptiveK(bd, q, cost).costs_at(len(st.seqs))[st.K] for st in res.steps) * 1e-3
            row["predicted_wall_s"] = round(pred, 4)
            row["prediction_error"] = round(pred / wall - 1, 4)
        return row, res, wall

    if args.loop_sweep:
        table = []
        for p in (0.4, 0.6, 0.8):
            rows = [one(K, p, False)[0] for K in range(k_max + 1)] + [one(0, p, True)[0]]
            best_fixed = max(r["committed_tok_s"] for r in rows[:-1])
            rows[-1]["vs_best_fixed_k"] = round(rows[-1]["committed_tok_s"] / best_fixed, 4)
            table += rows
        line = {"metric": "committed tokens/s of the decode loop, fixed K against adaptive K",
                "value": max(r["committed_tok_s"] for r in table), "unit": "committed tokens/s"}
        line.update(_header(args, wl))
        line.update({"scaling": "strong", "data": "synthetic (seeded; Zipf router bias, drafts = argmax w.p. p)",
                     "config": {"workload": wl.name, "sequences": B0, "lengths": args.loop_lengths,
                                "tokens": total_tokens,
                                "draft_block_in_step": mtp is not None,
                                "step_cost_ms": {str(b): [round(c, 4) for c in v] for b, v in cost.items()}},
                     "sweep": table, "roofline": None, "cpu_baseline": None})
        return line

    K = args.k_draft if args.k_draft is not None else wl.k_draft
    p = args.match_p if args.match_p is not None else wl.match_p
    row, res, wall = one(K, p, args.adaptive_k)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O

        K0 = res.steps[0].K
        T0 = B0 * (K0 + 1)
        dr = bd.to_host(res.steps[0].drafts).reshape(B0, K0)
        rows0 = h_np.reshape(B0, k_max + 1, -1)[:, np.minimum(np.arange(K0 + 1), k_max)].reshape(T0, -1)
        t1 = time.perf_counter()
        r = O.verify_step(rows0, dr, W, dims)
        dt = time.perf_counter() - t1
        cpu = {"value": round(float(np.sum(r["n_committed"])) / dt, 3), "unit": "committed tokens/s",
               "cores": _cores(), "kind": "oracle",
               "sample": f"the loop's first verify step ({B0} sequences, K={K0}); float64 numpy oracle",
               "s_per_step": round(dt, 3)}
    line = {"metric": METRIC, "value": row["committed_tok_s"], "unit": "committed tokens/s"}
    line.update(_header(args, wl))
    line.update({
        "steps": len(res.steps), "warmup": 1, "ms_per_step": row["ms_per_step"],
        "scaling": "strong",
        "data": "synthetic (seeded; weights N(0,0.02), Zipf router bias, drafts = argmax w.p. p)",
        "config": {"workload": wl.name, "sequences": B0, "k_draft": "adaptive" if args.adaptive_k else K,
                   "match_p": p, "lengths": args.loop_lengths, "tokens": total_tokens,
                   "draft_block_in_step": mtp is not None,
                   "draft_block_note": ("the draft block's work runs and is timed in every step; the verify "
                                        "step takes synthetic drafts of acceptance p, so this times drafting, it "
                                        "does not measure a speculative speedup") if mtp is not None else None,
                   **{k: v for k, v in row.items() if k not in ("k", "p")}},
        "roofline": None,
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 4),
    })
    return line


def draft_bytes(dims, d_ff_mtp, B, K):
    """Algorithmic HBM bytes of one mtp_draft call: per draft position the
    block's matrices (projection [d, 2d], gate/up [2Fm, d], down [d, Fm]),
    the LM head, four norm vectors, and per sequence an embedding row and
    the hidden rows in and out."""
    es = 2 if dims.dtype == "bf16" else 4
    d = dims.d_model
    per_pos = (2 * d * d + 3 * d_ff_mtp * d + dims.vocab * d + 4 * d) * es
    return K * (per_pos + B * 3 * d * es)


def bench_draft(args, wl, W, bd, synth, torch):
    """The FastMTP draft block: one mtp_draft call drafts K tokens for each of
    B sequences (K applications of the block, each with an LM-head pass)."""
    dims = wl.dims
    B, K = wl.batch, (args.k_draft if args.k_draft is not None else wl.k_draft)
    model = bd.DeviceModel(dims, W, max_tokens=B * (K + 1))
    M = synth.make_mtp_weights(dims, seed=args.seed, sigma=wl.weight_sigma)
    mtp = bd.DeviceMtp(dims, M, max_rows=B)
    h_np = synth.make_hidden(dims, B, args.seed, wl.code)
    tok_np = (np.arange(B, dtype=np.int32) * 7919 + 11) % dims.vocab
    h, tok = bd.to_device(h_np), bd.to_device(tok_np.astype(np.int32))
    out = bd.run_mtp_draft(model, mtp, h, tok, K)

    def step(stream):
        bd.mtp_draft(model.cfg, model.weights, mtp.weights, B, K, h, tok, out["drafts"], out["h_out"],
                     mtp.ws, mtp.ws_bytes, stream)

    stream = torch.cuda.current_stream()
    ms, wall, t_enq = _timed(step, stream, args.steps, args.warmup, torch)
    nbytes = draft_bytes(dims, mtp.d_ff, B, K)
    achieved = nbytes / (ms * 1e-3) / 1e9
    meas = MEASURED_TRAFFIC.get(wl.name + "_draft") if K == wl.k_draft else None
    traffic = meas["bytes_per_step"] if meas and meas["csrc_sha256_16"] == csrc_digest() else None
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O

        t0 = time.perf_counter()
        O.mtp_draft(h_np, tok_np, M, W, dims, K)
        dt = time.perf_counter() - t0
        cpu = {"value": round(B * K / dt, 3), "unit": "draft tokens/s", "cores": _cores(), "kind": "oracle",
               "sample": f"one mtp_draft call ({B} sequences, K={K}; float64 numpy oracle)",
               "s_per_call": round(dt, 3)}
    copy_gbs = None if args.no_copy_ceiling else copy_ceiling(torch)
    line = {"metric": "draft tokens/s (FastMTP draft block) + % of HBM roofline",
            "value": round(B * K / (ms * 1e-3), 1), "unit": "draft tokens/s"}
    line.update(_header(args, wl))
    line.update({
        "ms_per_step": round(ms, 4),
        "data": "synthetic (seeded; draft-block weights N(0,0.02), hidden N(0,1))",
        "config": {"workload": wl.name + "_draft", "batch": B, "k_draft": K, "d_model": dims.d_model,
                   "d_ff_draft": mtp.d_ff, "vocab": dims.vocab},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "whole mtp_draft call (K x [row norms, projection, FFN, LM head])",
                     "algorithmic_bytes_per_step": int(nbytes), "copy_gbs": copy_gbs,
                     "frac_of_copy": round(achieved / copy_gbs, 4) if copy_gbs else None},
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 4),
    })
    return line


def bench_choose_k(args, wl, W, bd, synth, torch):
    """Draft length: the cost of one speculative step (mtp_draft for K
    positions, then moe_verify_step over B (K + 1) rows) timed for K = 0..3,
    and the K that mv_choose_k picks from those costs, and from the byte model
    mv_step_bytes, for a range of per-position acceptance rates."""
    dims = wl.dims
    B, k_max = wl.batch, 3
    model = bd.DeviceModel(dims, W, max_tokens=B * (k_max + 1))
    M = synth.make_mtp_weights(dims, seed=args.seed, sigma=wl.weight_sigma)
    mtp = bd.DeviceMtp(dims, M, max_rows=B)
    h_rows = bd.to_device(synth.make_hidden(dims, B * (k_max + 1), args.seed, wl.code))
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    cost = []
    for K in range(k_max + 1):
        T = B * (K + 1)
        d_out = torch.empty((B, max(K, 1)), dtype=torch.int32, device="cuda")
        out = bd.run_verify_step(model, h_rows[:T], d_out, B, K)
        first = torch.arange(B, device="cuda") * (K + 1)

        def step(stream, K=K, T=T, d_out=d_out, out=out, first=first):
            if K:
                bd.mtp_draft(model.cfg, model.weights, mtp.weights, B, K, h_rows.index_select(0, first), tok,
                             d_out, None, mtp.ws, mtp.ws_bytes, stream)
            bd.moe_verify_step(model.cfg, model.weights, B, K, h_rows[:T], d_out, out["h_out"], out["argmax"],
                               out["n_accepted"], out["committed"], out["n_committed"], None, model.ws,
                               model.ws_bytes, stream)

        ms, _, _ = _timed(step, torch.cuda.current_stream(), args.steps, args.warmup, torch)
        cost.append(ms)
    nbytes = [bd.mv_step_bytes(model.cfg, B, K, mtp.d_ff) for K in range(k_max + 1)]
    table = []
    for q in (0.3, 0.4, 0.5, 0.576, 0.6, 0.7, 0.7485, 0.8, 0.9):
        k_t, r_t = bd.mv_choose_k(q, cost)
        k_b, _ = bd.mv_choose_k(q, [b / 1e9 for b in nbytes])
        table.append({"q": q, "k_time": k_t, "tok_per_s": round(B * r_t * 1e3, 1), "k_bytes": k_b})
    q0 = wl.match_p + (1 - wl.match_p) / dims.vocab
    k0, r0 = bd.mv_choose_k(q0, cost)
    line = {"metric": "committed tokens/s at the draft length chosen from measured step costs",
            "value": round(B * r0 * 1e3, 1), "unit": "committed tokens/s (expected)"}
    line.update(_header(args, wl))
    line.update({
        "ms_per_step": round(cost[k0], 4),
        "data": "synthetic (seeded; weights N(0,0.02)); expected commits 1 + q + ... + q^K",
        "config": {"workload": wl.name + "_choose_k", "batch": B, "k_max": k_max, "q": round(q0, 4),
                   "chosen_k": k0, "step_ms": [round(c, 4) for c in cost],
                   "step_gb_model": [round(b / 1e9, 4) for b in nbytes], "policy": table},
        "roofline": None,
        "cpu_baseline": None,
    })
    return line


def _mean_commits(bd, torch, g, p, vocab, seed, n):
    """Mean committed tokens per sequence over n seeded draft draws (each
    position equal to the step's argmax g with probability p), through the
    library's accept rule (spec_accept) on the device."""
    from speculative_decode_verification_router_amd import synth

    B, K1 = g.shape
    K = K1 - 1
    if K == 0:
        return 1.0
    gg = np.tile(g, (n, 1))
    dr = np.concatenate([synth.make_drafts(g, p, vocab, seed=seed, step=1000 + i) for i in range(n)])
    nb = gg.shape[0]
    n_acc = torch.empty(nb, dtype=torch.int32, device="cuda")
    com = torch.empty((nb, K + 1), dtype=torch.int32, device="cuda")
    n_com = torch.empty(nb, dtype=torch.int32, device="cuda")
    bd.spec_accept(nb, K, bd.to_device(gg.astype(np.int32)), bd.to_device(dr), n_acc, com, n_com)
    return float(bd.to_host(n_com).mean())


def forced_parity(bd, torch, model, W, dims, h, B, K, pre, drafts_np, out):
    """The oracle's check of the timed step, teacher-forced: the layer
    chain (moe_layer_forward, which reproduces the step's routing bit for
    bit) runs on the GPU, and each layer of the oracle is fed the GPU's input
    to that layer.  Counts routing decisions whose oracle margin is below
    1e-3 (near-ties), GPU decisions that differ from the oracle's outside a
    near-tie (mismatches), the largest row error of the layer outputs, and
    whether the commits equal the oracle's accept rule on the oracle's argmax.
    Every layer and the LM head take the GPU's own input on both sides, so a
    token counts as checked unless one of its decisions differs from the
    oracle's (which the rule tolerates only at a near-tie)."""
    from oracle import moe_oracle as O

    T = B * (K + 1)
    excluded = np.zeros(T, bool)      # tokens with a decision that differs from the oracle's
    argmax_off = np.zeros(T, bool)
    near = mism = 0
    worst = 0.0
    cur = h
    ids_step = bd.to_host(pre["topk_ids"])
    chain_same = True
    for layer in range(dims.n_layers):
        lo = bd.run_layer_forward(model, layer, cur)
        torch.cuda.synchronize()
        gid = bd.to_host(lo["topk_ids"])
        chain_same &= bool(np.array_equal(gid, ids_step[layer]))
        ref = O.moe_layer(O.widen(bd.to_host(cur), dims.dtype), W, layer, dims)
        is_near = ref["margin"] < 1e-3
        differ = np.any(np.sort(gid, 1) != np.sort(ref["ids"], 1), axis=1)
        near += int(np.sum(is_near))
        mism += int(np.sum(differ & ~is_near))
        excluded |= differ
        hg = O.widen(bd.to_host(lo["h_out"]), dims.dtype)
        err = np.abs(hg - ref["h_out"]).max(1) / np.abs(ref["h_out"]).max(1)
        if (~differ).any():   # rows whose routing matched: the layer's outputs are comparable
            worst = max(worst, float(err[~differ].max()))
        cur = lo["h_out"]
    lm = O.lm_head_argmax(O.widen(bd.to_host(cur), dims.dtype), W["final_norm"], W["lm_head"], dims)
    g_gpu = bd.to_host(out["argmax"])
    is_near = lm["margin"] < 1e-3
    differ = g_gpu != lm["argmax"]
    near += int(np.sum(is_near))
    mism += int(np.sum(differ & ~is_near))
    excluded |= differ
    argmax_off |= differ
    _, r_com, r_ncom = O.spec_accept(np.asarray(lm["argmax"]).reshape(B, K + 1), drafts_np)
    ok_seq = ~argmax_off.reshape(B, K + 1).any(axis=1)
    com_ok = bool(np.array_equal(bd.to_host(out["committed"])[ok_seq], r_com[ok_seq]) and
                  np.array_equal(bd.to_host(out["n_committed"])[ok_seq], r_ncom[ok_seq]))
    return {"kind": "teacher-forced (each layer of the oracle on the GPU's input to it)",
            "near_ties": near, "mismatches": mism, "checked_tokens": int(T - excluded.sum()), "tokens": T,
            "max_row_rel_err": round(worst, 5), "commits_equal": com_ok,
            "sequences_checked": int(ok_seq.sum()), "chain_reproduces_step": chain_same}


def cpu_baseline(wl, W, h_np, drafts_np, steps):
    """The CPU oracle timed on a bounded sample of the same workload."""
    from oracle import moe_oracle as O

    cores = _cores()
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
