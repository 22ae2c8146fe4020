#!/usr/bin/env python3
"""Throughput of the DFlash KV-injection drafter round on one MI355X.

A step is one steady-state speculative round of the whole hot path on one
batch of synthetic input, inputs resident in HBM:
  1. context projection of the gamma+1 tapped rows the last verify produced,
  2. per-layer context K/V append of the committed rows (counts on device),
  3. drafter forward: block init, every layer, out projection, LM-head argmax,
  4. greedy verify of the drafts against planted target logits,
  5. roll the context back to its prefilled length (O(1) length write).
Each distinct round input set is captured once as a HIP graph (through
torch.cuda.CUDAGraph on the stream the library launches on) and the graphs
are replayed in a cycle. The metric is draft blocks per second (B blocks per
step); tokens proposed per second is gamma * B * blocks/s.

The dominant kernel (the LM-head GEMV + argmax epilogue) is timed live inside
the timed region: each of its workgroups writes the device wall clock at its
start and end into a per-round buffer (a kernel argument, so graph replays
write it too); its duration is the first start to the last end, averaged over
the last timed run of every round.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config default]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import CONFIGS, gen  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s (published)
METRIC = "draft blocks/sec (drafter fwd+verify) at 1 MI355X; % HBM/MFMA roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_bytes_per_elem(wdtype):
    return {"f32": 4.0, "bf16": 2.0, "int4g64": 0.5 + 4.0 / 64}[wdtype]


def algorithmic_bytes(d, B, ctx_rows, n_new):
    """Minimum bytes of one round: every weight once (the K/V rows shared by
    the append and the block counted once), the borrowed LM head once, one
    embedding row per sequence, every layer's context K/V once, the new tap
    rows and the target logits."""
    wb = weight_bytes_per_elem(d.wdtype)
    layer = ((d.hq + 2 * d.hkv) * d.hd * d.d + d.d * d.hq * d.hd + 2 * d.F * d.d + d.d * d.F) * wb
    drafter = d.nl * layer + (d.d * d.m * d.H + d.d * d.H + d.H * d.d) * wb
    head = d.V * d.H * wb
    kv_elem = 4 if d.wdtype == "f32" else 2
    kv = d.nl * 2 * d.hkv * d.hd * kv_elem * (ctx_rows + n_new * B)
    act = 4 if d.wdtype == "f32" else 2
    other = B * (d.gamma + 1) * (d.m * d.H * act + d.V * 4) + B * d.H * wb
    return {"weights": drafter, "lm_head": head, "kv": kv, "other": other,
            "total": drafter + head + kv + other}


def describe(d, lengths):
    ctx = f"context {lengths[0]}" if len(set(lengths)) == 1 else f"contexts {min(lengths)}-{max(lengths)}"
    return (f"{d.name} drafter {d.wdtype}: target hidden {d.H}, {d.m} taps, width {d.d}, {d.nl} layers, "
            f"{d.hq}q/{d.hkv}kv heads x hd{d.hd}, FFN {d.F} ({d.act}), gamma {d.gamma} "
            f"(block {d.gamma + 1}), {ctx}, vocab {d.V}, batch {d.B}")


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample of the same rounds


def cpu_baseline(d, rounds_inputs, seconds, gpu_ids):
    from threadpoolctl import threadpool_info
    from oracle import dflash_oracle as O

    faithful = d.wdtype != "f32"
    w = gen.Model(d).materialise()
    lengths = gen.context_lengths(d)
    ctx = O.Context(d.nl, d.B, d.hkv, d.hd)
    for b in range(d.B):
        taps = gen.make_taps(d, 0, int(lengths[b]), stream="ctx", seq=b)
        Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], d.eps)
        O.append_context(ctx, w, d, Hc, [[]] * b + [list(range(int(lengths[b])))] + [[]] * (d.B - b - 1),
                         [0] * b + [int(lengths[b])] + [0] * (d.B - b - 1), faithful)
    W = d.gamma + 1
    n_done, agree, compared = 0, 0, 0
    anchor = gen.make_anchors(d, 0)
    t0 = time.perf_counter()
    while True:
        r = n_done % len(rounds_inputs)
        counts = rounds_inputs[r]["counts"]
        for b in range(d.B):
            taps = gen.make_taps(d, r * W, W, stream="round", seq=b)
            Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], d.eps)
            O.append_context(ctx, w, d, Hc, [[]] * b + [list(range(W))] + [[]] * (d.B - b - 1),
                             [0] * b + [int(counts[b])] + [0] * (d.B - b - 1), faithful)
        ids, ex = O.draft_forward(w, d, ctx, anchor, faithful, return_all=True)
        T = gen.plant_target_logits(d, ids, rounds_inputs[r]["accept"], r)
        _, _, _, nxt = O.verify_greedy(T, ids)
        for b in range(d.B):
            ctx.truncate(b, int(lengths[b]))
        if n_done < len(rounds_inputs):
            # parity spot check of the GPU chain (same seeded inputs, same schedule)
            s = np.sort(ex["logits"].reshape(d.B * d.gamma, -1), axis=1)
            decided = (s[:, -1] - s[:, -2]) >= 1e-3
            g = gpu_ids[r].reshape(-1)
            compared += int(decided.sum())
            agree += int((decided & (g == ids.reshape(-1))).sum())
        anchor = nxt
        n_done += 1
        if time.perf_counter() - t0 >= seconds and n_done >= 2:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": round(n_done * d.B / dt, 4),
        "unit": "blocks/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n_done} full rounds (append + forward + verify) of the same workload, numpy float64 "
                  f"bf16-faithful oracle, {dt:.1f} s wall on the host; context prefill untimed",
        "parity_ids_agree": f"{agree}/{compared}",
    }


# ----------------------------------------------------------------------------


COPY_BYTES = 256 << 20    # calibration copy: reads and writes this many bytes


def profile_head(d, dev, launches=20):
    """Workload for memory-counter passes: one elementwise copy of COPY_BYTES
    (a kernel whose HBM reads and writes are known, to scale the counters),
    then eager launches of the LM-head argmax alone at the workload's shape."""
    import torch
    from block_diffusion_draft_tap_amd import binding as bd
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    rows = d.B * d.gamma
    E = bd.Weight(gen.make_weight(d, "E_out"), dev)
    y16 = gen.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((rows, d.H)).astype(np.float32))
    y = torch.from_numpy(y16.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.empty(rows, dtype=torch.int32, device=dev)
    ws = bd.lm_head_workspace(d.V, rows, dev)
    for _ in range(launches):
        bd.check(bd.dflash_lm_head_argmax(E, y, ids, ws), "lm_head_argmax")
    torch.cuda.synchronize()
    log(f"[profile-head] copy {COPY_BYTES} B, {launches} LM-head launches ({d.V} x {d.H}, {rows} rows)")


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)


def bench_prefill(d, dev, args):
    """Context prefill of every sequence of the workload in one pass: the
    context projection (Eq 2) of all sum(L) rows, then every layer's context
    K/V. bf16 models run both as matrix-core GEMMs. Weights and taps are drawn
    on the device (N(0, 0.02) and N(0, 1) in bf16): the values do not change
    the work, and drawing ~10 GB of taps on the host would dominate the run."""
    import torch
    import block_diffusion_draft_tap_amd as dfa
    from block_diffusion_draft_tap_amd import binding as bd
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rnd(shape, std):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(torch.bfloat16)

    log(f"[prefill] drawing {d.name} weights on the device")
    w = {}
    for name in gen.weight_names(d):
        shape = gen.weight_shape(d, name)
        w[name] = torch.ones(shape, dtype=torch.bfloat16, device=dev) if gen.is_gain(name) else rnd(shape, 0.02)
    dm = dfa.DeviceModel(d, w, dev)
    del w
    lengths = [int(x) for x in gen.context_lengths(d)]
    n = sum(lengths)
    kv = dfa.KVCache(d, d.B, max(lengths) + 64, dev)
    ws = dfa.workspace(d, d.B, kv.cap, dev)
    taps = [rnd((n, d.H), 1.0) for _ in range(d.m)]
    h = torch.empty(n, d.d, dtype=torch.float32, device=dev)
    offs = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32, device=dev)
    # room for every layer's bf16 normalised rows: the K/V GEMM reads plain bf16 tiles
    kws = dfa.kv_prefill_workspace(d, n) if d.wdtype == "bf16" else ws
    flops_proj = 2.0 * n * d.m * d.H * d.d
    flops_kv = 2.0 * n * d.d * 2 * d.hkv * d.hd * d.nl
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    reps = max(1, args.steps)
    proj_ms, kv_ms = [], []
    for r in range(reps + 1):
        kv.len.zero_()
        torch.cuda.synchronize()
        ev[0].record()
        bd.check(dfa.dflash_context_project(dm, taps, h, ws), "context_project")
        ev[1].record()
        bd.check(dfa.dflash_ctx_kv_append(dm, h, offs, None, kv, kws), "append")
        ev[2].record()
        torch.cuda.synchronize()
        if r > 0:  # the first pass is the warm-up
            proj_ms.append(ev[0].elapsed_time(ev[1]))
            kv_ms.append(ev[1].elapsed_time(ev[2]))
    assert kv.len.cpu().tolist() == lengths
    pm, km = float(np.median(proj_ms)), float(np.median(kv_ms))
    tot_tf = (flops_proj + flops_kv) / ((pm + km) / 1e3) / 1e12
    res = {
        "metric": "context prefill (projection + per-layer K/V) TFLOP/s at 1 MI355X; % MFMA bf16 roofline",
        "value": round(tot_tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": reps,
        "higher_is_better": True,
        "dtype": "bf16" if d.wdtype == "bf16" else d.wdtype,
        "data": "synthetic (weights and taps drawn on the device)",
        "config": {"workload": describe(d, lengths), "rows": n,
                   "kv_workspace_bytes": int(kws.numel())},
        "projection": {"ms": round(pm, 3), "tflops": round(flops_proj / (pm / 1e3) / 1e12, 2),
                       "flops": flops_proj},
        "kv": {"ms": round(km, 3), "tflops": round(flops_kv / (km / 1e3) / 1e12, 2), "flops": flops_kv},
        "roofline": {"bound": "mfma", "achieved": round(tot_tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tot_tf / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="default", choices=sorted(CONFIGS))
    ap.add_argument("--rounds", type=int, default=8, help="distinct round inputs, replayed in a cycle")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every call from the host (no graphs)")
    ap.add_argument("--profile-head", action="store_true",
                    help="counter workload: a 256 MiB device copy (calibration), then eager LM-head launches")
    ap.add_argument("--device-taps", action="store_true",
                    help="draw the prefilled context's taps on the device (large batched contexts)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the context prefill (projection + K/V of every context row) instead of the round")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_draft_tap_amd as dfa
    from block_diffusion_draft_tap_amd import binding as bd

    d = CONFIGS[args.config]
    B, W, R = d.B, d.gamma + 1, args.rounds
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if bd.dflash_query(d) != bd.DFLASH_OK:
        print("libdflash declined this configuration on this device", file=sys.stderr)
        sys.exit(3)
    if args.profile_head:
        profile_head(d, dev)
        return
    if args.prefill:
        bench_prefill(d, dev, args)
        return
    if args.device_taps and not args.skip_cpu:
        print("--device-taps changes the prefilled context: use it with --skip-cpu", file=sys.stderr)
        sys.exit(2)

    t_setup = time.perf_counter()
    log(f"[bench] generating weights for {d.name}")
    w = gen.Model(d).materialise()
    dm = dfa.DeviceModel(d, w, dev)
    del w
    lengths = [int(x) for x in gen.context_lengths(d)]
    cap = max(lengths) + W + 64
    kv = dfa.KVCache(d, B, cap, dev)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    ws = dfa.workspace(d, B, kv.cap, dev)

    # prefill the retained context (untimed)
    log("[bench] prefilling the context")
    for b in range(B):
        L = lengths[b]
        if args.device_taps:
            gt = torch.Generator(device=dev)
            gt.manual_seed(1000 + b)
            taps = [torch.randn(L, d.H, generator=gt, device=dev).to(torch.bfloat16 if d.wdtype != "f32" else
                                                                      torch.float32) for _ in range(d.m)]
        else:
            taps = [up(t) for t in gen.make_taps(d, 0, L, stream="ctx", seq=b)]
        h = torch.empty(L, d.d, dtype=torch.float32, device=dev)
        bd.check(dfa.dflash_context_project(dm, taps, h, ws), "context_project")
        offs = torch.zeros(B + 1, dtype=torch.int32, device=dev)
        offs[b + 1:] = L
        bd.check(dfa.dflash_ctx_kv_append(dm, h, offs, None, kv, ws), "append")
        del taps, h
    torch.cuda.synchronize()
    len0 = kv.len.clone()
    assert kv.len.cpu().tolist() == lengths

    vws = bd.verify_workspace(B, d.gamma, d.V, dev)
    offs = torch.arange(0, (B + 1) * W, W, dtype=torch.int32, device=dev)
    h_new = torch.empty(B * W, d.d, dtype=torch.float32, device=dev)

    # per-round inputs, resident on the device
    accept = [gen.accept_schedule(d, r) for r in range(R)]
    head_wgs, head_launches = bd.dflash_lm_head_workgroups(d.V, d.H, d.wdtype, B * d.gamma)
    rounds = []
    for r in range(R):
        taps_r = [gen.make_taps(d, r * W, W, stream="round", seq=b) for b in range(B)]
        rr = {
            "taps": [up(np.concatenate([taps_r[b][j] for b in range(B)])) for j in range(d.m)],
            "counts_h": (accept[(r - 1) % R] + 1).astype(np.int32),
            "accept": accept[r],
            "anchors": torch.zeros(B, dtype=torch.int32, device=dev),
            "ids": torch.zeros(B, d.gamma, dtype=torch.int32, device=dev),
            "T": torch.zeros(B, W, d.V, dtype=torch.float32, device=dev),
            "acc": torch.zeros(B, dtype=torch.int32, device=dev),
            "com": torch.zeros(B, dtype=torch.int32, device=dev),
            "vids": torch.zeros(B, W, dtype=torch.int32, device=dev),
            "nxt": torch.zeros(B, dtype=torch.int32, device=dev),
            # LM-head workgroup wall-clock stamps of this round's latest run
            "stamps": torch.zeros(2 * head_wgs * head_launches, dtype=torch.int64, device=dev),
        }
        rr["counts"] = torch.from_numpy(rr["counts_h"]).to(dev)
        rounds.append(rr)

    def run_round(rr, verify=True):
        # the head kernel writes its workgroup stamps into this round's buffer (a kernel
        # argument: captured graphs keep writing them on every replay)
        bd.dflash_trace_head_stamps(rr["stamps"])
        bd.check(dfa.dflash_context_project(dm, rr["taps"], h_new, ws), "context_project")
        bd.check(dfa.dflash_ctx_kv_append(dm, h_new, offs, rr["counts"], kv, ws), "append")
        bd.check(dfa.dflash_draft_forward(dm, rr["anchors"], kv, B, rr["ids"], ws), "forward")
        if verify:
            bd.check(dfa.dflash_verify_greedy(rr["T"], rr["ids"], rr["acc"], rr["com"], rr["vids"], vws,
                                              next_anchor=rr["nxt"]), "verify")
        kv.len.copy_(len0)
        bd.dflash_trace_head_stamps(None)

    # untimed chain: drafts of each round plant that round's target logits
    log("[bench] building the round chain")
    anchor = gen.make_anchors(d, 0)
    chain_ids = []
    for r, rr in enumerate(rounds):
        rr["anchors"].copy_(torch.from_numpy(anchor))
        run_round(rr, verify=False)
        ids = rr["ids"].cpu().numpy().copy()
        chain_ids.append(ids)
        rr["T"].copy_(torch.from_numpy(gen.plant_target_logits(d, ids, accept[r], r)))
        bd.check(dfa.dflash_verify_greedy(rr["T"], rr["ids"], rr["acc"], rr["com"], rr["vids"], vws,
                                          next_anchor=rr["nxt"]), "verify")
        assert np.array_equal(rr["acc"].cpu().numpy(), accept[r])
        anchor = rr["nxt"].cpu().numpy().copy()
    torch.cuda.synchronize()

    # capture one graph per round
    graphs = []
    stream = torch.cuda.Stream(device=dev)
    use_graph = not args.eager
    if use_graph:
        log("[bench] capturing graphs")
        torch.cuda.synchronize()
        for rr in rounds:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                run_round(rr)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(i):
        if use_graph:
            graphs[i % R].replay()
        else:
            run_round(rounds[i % R])

    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; warmup {args.warmup}, timed {args.steps}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)

    # the replays must reproduce the chain exactly (deterministic kernels)
    for r, rr in enumerate(rounds):
        assert np.array_equal(rr["ids"].cpu().numpy(), chain_ids[r]), f"round {r}: drafts changed on replay"
        assert np.array_equal(rr["acc"].cpu().numpy(), accept[r]), f"round {r}: accepted changed on replay"
        assert np.array_equal(rr["com"].cpu().numpy(), accept[r] + 1)

    # the dominant kernel's duration, from the wall-clock stamps its workgroups wrote
    # during the timed region (the last run of each round)
    head_source = (f"device wall-clock stamps written by the kernel's workgroups (first start to last end), "
                   f"last timed run of each of the {R} rounds")
    head_us = [t * 1e6 for rr in rounds for t in bd.stamps_duration_s(rr["stamps"], head_launches)]
    assert all(0 < x < 1e5 for x in head_us), head_us
    head_us_avg = float(np.mean(head_us))
    ms_per_step = gpu_ms / args.steps
    blocks_per_s = B * args.steps / (gpu_ms / 1000.0)
    mean_new = float(np.mean([rr["counts_h"].sum() for rr in rounds]))
    ab = algorithmic_bytes(d, B, sum(lengths), mean_new / B)
    round_gbs = ab["total"] / (ms_per_step / 1000.0) / 1e9
    head_gbs = ab["lm_head"] / (head_us_avg / 1e6) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"lm_head_gemv_{d.name}_traffic.md")
    if os.path.exists(tfile):
        # counter-derived bytes per launch, valid only for the kernel sources they were taken with
        from block_diffusion_draft_tap_amd import prof_report
        vals = prof_report.read_summary(tfile)
        if vals.get("kernel sources sha256[:16]") == prof_report.kernel_sources_hash() and "bytes per launch" in vals:
            traffic = float(vals["bytes per launch"])

    res = {
        "metric": METRIC,
        "value": round(blocks_per_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": d.wdtype,
        "data": "synthetic",
        "config": {
            "workload": describe(d, lengths),
            "rounds_cycled": R,
            "mean_committed_rows_appended": round(mean_new / B, 3),
            "launch": "hip graph per round" if use_graph else "eager",
        },
        "tokens_proposed_per_s": round(blocks_per_s * d.gamma, 1),
        "round_algorithmic_bytes": int(ab["total"]),
        "round_hbm_frac": round(round_gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "LM head with argmax epilogue",
            "launches_x_workgroups": f"{head_launches} x {head_wgs}",
            "achieved": round(head_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(ab["lm_head"]),
            "avg_launch_us": round(head_us_avg, 3),
            "timing": head_source,
        },
        "wall_s_timed": round(wall, 4),
    }
    if not args.skip_cpu:
        log(f"[bench] cpu baseline (~{args.cpu_seconds:.0f}s of oracle rounds)")
        rounds_inputs = [{"counts": rr["counts_h"], "accept": rr["accept"]} for rr in rounds]
        res["cpu_baseline"] = cpu_baseline(d, rounds_inputs, args.cpu_seconds, chain_ids)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
