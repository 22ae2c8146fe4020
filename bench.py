#!/usr/bin/env python3
"""Throughput of the DFlash KV-injection drafter round on one MI355X.

A step is one steady-state speculative round of the whole hot path on one
batch of synthetic input, inputs resident in HBM:
  1. context projection of the gamma+1 tapped rows per sequence the last
     verify produced,
  2. per-layer context K/V append of the committed rows (counts on device),
  3. drafter forward: block init, every layer, out projection, LM-head argmax,
  4. greedy verify of the drafts against planted target logits,
  5. roll the context back to its prefilled length (O(1) length write).
Each distinct round input set is captured once as a HIP graph (through
torch.cuda.CUDAGraph on the stream the library launches on) and the graphs
are replayed in a cycle. The metric is draft blocks per second (B blocks per
step); tokens proposed per second is gamma * B * blocks/s.

The default workload is the largest single-GPU one: 16 sequences of the wide
bf16 drafter with contexts of 9050-16059 rows (the batched workload).

Before the rounds, the whole context of every sequence is prefilled in one
call per step (projection, then every layer's K/V) and timed: the matrix-core
figure of the prefill. Taps of the prefilled context are drawn on the device
(the values do not change the work), except for the one sequence the CPU
oracle replays, whose taps are the seeded ones; every round input is seeded.

Kernel durations come from the kernels themselves: while the rounds are
captured, the library's launch tracing is on, so during every replay each
traced workgroup writes the device wall clock at its start and end into the
round's stamp buffer. A kernel's duration is its first start to last end; the
line reports the last timed replay of every round.

The CPU baseline is the oracle (numpy float64) replaying the round of one
sequence, interleaved with further timed GPU segments in the same minute.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config batched]
"""

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import CONFIGS, gen, scaled  # noqa: E402

HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, GB/s (published)
MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak (published)
METRIC = "draft blocks/sec (drafter fwd+verify) at 1 MI355X; % HBM/MFMA roofline"
NEAR_TIE = 1e-3                   # draft ids are compared where the oracle's top-2 gap is at least this
FLUSH_BYTES = 1 << 30             # MALL flush between rounds: a 1 GiB read (the MALL holds 256 MB)
STAMP_ENTRIES = 1 << 20           # per round: room for every traced workgroup's (start, end)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_bytes_per_elem(wdtype):
    return {"f32": 4.0, "bf16": 2.0, "int4g64": 0.5 + 4.0 / 64}[wdtype]


def dspark_bytes(d, B, r):
    """Extra minimum bytes of a round with the DSpark heads: the base logits of
    every block row written once and read once, markov.w2 streamed once per
    step, one w1 row and the confidence weights per step and sequence."""
    wb = 4.0 if d.wdtype == "f32" else 2.0
    return 2 * B * d.gamma * d.V * 4 + d.gamma * d.V * r * wb + d.gamma * B * r * wb + (d.d + r) * wb


def algorithmic_bytes(d, B, ctx_rows, n_new):
    """Minimum bytes of one round: every weight once (the K/V rows shared by
    the append and the block counted once), the borrowed LM head once, one
    embedding row per sequence, every layer's attended context K/V once
    (ctx_rows: the rows the attention reads), the new tap rows and the target
    logits; a verify from the target's hidden states reads those rows instead
    of logits and streams the head a second time."""
    wb = weight_bytes_per_elem(d.wdtype)
    layer = ((d.hq + 2 * d.hkv) * d.hd * d.d + d.d * d.hq * d.hd + 2 * d.F * d.d + d.d * d.F) * wb
    drafter = d.nl * layer + (d.d * d.m * d.H + d.d * d.H + d.H * d.d) * wb
    head = d.V * d.H * wb
    kv_elem = 4 if d.wdtype == "f32" else 2
    kv = d.nl * 2 * d.hkv * d.hd * kv_elem * (ctx_rows + n_new * B)
    act = 4 if d.wdtype == "f32" else 2
    if d.verify == "hidden":
        head *= 2
        other = B * (d.gamma + 1) * (d.m * d.H * act + d.H * act) + B * d.H * wb
    else:
        other = B * (d.gamma + 1) * (d.m * d.H * act + d.V * 4) + B * d.H * wb
    return {"weights": drafter, "lm_head": head, "kv": kv, "other": other,
            "total": drafter + head + kv + other}


def attended_rows(d, lengths):
    """Context rows the attention reads: each sequence's, or its window's."""
    return sum(min(int(L), d.window) if d.window else int(L) for L in lengths)


def head_rows(E, tokens):
    """Rows of the stored head (the generator's formats) as float64, to plant
    target hidden states along them."""
    tokens = np.asarray(tokens, dtype=np.int64)
    if isinstance(E, dict):                    # int4-g64: w = scale * q + bias per group of 64
        codes = E["codes"][tokens]
        q = (codes[..., None] >> (np.uint32(4) * np.arange(8, dtype=np.uint32))) & np.uint32(15)
        q = q.reshape(len(tokens), -1).astype(np.float64)
        sc = np.repeat(gen.bf16_bits_to_f32(E["scales"][tokens]).astype(np.float64), 64, axis=1)
        bi = np.repeat(gen.bf16_bits_to_f32(E["biases"][tokens]).astype(np.float64), 64, axis=1)
        return sc * q + bi
    if E.dtype == np.uint16:
        return gen.bf16_bits_to_f32(E[tokens]).astype(np.float64)
    return E[tokens].astype(np.float64)


def plant_hidden(d, w, drafts, accept, r):
    """Target hidden rows [B, gamma+1, H] whose greedy tokens under the head
    realise the accept plan: each along its planted token's head row (that
    token's logit exceeds every other by far for random head rows)."""
    t = gen.plant_target_tokens(d, drafts, accept, r)
    rows = head_rows(w["E_out"], t.reshape(-1))
    h = 4.0 * rows / np.linalg.norm(rows, axis=1, keepdims=True)
    return h.reshape(t.shape + (d.H,)).astype(np.float32)


def describe(d, lengths):
    ctx = f"context {lengths[0]}" if len(set(lengths)) == 1 else f"contexts {min(lengths)}-{max(lengths)}"
    return (f"{d.name} drafter {d.wdtype}: target hidden {d.H}, {d.m} taps, width {d.d}, {d.nl} layers, "
            f"{d.hq}q/{d.hkv}kv heads x hd{d.hd}, FFN {d.F} ({d.act}), gamma {d.gamma} "
            f"(block {d.gamma + 1}), {ctx}, vocab {d.V}, batch {d.B}")


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model,
            "load_average": [round(x, 2) for x in os.getloadavg()]}


def tag(kernel):
    return re.sub(r"[^a-z0-9]+", "_", kernel.lower()).strip("_")


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on one sequence of the same rounds


class CpuLeg:
    """The oracle replaying the round of sequence `b` (seeded taps, the same
    round inputs and accept schedule as the GPU chain). Setup (the oracle's own
    prefill of that sequence's context) is untimed; each timed oracle round is
    context projection + K/V append of the committed rows, the forward, the LM
    head and verify, then the rollback."""

    def __init__(self, d, w, b, L, rounds, thresholds=None):
        from oracle import dflash_oracle as O
        self.O, self.d, self.w, self.b, self.L, self.rounds = O, d, w, b, L, rounds
        self.thresholds = thresholds     # the DSpark round (Markov and confidence heads, Alg 1)
        self.fm = d.wdtype != "f32"
        self.d1 = scaled(d, B=1)
        taps = gen.make_taps(d, 0, L, stream="ctx", seq=b)
        Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], d.eps)
        self.ctx = O.Context(d.nl, 1, d.hkv, d.hd)
        O.append_context(self.ctx, w, d, Hc, [list(range(L))], [L], self.fm)
        self.done = 0
        self.seconds = 0.0
        self.checked = []
        self.anchor = None

    def run(self, seconds):
        O, d, w, b = self.O, self.d, self.w, self.b
        W = d.gamma + 1
        t0 = time.perf_counter()
        while True:
            r = self.done % len(self.rounds)
            rr = self.rounds[r]
            taps = gen.make_taps(d, r * W, W, stream="round", seq=b)
            Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], d.eps)
            O.append_context(self.ctx, w, d, Hc, [list(range(W))], [int(rr["counts_h"][b])], self.fm)
            if r == 0:  # the chain starts from the seeded anchors, like the GPU's
                self.anchor = gen.make_anchors(d, 0)[b:b + 1]
            anchor = self.anchor
            if self.thresholds is None:
                ids, ex = O.draft_forward(w, self.d1, self.ctx, anchor, self.fm, return_all=True)
                lengths = None
            else:
                ids, _, lengths, extra = O.dspark_forward(w, self.d1, self.ctx, anchor, self.fm,
                                                          thresholds=self.thresholds)
                ex = {"logits": extra["scores"].reshape(d.gamma, -1)}
            full = np.zeros((d.B, d.gamma), np.int32)
            full[b] = ids[0]
            if d.verify == "hidden":
                hid = plant_hidden(d, w, full, rr["accept"], r)[b:b + 1].astype(np.float64)
                hid = hid if d.wdtype == "f32" else O.bf16(hid)
                _, _, _, nxt = O.verify_from_hidden(hid, w["E_out"], ids, lengths=lengths)
            else:
                T = gen.plant_target_logits(d, full, rr["accept"], r)
                _, _, _, nxt = O.verify_greedy(T[b:b + 1], ids, lengths=lengths)
            self.anchor = nxt
            self.ctx.truncate(0, self.L)
            if self.done < len(self.rounds):
                self.checked.append((r, int(anchor[0]), ids[0].copy(), ex["logits"]))
            self.done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        self.seconds += time.perf_counter() - t0

    def parity(self, gpu_anchors, gpu_ids, gpu_y):
        """The GPU chain's drafts of this sequence against the oracle's at the
        stated 1e-3 band, in the rounds where both chains drafted from the same
        anchor. A miss counts as explained when the oracle's head, evaluated on
        the GPU's own Y, picks the GPU's token."""
        O, b = self.O, self.b
        agree = compared = 0
        misses = []
        for r, anchor, ids, logits in self.checked:
            if anchor != int(gpu_anchors[r][b]):
                misses.append({"round": r, "anchor_differs": True})
                continue
            s = np.sort(logits, axis=1)
            decided = (s[:, -1] - s[:, -2]) >= NEAR_TIE
            g = gpu_ids[r][b]
            if self.thresholds is not None:
                # the Markov head conditions each step on the previous token: compare up to and
                # including the first step where the two chains differ
                diff = np.nonzero(g != ids)[0]
                if diff.size:
                    decided = decided & (np.arange(len(g)) <= diff[0])
            compared += int(decided.sum())
            agree += int((decided & (g == ids)).sum())
            for k in np.nonzero(decided & (g != ids))[0]:
                if self.thresholds is not None:
                    misses.append({"round": r, "pos": int(k), "gpu": int(g[k]), "oracle": int(ids[k]),
                                   "oracle_top2_gap": round(float(s[k, -1] - s[k, -2]), 6)})
                    continue
                y = gpu_y[r][b, k:k + 1].astype(np.float64)
                own, best, lg = O.lm_head_argmax(y, self.w["E_out"], want_logits=True)
                explained = int(own[0]) == int(g[k]) or best[0] - lg[0, g[k]] <= NEAR_TIE
                misses.append({"round": r, "pos": int(k), "gpu": int(g[k]), "oracle": int(ids[k]),
                               "oracle_top2_gap": round(float(s[k, -1] - s[k, -2]), 6),
                               "explained_by_gpu_Y": bool(explained)})
        return agree, compared, misses


# ----------------------------------------------------------------------------
# counter workload


COPY_BYTES = 256 << 20    # calibration copy: reads and writes this many bytes


def calibration_copy(dev):
    """One elementwise copy whose HBM reads and writes are known (COPY_BYTES
    each), to scale the memory counters of the kernels that follow."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


# ----------------------------------------------------------------------------


def prefill(d, dm, kv, ws, lengths, cpu_seq, dev, reps, up):
    """The whole context of every sequence in one projection call and one K/V
    call, `reps` + 1 times (the first untimed); returns the timing summary."""
    import torch
    import block_diffusion_draft_tap_amd as dfa
    from block_diffusion_draft_tap_amd import binding as bd
    n = sum(lengths)
    offs_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    act = torch.float32 if d.wdtype == "f32" else torch.bfloat16
    taps = [torch.empty(n, d.H, dtype=act, device=dev) for _ in range(d.m)]
    g = torch.Generator(device=dev)
    g.manual_seed(1000)
    for b in range(d.B):
        s0, s1 = int(offs_h[b]), int(offs_h[b + 1])
        if b == cpu_seq or n * d.m * d.H <= (64 << 20):
            for j, t in enumerate(gen.make_taps(d, 0, lengths[b], stream="ctx", seq=b)):
                taps[j][s0:s1] = up(t)
        else:
            for j in range(d.m):
                taps[j][s0:s1] = torch.randn(s1 - s0, d.H, generator=g, device=dev).to(act)
    h = torch.empty(n, d.d, dtype=torch.float32, device=dev)
    offs = torch.from_numpy(offs_h.astype(np.int32)).to(dev)
    # bf16: room to stage every layer's normalised rows; int4: room to expand the weights into
    # bf16 high and low parts for the matrix-core GEMMs (both calls)
    kws = ws
    if d.wdtype == "bf16" and n >= 64:
        kws = dfa.kv_prefill_workspace(d, n, dev)
    elif d.wdtype == "int4g64" and n >= 64:
        kws = dfa.int4_prefill_workspace(d, n, dev)
    pws = kws if d.wdtype == "int4g64" else ws
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    proj_ms, kv_ms = [], []
    for r in range(reps + 1):
        kv.len.zero_()
        torch.cuda.synchronize()
        ev[0].record()
        bd.check(dfa.dflash_context_project(dm, taps, h, pws), "context_project (prefill)")
        ev[1].record()
        bd.check(dfa.dflash_ctx_kv_append(dm, h, offs, None, kv, kws), "append (prefill)")
        ev[2].record()
        torch.cuda.synchronize()
        if r > 0:
            proj_ms.append(ev[0].elapsed_time(ev[1]))
            kv_ms.append(ev[1].elapsed_time(ev[2]))
    assert kv.len.cpu().tolist() == lengths
    del taps, h, kws, pws
    torch.cuda.empty_cache()
    if reps == 0:
        return None
    pm, km = float(np.median(proj_ms)), float(np.median(kv_ms))
    flops_proj = 2.0 * n * d.m * d.H * d.d
    flops_kv = 2.0 * n * d.d * 2 * d.hkv * d.hd * d.nl
    tot = (flops_proj + flops_kv) / ((pm + km) / 1e3) / 1e12
    return {"rows": n, "reps": reps,
            "projection": {"ms": round(pm, 3), "tflops": round(flops_proj / (pm / 1e3) / 1e12, 2)},
            "kv": {"ms": round(km, 3), "tflops": round(flops_kv / (km / 1e3) / 1e12, 2)},
            "tflops": round(tot, 2), "mfma_frac": round(tot / MFMA_BF16_PEAK_TFLOPS, 4),
            "peak_tflops": MFMA_BF16_PEAK_TFLOPS}


def kernel_table(rounds, lengths_after):
    """Per kernel: launches and time per round, algorithmic bytes, achieved
    GB/s, from the stamps of every round's last replay."""
    from block_diffusion_draft_tap_amd import binding as bd
    acc = {}
    for r, rr in enumerate(rounds):
        durs = bd.traced_durations_s(rr["stamps"], rr["records"])
        for rec, t in zip(rr["records"], durs):
            a = acc.setdefault(rec["kernel"], {"kind": rec["kind"], "launches": 0, "s": 0.0, "bytes": 0.0})
            a["launches"] += 1
            a["s"] += t
            a["bytes"] += rec["bytes"] + rec["ctx_row_bytes"] * lengths_after[r]
    R = len(rounds)
    table = []
    for k, a in acc.items():
        assert a["s"] > 0, k
        table.append({"kernel": k, "kind": {1: "lm_head", 2: "attention", 4: "projection"}[a["kind"]],
                      "launches_per_round": a["launches"] / R, "us_per_round": a["s"] / R * 1e6,
                      "avg_launch_us": a["s"] / a["launches"] * 1e6,
                      "algorithmic_bytes_per_launch": a["bytes"] / a["launches"],
                      "achieved_gbs": a["bytes"] / a["s"] / 1e9})
    table.sort(key=lambda x: -x["us_per_round"])
    return table


def roofline_entry(k, d, timing):
    entry = {
        "bound": "hbm",
        "kernel": k["kernel"],
        "launches_per_round": round(k["launches_per_round"], 2),
        "achieved": round(k["achieved_gbs"], 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(k["achieved_gbs"] / HBM_PEAK_GBS, 4),
        "traffic": None,
        "algorithmic_bytes_per_launch": int(k["algorithmic_bytes_per_launch"]),
        "avg_launch_us": round(k["avg_launch_us"], 3),
        "us_per_round": round(k["us_per_round"], 2),
        "timing": timing,
    }
    tfile = os.path.join(ROOT, "profiles", f"{tag(k['kernel'])}_{d.name}_traffic.md")
    if os.path.exists(tfile):
        # counter-derived bytes per launch, valid only for the kernel sources they were taken with
        from block_diffusion_draft_tap_amd import prof_report
        vals = prof_report.read_summary(tfile)
        if (vals.get("kernel sources sha256[:16]") == prof_report.kernel_sources_hash(vals.get("kernel", k["kernel"]))
                and "bytes per launch" in vals):
            entry["traffic"] = float(vals["bytes per launch"])
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="batched", choices=sorted(CONFIGS))
    ap.add_argument("--rounds", type=int, default=8, help="distinct round inputs, replayed in a cycle")
    ap.add_argument("--cpu-seconds", type=float, default=24.0, help="oracle time, split over the CPU segments")
    ap.add_argument("--cpu-segments", type=int, default=2, help="CPU segments interleaved with GPU segments")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--prefill-reps", type=int, default=2, help="timed whole-context prefills")
    ap.add_argument("--flush-steps", type=int, default=40, help="rounds timed one by one after a MALL flush")
    ap.add_argument("--eager", action="store_true", help="launch every call from the host (no graphs)")
    ap.add_argument("--no-trace", action="store_true", help="rounds without the in-kernel stamps")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="counter workload: a 256 MiB device copy (calibration), then eager rounds")
    ap.add_argument("--dspark", action="store_true",
                    help="the round with the DSpark heads (Markov sequential head of rank --rank, confidence "
                         "head, Alg 1 pruning at --threshold) and the length-capped verify")
    ap.add_argument("--rank", type=int, default=256, help="DSpark Markov rank (page 3's default config: 256)")
    ap.add_argument("--threshold", type=float, default=0.5, help="DSpark per-step pruning threshold (synthetic)")
    ap.add_argument("--one-call", action="store_true",
                    help="the round's projection, append and forward as one dflash_draft_round call")
    args = ap.parse_args()

    if args.one_call and args.dspark:
        sys.exit("bench.py: --one-call runs the plain drafter's round; it does not combine with --dspark")
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

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t_setup = time.perf_counter()
    log(f"[bench] generating weights for {d.name}")
    if args.dspark:
        d = scaled(d, r=args.rank)
    w = gen.Model(d).materialise()
    dm = dfa.DeviceModel(d, w, dev)
    head = dfa.DsparkHead(w, dev) if args.dspark else None
    thresholds = np.full(d.gamma, args.threshold, np.float32) if args.dspark else None
    lengths = [int(x) for x in gen.context_lengths(d)]
    cpu_seq = int(np.argmin(lengths))
    cap = max(lengths) + W + 64
    kv = dfa.KVCache(d, B, cap, dev)
    ws = dfa.workspace(d, B, kv.cap, dev)

    log(f"[bench] prefilling {sum(lengths)} context rows ({B} sequences)")
    pre = prefill(d, dm, kv, ws, lengths, cpu_seq, dev, 0 if args.profile_kernels else args.prefill_reps, up)
    len0 = kv.len.clone()

    vws = bd.verify_workspace(B, d.gamma, d.V, dev)
    hws = dfa.verify_hidden_workspace(d, B, dev) if d.verify == "hidden" else None
    rws = dfa.round_workspace(d, B, kv.cap, dev) if args.one_call else None
    if args.dspark:
        dws = dfa.dspark_workspace(d, d.r, B, kv.cap, dev)
        thr_d = torch.from_numpy(thresholds).to(dev)
    offs = torch.arange(0, (B + 1) * W, W, dtype=torch.int32, device=dev)
    h_new = torch.empty(B * W, d.d, dtype=torch.float32, device=dev)
    y_chain = torch.empty(B, d.gamma, d.H, dtype=dm.act_dtype, device=dev)

    # per-round inputs, resident on the device
    accept = [gen.accept_schedule(d, r) for r in range(R)]
    rounds = []
    for r in range(R):
        taps_r = [gen.make_taps(d, r * W, W, stream="round", seq=b) for b in range(B)]
        rr = {
            "taps": [up(np.concatenate([taps_r[b][j] for b in range(B)])) for j in range(d.m)],
            "counts_h": (accept[(r - 1) % R] + 1).astype(np.int32),
            "accept": accept[r],
            "anchors": torch.zeros(B, dtype=torch.int32, device=dev),
            "ids": torch.zeros(B, d.gamma, dtype=torch.int32, device=dev),
            "T": torch.zeros(B, W, d.V, dtype=torch.float32, device=dev) if d.verify == "logits" else None,
            "hid": torch.zeros(B, W, d.H, dtype=dm.act_dtype, device=dev) if d.verify == "hidden" else None,
            "acc": torch.zeros(B, dtype=torch.int32, device=dev),
            "com": torch.zeros(B, dtype=torch.int32, device=dev),
            "vids": torch.zeros(B, W, dtype=torch.int32, device=dev),
            "nxt": torch.zeros(B, dtype=torch.int32, device=dev),
            "stamps": torch.zeros(STAMP_ENTRIES, dtype=torch.int64, device=dev),
            "records": [],
            "lengths": torch.full((B,), d.gamma, dtype=torch.int32, device=dev),
        }
        rr["counts"] = torch.from_numpy(rr["counts_h"]).to(dev)
        rounds.append(rr)

    def verify_round(rr):
        if d.verify == "hidden":
            bd.check(dfa.dflash_verify_from_hidden(dm, rr["hid"], rr["ids"], rr["acc"], rr["com"], rr["vids"], hws,
                                                   lengths=rr["lengths"] if args.dspark else None,
                                                   next_anchor=rr["nxt"]), "verify from hidden")
        elif args.dspark:
            bd.check(dfa.dflash_verify_greedy_lengths(rr["T"], rr["ids"], rr["lengths"], rr["acc"], rr["com"],
                                                      rr["vids"], vws, next_anchor=rr["nxt"]), "verify lengths")
        else:
            bd.check(dfa.dflash_verify_greedy(rr["T"], rr["ids"], rr["acc"], rr["com"], rr["vids"], vws,
                                              next_anchor=rr["nxt"]), "verify")

    def run_round(rr, verify=True, trace=False, y=None):
        if trace:
            bd.dflash_trace_begin(bd.DFLASH_TRACE_LM_HEAD | bd.DFLASH_TRACE_ATTENTION | bd.DFLASH_TRACE_PROJECTIONS,
                                  rr["stamps"])
        if args.one_call:
            bd.check(dfa.dflash_draft_round(dm, rr["taps"], offs, rr["counts"], kv, B, rr["anchors"], rr["ids"], rws,
                                            y_out=y), "round")
        else:
            bd.check(dfa.dflash_context_project(dm, rr["taps"], h_new, ws), "context_project")
            bd.check(dfa.dflash_ctx_kv_append(dm, h_new, offs, rr["counts"], kv, ws), "append")
            if args.dspark:
                bd.check(dfa.dflash_draft_forward_dspark(dm, head, rr["anchors"], kv, B, rr["ids"], dws,
                                                         thresholds=thr_d, lengths=rr["lengths"], y_out=y),
                         "forward_dspark")
            else:
                bd.check(dfa.dflash_draft_forward(dm, rr["anchors"], kv, B, rr["ids"], ws, y_out=y), "forward")
        if verify:
            verify_round(rr)
        kv.len.copy_(len0)
        if trace:
            rr["records"] = bd.dflash_trace_end()

    # untimed chain: drafts of each round plant that round's target logits
    log("[bench] building the round chain")
    anchor = gen.make_anchors(d, 0)
    chain_ids, chain_y = [], []
    for r, rr in enumerate(rounds):
        rr["anchors"].copy_(torch.from_numpy(anchor))
        rr["anchors_h"] = anchor.copy()
        run_round(rr, verify=False, y=y_chain)
        ids = rr["ids"].cpu().numpy().copy()
        chain_ids.append(ids)
        chain_y.append(y_chain.float().cpu().numpy())
        if d.verify == "hidden":
            rr["hid"].copy_(torch.from_numpy(plant_hidden(d, w, ids, accept[r], r)))
        else:
            rr["T"].copy_(torch.from_numpy(gen.plant_target_logits(d, ids, accept[r], r)))
        verify_round(rr)
        rr["lengths_h"] = rr["lengths"].cpu().numpy().copy()
        rr["accepted_h"] = np.minimum(accept[r], rr["lengths_h"])     # a pruned block proposes fewer
        assert np.array_equal(rr["acc"].cpu().numpy(), rr["accepted_h"])
        anchor = rr["nxt"].cpu().numpy().copy()
    torch.cuda.synchronize()
    del y_chain

    if args.profile_kernels:
        calibration_copy(dev)
        for rr in rounds:
            run_round(rr)
        torch.cuda.synchronize()
        log(f"[profile-kernels] copy {COPY_BYTES} B, then {R} eager rounds of {d.name}")
        return

    # capture one graph per round, and a second set with launch tracing on (each traced launch
    # records its stamp slice): the headline replays the untraced graphs, the per-kernel
    # durations come from a timed pass over the traced ones
    trace = not args.no_trace
    graphs, tgraphs = [], []
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
            if trace:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    run_round(rr, trace=True)
                tgraphs.append(g)
        torch.cuda.synchronize()

    def step(i, traced=False):
        if use_graph:
            (tgraphs if traced else graphs)[i % R].replay()
        else:
            run_round(rounds[i % R], trace=traced)

    def timed(nsteps, first, traced=False):
        """nsteps consecutive rounds between synchronisations, one event pair
        around all of them: total ms."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(nsteps):
            step(first + i, traced)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def timed_per_step(nsteps, first):
        """nsteps consecutive rounds with an event between rounds: ms of each."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(nsteps):
            step(first + i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(nsteps)]

    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; warmup {args.warmup}, timed {args.steps}")
    for i in range(args.warmup):
        step(i)
    t0 = time.perf_counter()
    gpu_ms = timed(args.steps, args.warmup)
    wall = time.perf_counter() - t0
    nxt = args.warmup + args.steps
    per_step = timed_per_step(args.steps, nxt)
    nxt += args.steps
    if trace:
        traced_ms = timed(args.steps, nxt, traced=True)
        nxt += args.steps

    # the replays must reproduce the chain exactly (deterministic kernels)
    for r, rr in enumerate(rounds):
        assert np.array_equal(rr["ids"].cpu().numpy(), chain_ids[r]), f"round {r}: drafts changed on replay"
        assert np.array_equal(rr["acc"].cpu().numpy(), rr["accepted_h"]), f"round {r}: accepted changed on replay"
        assert np.array_equal(rr["com"].cpu().numpy(), rr["accepted_h"] + 1)
        assert np.array_equal(rr["lengths"].cpu().numpy(), rr["lengths_h"])

    ms_per_step = gpu_ms / args.steps
    blocks_per_s = B * args.steps / (gpu_ms / 1000.0)
    mean_new = float(np.mean([rr["counts_h"].sum() for rr in rounds]))
    # context rows the attention reads after each round's append (all of them, or the windows')
    read_rows = float(np.mean([attended_rows(d, [L + int(c) for L, c in zip(lengths, rr["counts_h"])])
                               for rr in rounds]))
    ab = algorithmic_bytes(d, B, read_rows, 0)
    if args.dspark:
        ab["dspark"] = dspark_bytes(d, B, d.r)
        ab["total"] += ab["dspark"]
    round_gbs = ab["total"] / (ms_per_step / 1000.0) / 1e9

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
        "data": "synthetic (seeded round inputs; prefilled context taps drawn on the device except the "
                "CPU-replayed sequence's)",
        "config": {
            "workload": describe(d, lengths),
            "rounds_cycled": R,
            "mean_committed_rows_appended": round(mean_new / B, 3),
            "launch": "hip graph per round" if use_graph else "eager",
            "round_calls": ("dflash_draft_round" if args.one_call else
                            "dflash_context_project + dflash_ctx_kv_append + dflash_draft_forward"
                            + ("_dspark" if args.dspark else "")) + " + verify",
        },
        "dspark": ({"rank": d.r, "thresholds": "synthetic: %.3f at every step k >= 1" % args.threshold,
                    "mean_proposed_per_block": round(float(np.mean([rr["lengths_h"].mean() for rr in rounds])), 3),
                    "round_algorithmic_bytes_heads": int(ab["dspark"])} if args.dspark else None),
        "tokens_proposed_per_s": round(blocks_per_s * (np.mean([rr["lengths_h"].mean() for rr in rounds])
                                                       if args.dspark else d.gamma), 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, q)), 5) for q in (10, 50, 90)],
        "step_ms_note": "per-round distribution from a second run of the same steps with an event between rounds",
        "round_algorithmic_bytes": int(ab["total"]),
        "round_hbm_frac": round(round_gbs / HBM_PEAK_GBS, 4),
    }

    lengths_after = [attended_rows(d, [L + int(c) for L, c in zip(lengths, rr["counts_h"])]) for rr in rounds]
    if trace:
        table = kernel_table(rounds, lengths_after)
        timing = (f"device wall-clock stamps written by the kernel's workgroups (first start to last end per "
                  f"launch), last replay of each of the {R} rounds in a timed pass of {args.steps} traced rounds "
                  f"({traced_ms / args.steps:.5f} ms per round; the headline replays untraced graphs)")
        res["roofline"] = roofline_entry(table[0], d, timing)
        head = [k for k in table if k["kind"] == "lm_head"]
        if head and head[0] is not table[0]:
            res["roofline_lm_head"] = roofline_entry(head[0], d, timing)
        res["kernels_per_round"] = [{k2: (round(v, 2) if isinstance(v, float) else v) for k2, v in k.items()}
                                    for k in table[:8]]
        traced = sum(k["us_per_round"] for k in table)
        res["traced_ms_per_step"] = round(traced_ms / args.steps, 5)
        res["wall_clock_hz"] = {"measured": round(bd.dflash_wall_clock_hz(), 1),
                                "runtime_reported": round(bd.dflash_wall_clock_hz_reported(), 1)}
        res["traced_share_of_round"] = round(traced / (traced_ms / args.steps * 1e3), 4)
    res["prefill"] = pre
    res["wall_s_timed"] = round(wall, 4)

    # rounds one by one, each after a 1 GiB read that evicts the MALL (a decode loop runs the
    # target model between drafter rounds, streaming its weights; a read leaves the cache
    # clean, where a write would leave dirty lines for the round to write back)
    if args.flush_steps > 0:
        junk = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fl = []
        for i in range(args.flush_steps):
            junk.sum()
            e0.record()
            step(nxt + i)
            e1.record()
            torch.cuda.synchronize()
            fl.append(e0.elapsed_time(e1))
        nxt += args.flush_steps
        del junk
        med = float(np.median(fl))
        res["mall_flushed"] = {"rounds": args.flush_steps, "flush_bytes": FLUSH_BYTES,
                               "ms_p10_p50_p90": [round(float(np.percentile(fl, q)), 5) for q in (10, 50, 90)],
                               "blocks_per_s_at_median": round(B / (med / 1e3), 2)}

    if not args.skip_cpu:
        log(f"[bench] cpu baseline: oracle setup for sequence {cpu_seq} ({lengths[cpu_seq]} context rows)")
        cpu = CpuLeg(d, w, cpu_seq, lengths[cpu_seq], rounds, thresholds)
        seg_gpu = []
        nseg = max(1, args.cpu_segments)
        for sgi in range(nseg):
            log(f"[bench] cpu segment {sgi + 1}/{nseg}")
            cpu.run(args.cpu_seconds / nseg)
            ms = timed(args.steps, nxt)
            nxt += args.steps
            seg_gpu.append(round(B * args.steps / (ms / 1e3), 2))
        agree, compared, misses = cpu.parity([rr["anchors_h"] for rr in rounds], chain_ids, chain_y)
        threads = 1
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except ImportError:
            pass
        res["cpu_baseline"] = {
            "value": round(cpu.done / cpu.seconds, 5),
            "unit": "blocks/s",
            "cores": int(threads),
            "kind": "oracle",
            "sample": f"{cpu.done} rounds of one sequence (seq {cpu_seq}, context {lengths[cpu_seq]}) of the same "
                      f"workload: context projection + K/V append of the committed rows, forward, LM head, "
                      f"verify; numpy float64 bf16-faithful oracle, {cpu.seconds:.1f} s on the host in {nseg} "
                      f"segments interleaved with timed GPU segments; its context prefill untimed",
            "host": host_info(),
            "gpu_blocks_per_s_interleaved_segments": seg_gpu,
            "parity_ids_agree_1e-3": f"{agree}/{compared}",
            "parity_misses": misses,
        }
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
