"""Helpers for the GPU parity tests: upload generated inputs, run the oracle on
the same inputs, and compare with the tolerances the workload fixes
(max |gpu - ref| / max |ref| <= 1e-4 for fp32 models, 2e-2 for bf16/int4
models against the bf16-faithful oracle; ids equal except where the
oracle's top-2 logit gap is below 1e-3; integer outputs bit-exact)."""

import sys

import numpy as np
import torch

from oracle import dflash_oracle as O
from synth import gen

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
NEAR_TIE = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol(dims):
    return TOL_F32 if dims.wdtype == "f32" else TOL_BF16


def faithful(dims):
    return dims.wdtype != "f32"


def rel_err(gpu, ref):
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    return float(np.max(np.abs(g - r)) / max(1e-30, np.max(np.abs(r))))


def dev(a, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def top2_gap(logits):
    s = np.sort(logits, axis=-1)
    return s[..., -1] - s[..., -2]


def compare_ids(gpu_ids, ref_ids, ref_logits):
    """Ids must agree wherever the oracle's winner leads by >= 1e-3."""
    g = gpu_ids.cpu().numpy().reshape(-1)
    r = np.asarray(ref_ids).reshape(-1)
    gap = top2_gap(np.asarray(ref_logits).reshape(len(r), -1))
    decided = gap >= NEAR_TIE
    bad = np.nonzero(decided & (g != r))[0]
    assert bad.size == 0, f"id mismatch at {bad[:10]}: gpu {g[bad[:10]]} oracle {r[bad[:10]]}"
    return int(decided.sum())


def oracle_prefill(dims, w, lengths, faithful_mode, stream="ctx"):
    """Oracle context for B sequences with the given lengths; returns
    (Context, list of H_ctx per sequence, list of taps per sequence)."""
    ctx = O.Context(dims.nl, len(lengths), dims.hkv, dims.hd)
    Hs, taps_all = [], []
    for b, L in enumerate(lengths):
        taps = gen.make_taps(dims, 0, int(L), stream=stream, seq=b)
        Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], dims.eps)
        for i in range(dims.nl):
            K, V = O.context_kv(Hc, w[f"bb.{i}.attn_norm"], w[f"bb.{i}.k"], w[f"bb.{i}.v"], dims.hkv, dims.hd,
                                dims.eps, faithful_mode)
            ctx.append(i, b, K, V)
        Hs.append(Hc)
        taps_all.append(taps)
    return ctx, Hs, taps_all
