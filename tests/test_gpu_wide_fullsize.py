"""GPU parity at the wide workloads' full sizes: one prefill and one round of
each, against the CPU oracle.

  * wide    bf16, d 5120, 40q/8kv heads, FFN 17408 (SiLU), vocab 151936,
            context 4096, gamma 7: every context row, the whole round.
  * wide4   the same drafter with int4-g64 weights on every matrix, context
            8192, gamma 4: every context row, the whole round.
  * dflash2 the wide geometry in int4-g64 weights with block 8 (gamma 7), a
            2048-key window over a context of 8192 and rotary positions (base
            1e6); verification from the target's hidden states, planted along
            the head rows of the target tokens that realise the accept plan.
  * batched 16 sequences with contexts of 9050-16059 rows (192,011 in all),
            gamma 7. The whole prefill runs as one call per step (the K/V
            prefill with its ~9.8 GB staged workspace, whose offsets exceed
            32 bits). The two shortest sequences take seeded taps and are
            compared in full (H_ctx, every layer's K/V, the round's drafts, Y
            and winning logits); the other 14 take taps drawn on the device,
            and 20 sampled context rows of each are compared (rows are
            independent, so the oracle computes them one by one from the same
            taps). Verify runs on all 16 against logits planted from the
            oracle's drafts (the two compared sequences) or from seeded ids.

Weights are N(0, 0.02) with norm gains 1 + U(-0.5, 0.5) (so a dropped norm
fails). Each test prints its progress; the oracle's share dominates the run
time (about a minute per workload on the host cores).
"""

import numpy as np
import pytest
import torch

import block_diffusion_draft_tap_amd as dfa
from block_diffusion_draft_tap_amd import binding as bd
from gpu_common import compare_ids, dev, log, rel_err, tol, v_rows
from oracle import dflash_oracle as O
from synth import gen, WIDE, WIDE4, BATCHED, DFLASH2, scaled

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

_weights = {}


def weights_for(d):
    """The stored weights of a workload (wide and batched share one geometry
    and therefore the same generated weights)."""
    key = (d.H, d.m, d.d, d.nl, d.hq, d.hkv, d.hd, d.F, d.V, d.gamma, d.wdtype)
    if key not in _weights:
        _weights.clear()
        log(f"[full {d.name}] generating weights")
        _weights[key] = gen.Model(d, gains="random").materialise()
    return _weights[key]


def bits(t):
    """A bf16 device tensor as the generator's storage format (uint16 bits)."""
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def rot(d, positions):
    """context_kv's rotary arguments for rows at these positions (none without rotation)"""
    return {"positions": np.asarray(positions), "theta": d.rope_theta} if d.rope_theta else {}


def oracle_context(d, w, taps, fm, positions=None):
    Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], d.eps)
    ks, vs = [], []
    pos = np.arange(Hc.shape[0]) if positions is None else positions
    for i in range(d.nl):
        K, V = O.context_kv(Hc, w[f"bb.{i}.attn_norm"], w[f"bb.{i}.k"], w[f"bb.{i}.v"], d.hkv, d.hd, d.eps, fm,
                            **rot(d, pos))
        ks.append(K)
        vs.append(V)
    return Hc, ks, vs


def check_kv_rows(kv, i, b, rows, K, V, t, what):
    rows_t = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=kv.k.device)
    gk = kv.k[i, b][:, rows_t, :].permute(1, 0, 2)          # [rows, hkv, hd]
    gv = v_rows(kv, i, b, rows_t)
    ek, ev = rel_err(gk, K), rel_err(gv, V)
    assert ek <= t and ev <= t, (what, i, b, ek, ev)
    return max(ek, ev)


def full_round(d, full_seqs, device_taps, samples_per_seq=20):
    fm = d.wdtype != "f32"
    t = tol(d)
    W = d.gamma + 1
    w = weights_for(d)
    B = d.B
    lengths = [int(x) for x in gen.context_lengths(d)]
    n = sum(lengths)
    offs_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    log(f"[full {d.name}] {B} sequences, {n} context rows, uploading weights")
    dm = dfa.DeviceModel(d, w)
    cap = max(lengths) + W + 64
    kv = dfa.KVCache(d, B, cap)
    ws = dfa.workspace(d, B, kv.cap)

    # ---- prefill: one projection and one K/V append over every sequence's rows
    act = torch.bfloat16 if fm else torch.float32
    taps_d = [torch.empty(n, d.H, dtype=act, device="cuda") for _ in range(d.m)]
    host_taps = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    for b in range(B):
        s0, s1 = int(offs_h[b]), int(offs_h[b + 1])
        if b in device_taps:
            for j in range(d.m):
                taps_d[j][s0:s1] = torch.randn(s1 - s0, d.H, generator=g, device="cuda").to(act)
        else:
            tb = gen.make_taps(d, 0, lengths[b], stream="ctx", seq=b)
            host_taps[b] = tb
            for j in range(d.m):
                taps_d[j][s0:s1] = dev(tb[j])
    h_ctx = torch.empty(n, d.d, dtype=torch.float32, device="cuda")
    bd.check(dfa.dflash_context_project(dm, taps_d, h_ctx, ws), "context_project (prefill)")
    offs_d = torch.from_numpy(offs_h.astype(np.int32)).cuda()
    kws = dfa.kv_prefill_workspace(d, n) if d.wdtype == "bf16" else ws
    log(f"[full {d.name}] prefill: K/V workspace {kws.numel() / 2**30:.2f} GiB")
    bd.check(dfa.dflash_ctx_kv_append(dm, h_ctx, offs_d, None, kv, kws), "ctx_kv_append (prefill)")
    torch.cuda.synchronize()
    del kws
    assert kv.len.cpu().tolist() == lengths

    # sampled rows of the device-tap sequences: taps copied back, oracle row by row
    rng = np.random.default_rng(99)
    worst = 0.0
    nsamp = 0
    for b in sorted(device_taps):
        s0 = int(offs_h[b])
        rows = np.sort(rng.choice(lengths[b], size=min(samples_per_seq, lengths[b]), replace=False))
        rows[0], rows[-1] = 0, lengths[b] - 1                   # first and last rows always
        rows = np.unique(rows)
        taps_rows = [bits(taps_d[j][s0 + rows]) for j in range(d.m)]
        Hc, ks, vs = oracle_context(d, w, taps_rows, fm, positions=rows)
        e = rel_err(h_ctx[s0 + torch.as_tensor(rows, device="cuda")], Hc)
        assert e <= 1e-4, (b, e)
        worst = max(worst, e)
        for i in range(d.nl):
            worst = max(worst, check_kv_rows(kv, i, b, rows, ks[i], vs[i], t, "sampled"))
        nsamp += len(rows)
    if device_taps:
        log(f"[full {d.name}] {nsamp} sampled context rows of {len(device_taps)} sequences: worst rel err "
            f"{worst:.3e}")
    del taps_d

    # the fully compared sequences: every context row
    ctx = O.Context(d.nl, len(full_seqs), d.hkv, d.hd)
    for q, b in enumerate(full_seqs):
        log(f"[full {d.name}] oracle prefill of sequence {b} ({lengths[b]} rows)")
        Hc, ks, vs = oracle_context(d, w, host_taps[b], fm)
        s0, s1 = int(offs_h[b]), int(offs_h[b + 1])
        e = rel_err(h_ctx[s0:s1], Hc)
        assert e <= 1e-4, (b, e)
        worst = e
        for i in range(d.nl):
            worst = max(worst, check_kv_rows(kv, i, b, np.arange(lengths[b]), ks[i], vs[i], t, "full"))
            ctx.append(i, q, ks[i], vs[i])
        log(f"[full {d.name}] sequence {b}: H_ctx rel err {e:.3e}, worst K/V rel err {worst:.3e}")
    del h_ctx

    # ---- one round: append the previous verify's committed rows, forward, verify
    counts = (np.arange(B) % W + 1).astype(np.int32)           # every count 1..gamma+1 occurs
    taps_r = [gen.make_taps(d, 0, W, stream="round", seq=b) for b in range(B)]
    taps_rd = [dev(np.concatenate([taps_r[b][j] for b in range(B)])) for j in range(d.m)]
    h_new = torch.empty(B * W, d.d, dtype=torch.float32, device="cuda")
    bd.check(dfa.dflash_context_project(dm, taps_rd, h_new, ws), "context_project (round)")
    offs_r = torch.arange(0, (B + 1) * W, W, dtype=torch.int32, device="cuda")
    bd.check(dfa.dflash_ctx_kv_append(dm, h_new, offs_r, torch.from_numpy(counts).cuda(), kv, ws),
             "ctx_kv_append (round)")
    anchors = gen.make_anchors(d, 0)
    ids = torch.empty(B, d.gamma, dtype=torch.int32, device="cuda")
    y = torch.empty(B, d.gamma, d.H, dtype=dm.act_dtype, device="cuda")
    maxl = torch.empty(B, d.gamma, dtype=torch.float32, device="cuda")
    bd.check(dfa.dflash_draft_forward(dm, torch.from_numpy(anchors).cuda(), kv, B, ids, ws, y_out=y,
                                      max_logit=maxl), "forward")
    torch.cuda.synchronize()
    assert kv.len.cpu().tolist() == [lengths[b] + int(counts[b]) for b in range(B)]

    for q, b in enumerate(full_seqs):
        Hr = O.context_project(taps_r[b], w["W_c"], w["ctx_norm"], d.eps)
        e = rel_err(h_new[b * W:(b + 1) * W], Hr)
        assert e <= 1e-4, (b, e)
        for i in range(d.nl):
            K, V = O.context_kv(Hr[:counts[b]], w[f"bb.{i}.attn_norm"], w[f"bb.{i}.k"], w[f"bb.{i}.v"], d.hkv,
                                d.hd, d.eps, fm, **rot(d, lengths[b] + np.arange(counts[b])))
            ctx.append(i, q, K, V)
            rows = np.arange(lengths[b], lengths[b] + counts[b])
            check_kv_rows(kv, i, b, rows, K, V, t, "appended")
    log(f"[full {d.name}] oracle forward of sequences {full_seqs}")
    dq = scaled(d, B=len(full_seqs))
    sel = np.array(full_seqs)
    ref_ids, ex = O.draft_forward(w, dq, ctx, anchors[sel], fm, return_all=True)
    sel_t = torch.as_tensor(sel, device="cuda")
    ey = rel_err(y[sel_t], ex["Y"])
    em = rel_err(maxl[sel_t], ex["max_logit"])
    assert ey <= t and em <= t, (ey, em)
    c = compare_ids(ids[sel_t], ref_ids, ex["logits"], gpu_y=y[sel_t], head=w["E_out"], what=f"full {d.name}")
    log(f"[full {d.name}] Y rel err {ey:.3e}, max-logit rel err {em:.3e}, ids decided {c['decided']}/"
        f"{c['total']}, misses explained by Y: {c['misses']}")

    # verify: drafts of the compared sequences are the oracle's, the others seeded ids
    drafts = np.random.default_rng(5).integers(0, d.V, size=(B, d.gamma)).astype(np.int32)
    drafts[sel] = ref_ids
    acc_plan = gen.accept_schedule(d, 0)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    com, nxt = torch.empty_like(acc), torch.empty_like(acc)
    vid = torch.empty(B, W, dtype=torch.int32, device="cuda")
    if d.verify == "hidden":
        # the target's hidden rows along the head rows of tokens that realise the plan
        rng = np.random.default_rng(6)
        tt = np.concatenate([drafts, rng.integers(0, d.V, size=(B, 1))], axis=1).astype(np.int64)
        for b in range(B):
            if acc_plan[b] < d.gamma:
                tt[b, acc_plan[b]] = (drafts[b, acc_plan[b]] + 1 + rng.integers(0, d.V - 1)) % d.V
        E = O.dense(w["E_out"], rows=tt.reshape(-1))
        hidden = O.bf16(4.0 * E / np.linalg.norm(E, axis=1, keepdims=True)).reshape(B, W, d.H)
        acc_o, com_o, ids_o, nxt_o = O.verify_from_hidden(hidden, w["E_out"], drafts)
        hid_d = torch.from_numpy(hidden.astype(np.float32)).cuda().to(torch.bfloat16)
        bd.check(dfa.dflash_verify_from_hidden(dm, hid_d, torch.from_numpy(drafts).cuda(), acc, com, vid,
                                               dfa.verify_hidden_workspace(d, B), next_anchor=nxt),
                 "verify from hidden")
    else:
        T = gen.plant_target_logits(d, drafts, acc_plan, 0)
        acc_o, com_o, ids_o, nxt_o = O.verify_greedy(T, drafts)
        bd.check(dfa.dflash_verify_greedy(torch.from_numpy(T).cuda(), torch.from_numpy(drafts).cuda(), acc, com,
                                          vid, bd.verify_workspace(B, d.gamma, d.V), next_anchor=nxt), "verify")
    assert np.array_equal(acc_o, acc_plan)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_o) and np.array_equal(com.cpu().numpy(), com_o)
    assert np.array_equal(vid.cpu().numpy(), ids_o) and np.array_equal(nxt.cpu().numpy(), nxt_o)
    log(f"[full {d.name}] verify bit-exact on {B} sequences, accepted {acc_o.tolist()}")
    del dm, kv, ws
    torch.cuda.empty_cache()


def test_wide_full_size():
    full_round(WIDE, full_seqs=[0], device_taps=set())


def test_batched_full_size():
    lengths = gen.context_lengths(BATCHED)
    full = sorted(np.argsort(lengths, kind="stable")[:2].tolist())
    full_round(BATCHED, full_seqs=full, device_taps=set(range(BATCHED.B)) - set(full))


def test_wide4_full_size():
    full_round(WIDE4, full_seqs=[0], device_taps=set())


def test_dflash2_full_size():
    full_round(DFLASH2, full_seqs=[0], device_taps=set())
