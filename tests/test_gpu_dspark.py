"""GPU parity of the DSpark heads (page 3: #markov, #confidence, the greedy loop
of forwardRows and Alg 1 pruning) and of the length-capped verify, against the
CPU oracle on the same seeded inputs.

The Markov head's w2 is drawn with a large scale so its bias moves the argmax
away from the plain drafter's (the page initialises it to zero, which the
oracle pins as a reduction). Drafts are compared step by step: a step whose
oracle top-2 gap is at least 1e-3 must agree, or be explained by the GPU's own
base logits (the oracle's scores recomputed from the GPU's Y); after a
difference the two chains condition on different tokens, so the row is not
compared further (no such difference is expected at these gaps).
"""

import numpy as np
import pytest
import torch

import block_diffusion_draft_tap_amd as dfa
from block_diffusion_draft_tap_amd import binding as bd
from gpu_common import compare_ids, log, rel_err, tol, NEAR_TIE
from oracle import dflash_oracle as O
from synth import gen, scaled
from test_gpu_parity import get

pytestmark = pytest.mark.gpu

# (parity case, rank r, w2 scale): fp32 GEMV head; bf16 GQA (GEMV); 21 block rows on matrix
# cores with 3-row GEMV Markov steps; 16 sequences whose Markov steps run on matrix cores
# (r a multiple of 128); the default drafter at full size; int4 weights (bf16 head)
CASES = [("tiny", 16, 1.0), ("gqa_bf16", 64, 1.0), ("batched_r21", 64, 1.0), ("batched_small", 128, 1.0),
         ("default", 256, 0.5), ("wide4_small", 64, 1.0)]


def head_weights(dims, r, std, seed=0):
    d = scaled(dims, r=r)
    return {n: gen.make_weight(d, n, seed=seed, std=(std if n == "markov.w2" else 0.02)) for n in gen.HEAD_NAMES}


def alg1_lengths(conf, thresholds, min_conf):
    """Alg 1 applied to given confidences (host check of the kernel's rule)."""
    B, G = conf.shape
    out = np.full(B, G, np.int32)
    for b in range(B):
        for k in range(1, G):
            thr = thresholds[k] if thresholds is not None else min_conf
            if conf[b, k] < thr:
                out[b] = k
                break
    return out


@pytest.mark.parametrize("name,r,std", CASES, ids=[c[0] for c in CASES])
def test_dspark_forward(name, r, std):
    s = get(name)
    d = s.dims
    hw = head_weights(d, r, std)
    w = dict(s.w)
    w.update(hw)
    head = dfa.DsparkHead(hw)
    anchors = gen.make_anchors(d, 3)
    a_d = torch.from_numpy(anchors).cuda()
    ws = dfa.dspark_workspace(d, r, s.B, s.kv.cap)
    # thresholds: per step, between the oracle's confidences of that step (so some rows are
    # cut), at least 2.5e-2 away from every one of them (several times the confidence bound below)
    tok_o, conf_o, _, ex = O.dspark_forward(w, d, s.ctx, anchors, s.fm)
    thr = np.zeros(d.gamma, np.float32)
    for k in range(1, d.gamma):
        c = np.sort(conf_o[:, k])
        mids = [(c[i] + c[i + 1]) / 2 for i in range(len(c) - 1) if c[i + 1] - c[i] > 5e-2]
        if mids:
            thr[k] = mids[len(mids) // 2]
        else:                                   # one sequence: cut it half way
            thr[k] = c[0] + 0.05 if k == d.gamma // 2 else c[0] - 0.05
    _, _, len_o, _ = O.dspark_greedy(ex["base"], anchors, hw["markov.w1"], hw["markov.w2"], hw["conf.w"],
                                     hw["conf.b"], ex["block"], thresholds=thr)
    ids = torch.empty(s.B, d.gamma, dtype=torch.int32, device="cuda")
    conf = torch.empty(s.B, d.gamma, dtype=torch.float32, device="cuda")
    lengths = torch.empty(s.B, dtype=torch.int32, device="cuda")
    y = torch.empty(s.B, d.gamma, d.H, dtype=s.dm.act_dtype, device="cuda")
    thr_d = torch.from_numpy(thr).cuda()
    bd.check(dfa.dflash_draft_forward_dspark(s.dm, head, a_d, s.kv, s.B, ids, ws, thresholds=thr_d, conf=conf,
                                             lengths=lengths, y_out=y), "forward_dspark")
    torch.cuda.synchronize()
    t = tol(d)
    ey = rel_err(y, ex["Y"])
    assert ey <= t, ey
    # drafts, step by step
    g_ids = ids.cpu().numpy()
    g_conf = conf.cpu().numpy()
    decided = compared = 0
    explained = []
    for b in range(s.B):
        for k in range(d.gamma):
            sc = ex["scores"][b, k]
            top2 = np.sort(sc)[-2:]
            if g_ids[b, k] == tok_o[b, k]:
                compared += 1
                decided += int(top2[1] - top2[0] >= NEAR_TIE)
                continue
            deficit = sc.max() - sc[g_ids[b, k]]
            if top2[1] - top2[0] < NEAR_TIE:
                assert deficit <= NEAR_TIE, (b, k, deficit)
            else:
                # the oracle's scores on the GPU's own Y must pick the GPU's token
                yb = y[b, k:k + 1].float().cpu().numpy().astype(np.float64)
                _, _, base_y = O.lm_head_argmax(yb, w["E_out"], want_logits=True)
                prev = anchors[b] if k == 0 else tok_o[b, k - 1]
                own = base_y[0] + O.dense(hw["markov.w1"])[prev] @ O.dense(hw["markov.w2"])
                assert int(np.argmax(own)) == int(g_ids[b, k]) or own.max() - own[g_ids[b, k]] <= NEAR_TIE, (b, k)
                explained.append((b, k))
            break                      # the chains condition on different tokens from here on
    # confidence of the compared steps (same conditioning token), lengths by Alg 1. The GPU's
    # block rows carry the rounding-order differences Y shows (relative error ey); under a
    # random-sign model they move z = [block; e1] . conf.w by about ey * |block * conf.w|_2,
    # and sigma by at most a quarter of that: the bound is 3 such sigmas (fp32: 1e-5)
    cw = O.dense(hw["conf.w"]).reshape(-1)[:d.d]
    for b in range(s.B):
        same = np.cumprod(np.concatenate([[True], g_ids[b, :-1] == tok_o[b, :-1]])).astype(bool)
        err = np.abs(g_conf[b, same] - conf_o[b, same])
        spread = np.linalg.norm(ex["block"][b][same] * cw[None, :], axis=1)
        bound = 1e-5 if d.wdtype == "f32" else 0.75 * max(ey, 1e-3) * spread
        assert np.all(err <= bound), (b, err, bound)
    g_len = lengths.cpu().numpy()
    assert np.array_equal(g_len, alg1_lengths(g_conf, thr, 0.0))
    if not explained:
        assert np.array_equal(g_len, len_o), (g_len, len_o)
    log(f"[dspark {name} r={r}] Y rel err {ey:.3e}, steps compared {compared}/{s.B * d.gamma} "
        f"({decided} decided), explained by Y {explained}, lengths {g_len.tolist()} (oracle {len_o.tolist()})")
    # no pruning: min_conf 0 keeps every row at gamma; results otherwise identical
    ids2 = torch.empty_like(ids)
    len2 = torch.empty_like(lengths)
    bd.check(dfa.dflash_draft_forward_dspark(s.dm, head, a_d, s.kv, s.B, ids2, ws, min_conf=0.0, lengths=len2),
             "forward_dspark (no pruning)")
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and np.all(len2.cpu().numpy() == d.gamma)


@pytest.mark.parametrize("name", ["gqa_bf16", "batched_small"])
def test_dspark_w2_zero_equals_plain_forward(name):
    """With markov.w2 = 0 (page 3's initialisation) the DSpark drafts are the
    plain drafter's: against the oracle's plain forward at the stated band, and
    equal to the GPU's plain forward wherever that band decides."""
    s = get(name)
    d = s.dims
    hw = head_weights(d, 64 if name == "gqa_bf16" else 128, 1.0)
    hw["markov.w2"] = np.zeros_like(hw["markov.w2"])
    head = dfa.DsparkHead(hw)
    anchors = gen.make_anchors(d, 4)
    a_d = torch.from_numpy(anchors).cuda()
    ids = torch.empty(s.B, d.gamma, dtype=torch.int32, device="cuda")
    y = torch.empty(s.B, d.gamma, d.H, dtype=s.dm.act_dtype, device="cuda")
    ws = dfa.dspark_workspace(d, head.r, s.B, s.kv.cap)
    bd.check(dfa.dflash_draft_forward_dspark(s.dm, head, a_d, s.kv, s.B, ids, ws, y_out=y), "forward_dspark")
    ref = torch.empty_like(ids)
    bd.check(dfa.dflash_draft_forward(s.dm, a_d, s.kv, s.B, ref, s.ws), "forward")
    torch.cuda.synchronize()
    ref_ids, ex = O.draft_forward(s.w, d, s.ctx, anchors, s.fm, return_all=True)
    assert rel_err(y, ex["Y"]) <= tol(d)
    c = compare_ids(ids, ref_ids, ex["logits"], gpu_y=y, head=s.w["E_out"], what=f"dspark w2=0 {name}")
    gap = np.sort(ex["logits"], axis=1)
    decided = (gap[:, -1] - gap[:, -2] >= NEAR_TIE).reshape(s.B, d.gamma)
    assert np.array_equal(ids.cpu().numpy()[decided], ref.cpu().numpy()[decided]) or c["misses"]


@pytest.mark.parametrize("V", [5001, 151936])
def test_verify_lengths_exhaustive(V):
    """Every match pattern of a block-8 verify with every length 1..7, in one
    batch; bit-exact against the oracle."""
    G = 7
    rows = [(bits, l) for bits in range(2 ** G) for l in range(1, G + 1)]
    rows = rows[::7] if V > 100000 else rows       # a sample at the full vocabulary
    B = len(rows)
    rng = np.random.default_rng(V)
    t = rng.integers(0, V, size=(B, G + 1))
    draft = np.empty((B, G), dtype=np.int32)
    lens = np.empty(B, dtype=np.int32)
    for b, (bits, l) in enumerate(rows):
        lens[b] = l
        for k in range(G):
            draft[b, k] = t[b, k] if (bits >> k) & 1 else (t[b, k] + 1 + rng.integers(0, V - 1)) % V
    T = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    T[np.arange(B)[:, None], np.arange(G + 1)[None, :], t] = T.max(axis=2) + 1.0
    acc_o, com_o, ids_o, nxt_o = O.verify_greedy(T, draft, lengths=lens)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    com, nxt = torch.empty_like(acc), torch.empty_like(acc)
    ids = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")
    bd.check(dfa.dflash_verify_greedy_lengths(torch.from_numpy(T).cuda(), torch.from_numpy(draft).cuda(),
                                              torch.from_numpy(lens).cuda(), acc, com, ids,
                                              bd.verify_workspace(B, G, V), next_anchor=nxt), "verify lengths")
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_o) and np.array_equal(com.cpu().numpy(), com_o)
    assert np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(nxt.cpu().numpy(), nxt_o)
