"""Pins for the CPU oracle: each test ties a piece of the oracle to something
other than itself -- a library routine (torch CPU, float64), a closed form, an
invariant the method fixes, brute force on tiny inputs, or the values the pages
print. Several tests also plant a plausible mistake in a copy of an oracle
function and check that the pin catches it.
"""

import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import dflash_oracle as O
from synth import gen, TINY, DEFAULT, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(1e-300, np.max(np.abs(b))))


# ----------------------------------------------------------------------------
# number formats


def test_bf16_rounding_known_values():
    one = 1.0
    ulp = 2.0 ** -7                               # bf16 spacing at 1.0
    assert O.bf16(one + ulp / 2) == one           # tie -> even (1.0)
    assert O.bf16(one + 1.5 * ulp) == one + 2 * ulp   # tie -> even (1 + 2 ulp)
    assert O.bf16(one + 0.51 * ulp) == one + ulp
    assert O.bf16(-3.0) == -3.0
    assert O.bf16(0.0) == 0.0
    assert O.bf16(255.5) == 256.0                 # carries into the next binade


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16(x.astype(np.float64)), ref)


def test_decode_bf16_matches_torch():
    bits = gen.f32_to_bf16_bits(np.random.default_rng(1).standard_normal(1000).astype(np.float32))
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.decode_bf16(bits), ref)


def test_int4_dequant_hand_example():
    # one row, one group: codes 0..15 then 15..0 (low nibble first), scale 0.5, bias -2
    q = list(range(16)) + list(range(15, -1, -1)) + [3] * 32
    words = []
    for c in range(8):
        w = 0
        for j in range(8):
            w |= q[8 * c + j] << (4 * j)
        words.append(w)
    w = {"codes": np.array([words], dtype=np.uint32),
         "scales": gen.f32_to_bf16_bits(np.array([[0.5]], dtype=np.float32)),
         "biases": gen.f32_to_bf16_bits(np.array([[-2.0]], dtype=np.float32))}
    got = O.dense(w)
    assert got.shape == (1, 64)
    assert np.array_equal(got[0], 0.5 * np.array(q, dtype=np.float64) - 2.0)


def test_int4_bf16_exact_special_case():
    """When scale*q + bias is exactly bf16-representable, the 4-bit weight and
    the bf16 weight holding the dequantised values are the same matrix."""
    dims = scaled(DEFAULT, wdtype="int4g64", d=128, H=128, V=64)
    w = gen.make_weight(dims, "tok_proj")
    w["scales"][:] = gen.f32_to_bf16_bits(np.full(w["scales"].shape, 0.125, np.float32))
    w["biases"][:] = gen.f32_to_bf16_bits(np.full(w["biases"].shape, -1.0, np.float32))
    deq = O.dense(w)
    as_bf16 = gen.f32_to_bf16_bits(deq.astype(np.float32))
    assert np.array_equal(O.dense(as_bf16), deq)


# ----------------------------------------------------------------------------
# elementwise pieces


def test_rmsnorm_closed_form():
    y = O.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    r = math.sqrt(12.5)
    assert np.allclose(y, [3.0 / r, 8.0 / r], rtol=0, atol=1e-15)


def test_rmsnorm_matches_torch_and_invariants():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96))
    g = 1 + rng.uniform(-0.5, 0.5, 96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    y = O.rmsnorm(x, g, 1e-6)
    assert rel(y, ref) < 1e-14
    # scale invariance and unit RMS of y/g
    assert rel(O.rmsnorm(3.7 * x, g, 0.0), O.rmsnorm(x, g, 0.0)) < 1e-14
    assert np.allclose(np.sqrt(np.mean((O.rmsnorm(x, g, 0.0) / g) ** 2, axis=-1)), 1.0, atol=1e-14)


def test_activations_match_torch():
    x = np.linspace(-8, 8, 4001)
    t = torch.from_numpy(x)
    assert rel(O.gelu_tanh(x), torch.nn.functional.gelu(t, approximate="tanh").numpy()) < 1e-14
    assert rel(O.silu(x), torch.nn.functional.silu(t).numpy()) < 1e-14


# ----------------------------------------------------------------------------
# attention


def _torch_attention(Q, K, V, scale, mask=None):
    hq, hkv = Q.shape[1], K.shape[1]
    q = torch.from_numpy(Q).permute(1, 0, 2)
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=False, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2), (5, 1)])
def test_attention_matches_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((5, hq, 16))
    K = rng.standard_normal((37, hkv, 16))
    V = rng.standard_normal((37, hkv, 16))
    assert rel(O.attention(Q, K, V, 0.25), _torch_attention(Q, K, V, 0.25)) < 1e-13


def test_attention_invariants():
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((3, 2, 8))
    V = rng.standard_normal((1, 2, 8))
    K = rng.standard_normal((1, 2, 8))
    # a single key returns its value
    assert np.allclose(O.attention(Q, K, V, 1.0), np.broadcast_to(V[0], (3, 2, 8)), atol=1e-15)
    # identical keys return the mean of the values
    K4 = np.repeat(K, 4, axis=0)
    V4 = rng.standard_normal((4, 2, 8))
    assert np.allclose(O.attention(Q, K4, V4, 1.0), np.broadcast_to(V4.mean(axis=0), (3, 2, 8)), atol=1e-14)
    # permuting (key, value) rows leaves the output unchanged
    K9, V9 = rng.standard_normal((9, 2, 8)), rng.standard_normal((9, 2, 8))
    p = rng.permutation(9)
    assert rel(O.attention(Q, K9[p], V9[p], 0.3), O.attention(Q, K9, V9, 0.3)) < 1e-14
    # weights of each row sum to one: values = one-hot key index recover the weights
    Vid = np.zeros((9, 2, 9))
    for j in range(9):
        Vid[j, :, j] = 1.0
    Qw = rng.standard_normal((3, 2, 8))
    A = O.attention(np.concatenate([Qw, np.zeros((3, 2, 1))], axis=2),
                    np.concatenate([K9, np.zeros((9, 2, 1))], axis=2), Vid, 0.3)
    assert np.allclose(A.sum(axis=-1), 1.0, atol=1e-14)


def test_varlen_equals_padding_bias():
    """Attending over the first n context rows equals attending over a padded
    context whose pad columns carry a -1e9 additive bias (page 3, #maskBias)."""
    rng = np.random.default_rng(5)
    G, hq, hkv, hd = 4, 4, 2, 16
    n, pad = 11, 6
    Q = rng.standard_normal((G, hq, hd))
    Kc, Vc = rng.standard_normal((n + pad, hkv, hd)), rng.standard_normal((n + pad, hkv, hd))
    Kb, Vb = rng.standard_normal((G, hkv, hd)), rng.standard_normal((G, hkv, hd))
    bias = np.zeros(n + pad + G)
    bias[n:n + pad] = -1e9
    padded = _torch_attention(Q, np.concatenate([Kc, Kb]), np.concatenate([Vc, Vb]), hd ** -0.5,
                              mask=torch.from_numpy(bias))
    got = O.attention(Q, np.concatenate([Kc[:n], Kb]), np.concatenate([Vc[:n], Vb]), hd ** -0.5)
    assert rel(got, padded) < 1e-13


# ----------------------------------------------------------------------------
# model-level pins (tiny shapes)


def tiny_model(gains="random", **kw):
    dims = scaled(TINY, **kw) if kw else TINY
    return dims, gen.Model(dims, gains=gains).materialise()


def tiny_context(dims, w, L, faithful=False, seed_stream="ctx"):
    taps = gen.make_taps(dims, 0, L, stream=seed_stream)
    Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], dims.eps)
    ctx = O.Context(dims.nl, dims.B, dims.hkv, dims.hd)
    O.append_context(ctx, w, dims, Hc, [list(range(L))], [L], faithful)
    return ctx, Hc, taps


def test_context_project_concat_order_and_linearity():
    """A one-hot tap row selects one column of W_c, so the tap order of the
    concatenation is pinned: tap j, column c is input feature j*H + c."""
    dims, w = tiny_model()
    H = dims.H
    for j, c in [(0, 5), (1, 17), (1, H - 1)]:
        taps = [np.zeros((1, H), np.float32) for _ in range(dims.m)]
        taps[j][0, c] = 1.0
        got = O.context_project(taps, w["W_c"], w["ctx_norm"], 0.0)
        col = O.dense(w["W_c"])[:, j * H + c]
        assert rel(got[0], O.rmsnorm(col, O.dense(w["ctx_norm"]), 0.0)) < 1e-14
    # linearity before the norm: the norm removes a positive scale
    taps = gen.make_taps(dims, 0, 3)
    a = O.context_project(taps, w["W_c"], w["ctx_norm"], 0.0)
    b = O.context_project([4.0 * t for t in taps], w["W_c"], w["ctx_norm"], 0.0)
    assert rel(a, b) < 1e-14


def test_context_kv_reprojects_with_each_layers_norm():
    """Layer i re-normalises H_ctx with its own attn_norm before W_K / W_V
    (page 3, projectContextRows and the 'SAME norm as block' line of #layer):
    K is invariant to a positive rescale of H_ctx and linear in the gain."""
    dims, w = tiny_model()
    rng = np.random.default_rng(6)
    Hc = rng.standard_normal((5, dims.d))
    K1, V1 = O.context_kv(Hc, w["bb.0.attn_norm"], w["bb.0.k"], w["bb.0.v"], dims.hkv, dims.hd, 0.0, False)
    K2, V2 = O.context_kv(9.0 * Hc, w["bb.0.attn_norm"], w["bb.0.k"], w["bb.0.v"], dims.hkv, dims.hd, 0.0, False)
    assert rel(K1, K2) < 1e-14 and rel(V1, V2) < 1e-14
    g2 = (2.0 * O.dense(w["bb.0.attn_norm"])).astype(np.float32)
    K3, _ = O.context_kv(Hc, g2, w["bb.0.k"], w["bb.0.v"], dims.hkv, dims.hd, 0.0, False)
    assert rel(K3, 2.0 * K1) < 1e-14

    # planted mistake: dropping the per-layer norm breaks the scale invariance
    def no_norm_kv(H, g, Wk, Wv):
        return H @ O.dense(Wk).T
    assert rel(no_norm_kv(9.0 * Hc, None, w["bb.0.k"], None), no_norm_kv(Hc, None, w["bb.0.k"], None)) > 1.0


def test_context_append_chunk_invariance_and_per_layer_weights():
    dims, w = tiny_model()
    L = 20
    taps = gen.make_taps(dims, 0, L)
    Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], dims.eps)
    one = O.Context(dims.nl, 1, dims.hkv, dims.hd)
    O.append_context(one, w, dims, Hc, [list(range(L))], [L], False)
    # rows are independent: projecting in chunks gives identical caches
    two = O.Context(dims.nl, 1, dims.hkv, dims.hd)
    for s, e in [(0, 7), (7, 8), (8, 20)]:
        part = O.context_project([t[s:e] for t in taps], w["W_c"], w["ctx_norm"], dims.eps)
        O.append_context(two, w, dims, part, [list(range(e - s))], [e - s], False)
    for i in range(dims.nl):
        assert np.array_equal(one.k[i][0], two.k[i][0]) or rel(two.k[i][0], one.k[i][0]) < 1e-14
    # a count below the row count appends only the first rows
    part = O.Context(dims.nl, 1, dims.hkv, dims.hd)
    O.append_context(part, w, dims, Hc, [list(range(L))], [5], False)
    assert part.length(0) == 5 and rel(part.k[1][0], one.k[1][0][:5]) < 1e-14
    # perturbing layer 1's W_K changes only cache 1
    w2 = dict(w)
    w2["bb.1.k"] = w["bb.1.k"] * np.float32(2.0)
    three = O.Context(dims.nl, 1, dims.hkv, dims.hd)
    O.append_context(three, w2, dims, Hc, [list(range(L))], [L], False)
    assert np.array_equal(three.k[0][0], one.k[0][0]) and np.array_equal(three.v[1][0], one.v[1][0])
    assert rel(three.k[1][0], 2.0 * one.k[1][0]) < 1e-15


def test_block_init_rows():
    dims, w = tiny_model()
    anchors = np.array([7, 300], dtype=np.int32)
    H = O.block_init(anchors, w["E_in"], w["tok_proj"], w["mask_emb"], w["block_pos"], dims.gamma, False)
    P = O.dense(w["block_pos"])
    E = O.dense(w["E_in"])
    T = O.dense(w["tok_proj"])
    for b, a in enumerate(anchors):
        # brute force: explicit sums
        row0 = np.array([sum(E[a, c] * T[o, c] for c in range(dims.H)) for o in range(dims.d)]) + P[0]
        assert rel(H[b, 0], row0) < 1e-13
        for k in range(1, dims.gamma):
            assert np.array_equal(H[b, k], O.dense(w["mask_emb"])[k - 1] + P[k])


def _layer_inputs(dims, w, L=9, B=1, seed=7):
    ctx, _, _ = tiny_context(dims, w, L)
    rng = np.random.default_rng(seed)
    return ctx, rng.standard_normal((B, dims.gamma, dims.d))


def test_draft_layer_is_noncausal_and_context_read_only():
    """Perturbing the LAST block row changes row 0's output (no causal mask,
    page 'A Refusal Is Not A Failure', is_causal is false); the context
    arrays are not modified by a layer."""
    dims, w = tiny_model()
    ctx, Hd = _layer_inputs(dims, w)
    k_before = [a.copy() for a in ctx.k[0]]
    out = O.draft_layer(Hd, ctx, 0, w, dims, False)
    assert all(np.array_equal(a, b) for a, b in zip(ctx.k[0], k_before))
    Hd2 = Hd.copy()
    Hd2[0, -1] += 0.5
    out2 = O.draft_layer(Hd2, ctx, 0, w, dims, False)
    assert rel(out2[0, 0], out[0, 0]) > 1e-6

    # planted mistake: a causal block mask makes row 0 blind to the last row
    def causal_attention(Q, K, V, scale):
        Lc = K.shape[0] - Q.shape[0]
        Oc = np.empty_like(Q)
        for r in range(Q.shape[0]):
            Oc[r:r + 1] = O.attention(Q[r:r + 1], K[:Lc + r + 1], V[:Lc + r + 1], scale)
        return Oc
    c1 = O.draft_layer(Hd, ctx, 0, w, dims, False, attn=causal_attention)
    c2 = O.draft_layer(Hd2, ctx, 0, w, dims, False, attn=causal_attention)
    assert rel(c2[0, 0], c1[0, 0]) < 1e-14          # the pin above would catch it


def test_draft_layer_matches_torch_layer():
    """The whole layer against an independent torch float64 composition
    using library primitives (rms_norm, SDPA, gelu)."""
    dims, w = tiny_model()
    ctx, Hd = _layer_inputs(dims, w, L=13)
    got = O.draft_layer(Hd, ctx, 1, w, dims, False)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    W = {n: t(O.dense(w[f"bb.1.{n}"])) for n in ("q", "k", "v", "o", "gate", "up", "down", "attn_norm", "ff_norm")}
    x = t(Hd[0])
    n = torch.nn.functional.rms_norm(x, (dims.d,), W["attn_norm"], eps=dims.eps)
    q = (n @ W["q"].T).reshape(dims.gamma, dims.hq, dims.hd).transpose(0, 1)
    kb = (n @ W["k"].T).reshape(dims.gamma, dims.hkv, dims.hd).transpose(0, 1)
    vb = (n @ W["v"].T).reshape(dims.gamma, dims.hkv, dims.hd).transpose(0, 1)
    k = torch.cat([t(ctx.k[1][0]).transpose(0, 1), kb], dim=1)
    v = torch.cat([t(ctx.v[1][0]).transpose(0, 1), vb], dim=1)
    a = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=False)
    x = x + a.transpose(0, 1).reshape(dims.gamma, -1) @ W["o"].T
    n2 = torch.nn.functional.rms_norm(x, (dims.d,), W["ff_norm"], eps=dims.eps)
    x = x + (torch.nn.functional.gelu(n2 @ W["gate"].T, approximate="tanh") * (n2 @ W["up"].T)) @ W["down"].T
    assert rel(got[0], x.numpy()) < 1e-12


def _torch_nonretained_layer(dims, w, taps, Hd, layer, faithful=False):
    """One drafter layer for one sequence by the non-retained branch of page 3
    (#layer with the context passed in, no cache): Eq 2 from the raw taps, then
    the layer's own attn_norm applied to BOTH the context and the block, one
    K/V projection over [context ++ block] rows, SDPA with no mask (grouped
    query heads), O projection and the gated FFN. Every step is a torch float64
    library call; nothing here reuses the oracle. With faithful, values are cast
    to bfloat16 and back at the rounding points the GPU contract names."""
    t = lambda a: torch.from_numpy(np.array(a, dtype=np.float64))
    r = (lambda x: x.to(torch.bfloat16).to(torch.float64)) if faithful else (lambda x: x)
    F = torch.nn.functional
    W = {n: t(O.dense(w[f"bb.{layer}.{n}"])) for n in
         ("q", "k", "v", "o", "gate", "up", "down", "attn_norm", "ff_norm")}
    # Eq 2: concatenate the taps on the feature axis, project, normalise with ctx_norm
    X = torch.cat([t(O.dense(a)) for a in taps], dim=1)
    Hc = F.rms_norm(X @ t(O.dense(w["W_c"])).T, (dims.d,), t(O.dense(w["ctx_norm"])), eps=dims.eps)
    x = t(Hd)
    G, Lc = x.shape[0], Hc.shape[0]
    # the same norm and the same K/V weights for the context rows and the block rows
    rows = torch.cat([Hc, x], dim=0)
    n_all = r(F.rms_norm(rows, (dims.d,), W["attn_norm"], eps=dims.eps))
    k = r(n_all @ W["k"].T).reshape(Lc + G, dims.hkv, dims.hd).transpose(0, 1)
    v = r(n_all @ W["v"].T).reshape(Lc + G, dims.hkv, dims.hd).transpose(0, 1)
    q = r(n_all[Lc:] @ W["q"].T).reshape(G, dims.hq, dims.hd).transpose(0, 1)
    a = F.scaled_dot_product_attention(q, k, v, is_causal=False, enable_gqa=True)
    x = x + r(a.transpose(0, 1).reshape(G, -1)) @ W["o"].T
    n2 = r(F.rms_norm(x, (dims.d,), W["ff_norm"], eps=dims.eps))
    act = F.silu(n2 @ W["gate"].T) if dims.act == "silu" else F.gelu(n2 @ W["gate"].T, approximate="tanh")
    return (x + r(act * (n2 @ W["up"].T)) @ W["down"].T).numpy()


# a grouped-query SiLU layer whose K/V width (hkv * hd = 64) differs from the drafter
# width (d = 256), and a square multi-head GELU layer (hkv * hd = d) on which a
# transposed K/V weight still has the right shape
EQ3_GQA = dict(H=96, m=3, d=256, hq=4, hkv=1, hd=64, F=192, act="silu", gamma=3, V=64)
EQ3_MHA = dict(H=96, m=2, d=128, hq=2, hkv=2, hd=64, F=160, gamma=4, V=64)


def _eq3_case(geom, L=11, seed=21):
    dims = scaled(TINY, **geom)
    w = gen.Model(dims, gains="random").materialise()
    taps = gen.make_taps(dims, 0, L, stream="ctx")
    Hd = np.random.default_rng(seed).standard_normal((dims.gamma, dims.d))
    return dims, w, taps, Hd


def _oracle_retained_layer(dims, w, taps, Hd, layer, faithful=False):
    Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], dims.eps)
    ctx = O.Context(dims.nl, 1, dims.hkv, dims.hd)
    O.append_context(ctx, w, dims, Hc, [list(range(Hc.shape[0]))], [Hc.shape[0]], faithful)
    return O.draft_layer(Hd[None], ctx, layer, w, dims, faithful)[0]


@pytest.mark.parametrize("geom", [EQ3_GQA, EQ3_MHA], ids=["gqa_silu_nonsquare", "mha_gelu_square"])
@pytest.mark.parametrize("layer", [0, 1])
def test_eq3_context_half_against_nonretained_torch_layer(geom, layer):
    """Eq 3 with the context K/V computed from H_ctx: the oracle's retained
    path (context_kv into a Context, then draft_layer) equals a torch float64
    layer that re-projects the context itself from the taps."""
    dims, w, taps, Hd = _eq3_case(geom)
    got = _oracle_retained_layer(dims, w, taps, Hd, layer)
    ref = _torch_nonretained_layer(dims, w, taps, Hd, layer)
    assert rel(got, ref) < 1e-12
    # the faithful (bf16-rounding) mode against the same layer with the casts in torch.
    # The roundings move the output by 4e-5..1.2e-4 from the fp64 layer; the two
    # faithful computations agree far inside that (a summation order that flips one
    # rare rounding moves a single element by one bf16 ulp, well under 1e-5 here)
    got_f = _oracle_retained_layer(dims, w, taps, Hd, layer, faithful=True)
    ref_f = _torch_nonretained_layer(dims, w, taps, Hd, layer, faithful=True)
    assert rel(got_f, ref_f) < 1e-5 and rel(got_f, ref) > 3e-5


def test_eq3_context_half_catches_planted_slips(monkeypatch):
    """Plausible slips in the context half of Eq 3, planted in copies of
    context_kv, each fail the non-retained torch pin above."""
    real = O.context_kv

    def transposed_wk(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful):
        n = O.rmsnorm(H_ctx, O.dense(g_attn), eps)
        K = n @ O.dense(W_k)                         # W_K not transposed
        V = n @ O.dense(W_v).T
        return K.reshape(len(H_ctx), hkv, hd), V.reshape(len(H_ctx), hkv, hd)

    def swapped_kv(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful):
        K, V = real(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful)
        return V, K

    def head_major_reshape(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful):
        K, V = real(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful)
        n = len(H_ctx)
        return (K.reshape(n, hkv * hd).reshape(n, hd, hkv).transpose(0, 2, 1),
                V.reshape(n, hkv * hd).reshape(n, hd, hkv).transpose(0, 2, 1))

    def block_weights_for_context(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful):
        # the context projected with the NEXT layer's W_K / W_V (layers 0 and 1 of the case)
        return real(H_ctx, g_attn, w["bb.1.k"], w["bb.1.v"], hkv, hd, eps, faithful)

    # the square case: every slip keeps valid shapes and must change the values
    dims, w, taps, Hd = _eq3_case(EQ3_MHA)
    ref = _torch_nonretained_layer(dims, w, taps, Hd, 0)
    for slip in (transposed_wk, swapped_kv, head_major_reshape, block_weights_for_context):
        monkeypatch.setattr(O, "context_kv", slip)
        bad = _oracle_retained_layer(dims, w, taps, Hd, 0)
        monkeypatch.setattr(O, "context_kv", real)
        assert rel(bad, ref) > 1e-4, slip.__name__
    # the non-square case: the transposed weight cannot even be applied
    dims, w, taps, Hd = _eq3_case(EQ3_GQA)
    monkeypatch.setattr(O, "context_kv", transposed_wk)
    with pytest.raises(ValueError):
        _oracle_retained_layer(dims, w, taps, Hd, 0)


def test_single_key_layer_closed_form():
    """Empty context and a one-row block: attention over the single block key
    returns V_b exactly, so the layer has a closed form."""
    dims, w = tiny_model(gamma=1)
    ctx = O.Context(dims.nl, 1, dims.hkv, dims.hd)
    Hd = np.random.default_rng(8).standard_normal((1, 1, dims.d))
    got = O.draft_layer(Hd, ctx, 0, w, dims, False)
    D = lambda n: O.dense(w[f"bb.0.{n}"])
    n = O.rmsnorm(Hd[0], D("attn_norm"), dims.eps)
    x = Hd[0] + (n @ D("v").T) @ D("o").T          # hq == hkv: head h reads kv head h
    n2 = O.rmsnorm(x, D("ff_norm"), dims.eps)
    x = x + (O.gelu_tanh(n2 @ D("gate").T) * (n2 @ D("up").T)) @ D("down").T
    assert rel(got[0], x) < 1e-13


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    Q = rng.standard_normal((4, 6, 8))
    K, V = rng.standard_normal((10, 2, 8)), rng.standard_normal((10, 2, 8))
    mha = O.attention(Q, np.repeat(K, 3, axis=1), np.repeat(V, 3, axis=1), 0.35)
    assert rel(O.attention(Q, K, V, 0.35), mha) < 1e-15


# ----------------------------------------------------------------------------
# LM head argmax


def test_lm_head_argmax_planted_and_ties():
    rng = np.random.default_rng(10)
    H, V = 16, 37
    E = rng.standard_normal((V, H)).astype(np.float32)
    Y = np.zeros((3, H))
    Y[0, 4] = 1.0                       # logits = E[:, 4]
    E[:, 4] = -1.0
    E[22, 4] = 5.0
    E[9, 4] = 5.0                       # tie at 9 and 22 -> 9
    Y[1, 2] = 1.0
    E[:, 2] = 0.0                       # all equal -> 0
    Y[2] = rng.standard_normal(H)
    for chunk in (4, 5, 100):
        ids, best, logits = O.lm_head_argmax(Y, E, chunk=chunk, want_logits=True)
        assert ids[0] == 9 and ids[1] == 0
        full = Y @ E.astype(np.float64).T
        assert ids[2] == int(np.argmax(full[2])) and best[2] == full[2].max()


# ----------------------------------------------------------------------------
# verification


def _planted_verify_inputs(G, V, pattern, rng):
    """Target argmax t and drafts agreeing exactly where pattern[k] is True."""
    t = rng.integers(0, V, size=G + 1)
    draft = np.array([t[k] if pattern[k] else (t[k] + 1 + rng.integers(0, V - 1)) % V for k in range(G)])
    T = rng.standard_normal((1, G + 1, V)).astype(np.float32)
    for j in range(G + 1):
        T[0, j, t[j]] = T[0, j].max() + 1.0
    return T, draft[None, :].astype(np.int32), t


@pytest.mark.parametrize("G", [1, 2, 4, 5, 7])
def test_verify_exhaustive_match_patterns(G):
    rng = np.random.default_rng(11)
    V = 50
    for bits in range(2 ** G):
        pattern = [(bits >> k) & 1 == 1 for k in range(G)]
        expect = next((k for k in range(G) if not pattern[k]), G)
        T, draft, t = _planted_verify_inputs(G, V, pattern, rng)
        acc, com, ids, nxt = O.verify_greedy(T, draft)
        assert acc[0] == expect and com[0] == expect + 1
        assert list(ids[0, :expect + 1]) == list(t[:expect + 1]) and all(ids[0, expect + 1:] == -1)
        assert nxt[0] == t[expect]
        assert 0 <= acc[0] <= G


def test_verify_printed_examples():
    g = json.load(open(os.path.join(GOLDEN, "verify_examples.json")))
    G = g["gamma"]
    rng = np.random.default_rng(12)
    for case in g["cases"]:
        assert case["block"] == G + 1
        k = case["matching_prefix"]
        pattern = [i < k for i in range(G)]
        T, draft, _ = _planted_verify_inputs(G, 1000, pattern, rng)
        acc, com, _, _ = O.verify_greedy(T, draft)
        assert (int(acc[0]), int(com[0])) == (case["accepted"], case["committed"])

    # planted mistake: counting the committed tokens without the bonus token
    def off_by_one(T, d):
        a, c, i, n = O.verify_greedy(T, d)
        return a, a, i, n
    T, draft, _ = _planted_verify_inputs(G, 1000, [True] * G, rng)
    assert int(off_by_one(T, draft)[1][0]) != g["cases"][0]["committed"]


def test_verify_tie_resolves_to_lowest_index():
    T = np.zeros((1, 3, 10), dtype=np.float32)
    T[0, 0, [3, 7]] = 2.0
    T[0, 1, [1, 2]] = 2.0
    acc, com, ids, _ = O.verify_greedy(T, np.array([[3, 1]], dtype=np.int32))
    assert acc[0] == 2 and list(ids[0]) == [3, 1, 0]
    acc, _, _, _ = O.verify_greedy(T, np.array([[7, 1]], dtype=np.int32))
    assert acc[0] == 0


# ----------------------------------------------------------------------------
# composition


def test_forward_closed_form_without_layers():
    """No layers and a one-row block: with tok_proj zero and block_pos[0] a
    one-hot e_j, the block row is e_j, out_norm gives sqrt(d) e_j (eps 0),
    out_proj maps it to sqrt(d) W_out[:, j], and the head's argmax is planted."""
    dims = scaled(TINY, nl=0, gamma=1, eps=0.0)
    w = gen.Model(dims).materialise()
    j, c, target = 11, 40, 123
    w["tok_proj"] = np.zeros_like(w["tok_proj"])
    bp = np.zeros_like(w["block_pos"])
    bp[0, j] = 1.0
    w["block_pos"] = bp
    Wout = np.zeros_like(w["out_proj"])
    Wout[c, j] = 1.0
    w["out_proj"] = Wout
    E = np.abs(w["E_out"]).copy()
    E[:, c] = np.linspace(0.0, 1.0, dims.V, dtype=np.float32)[::-1].copy()
    E[target, c] = 2.0
    w["E_out"] = E
    ctx = O.Context(0, 1, dims.hkv, dims.hd)
    ids, extra = O.draft_forward(w, dims, ctx, np.array([5], np.int32), False, return_all=True)
    assert ids[0, 0] == target
    assert abs(extra["max_logit"][0, 0] - 2.0 * math.sqrt(dims.d)) < 1e-12


def test_default_config_matches_page_defaults():
    g = json.load(open(os.path.join(GOLDEN, "default_drafter_config.json")))
    assert (DEFAULT.gamma, DEFAULT.d, DEFAULT.nl, DEFAULT.hq, DEFAULT.F // DEFAULT.d, DEFAULT.m) == \
        (g["gamma"], g["dDraft"], g["nLayers"], g["nHeads"], g["ffMult"], g["n_taps"])
    geo = json.load(open(os.path.join(GOLDEN, "dflash2_geometry.json")))
    from synth import WIDE, WIDE4
    for c in (WIDE, WIDE4):
        assert (c.nl, c.m, c.H, c.F, c.hd) == (geo["n_layers"], geo["n_taps"], geo["hidden_size"],
                                               geo["intermediate_size"], geo["head_dim"])
    assert WIDE.gamma + 1 == geo["block"] and WIDE.gamma == geo["proposals"]


def test_multi_round_accept_schedule_tiny():
    """Planted target logits realise the accept schedule r mod 5 through the
    oracle's own verify; committed rows are appended and the next anchor is
    the target's token at the first disagreement."""
    dims, w = tiny_model(gains="ones")
    ctx, _, _ = tiny_context(dims, w, dims.L)
    anchor = gen.make_anchors(dims, 0)
    seen = set()
    for r in range(6):
        ids = O.draft_forward(w, dims, ctx, anchor, False)
        a = gen.accept_schedule(dims, r)
        T = gen.plant_target_logits(dims, ids, a, r)
        acc, com, out_ids, nxt = O.verify_greedy(T, ids)
        assert np.array_equal(acc, a)
        assert list(out_ids[0, :acc[0]]) == list(ids[0, :acc[0]])
        seen.add(int(acc[0]))
        taps = gen.make_taps(dims, r * (dims.gamma + 1), dims.gamma + 1, stream="round")
        Hc = O.context_project(taps, w["W_c"], w["ctx_norm"], dims.eps)
        before = ctx.length(0)
        O.append_context(ctx, w, dims, Hc, [list(range(dims.gamma + 1))], com, False)
        assert ctx.length(0) == before + int(com[0])
        anchor = nxt
    assert seen == set(range(dims.gamma + 1))


def test_faithful_mode_is_close_to_pure():
    dims = scaled(TINY, wdtype="bf16")
    w = gen.Model(dims, gains="random").materialise()
    ctx_p, _, _ = tiny_context(dims, w, 16, faithful=False)
    ctx_f, _, _ = tiny_context(dims, w, 16, faithful=True)
    anchor = np.array([3], np.int32)
    _, ep = O.draft_forward(w, dims, ctx_p, anchor, False, return_all=True)
    _, ef = O.draft_forward(w, dims, ctx_f, anchor, True, return_all=True)
    r = rel(ef["Y"], ep["Y"])
    assert 1e-5 < r < 3e-2          # rounding is applied, and it is small
    # faithful K/V caches hold bf16 values exactly
    assert np.array_equal(O.bf16(ctx_f.k[0][0]), ctx_f.k[0][0])


# ----------------------------------------------------------------------------
# DSpark sequential head, confidence head and pruning (page 3: #markov, #confidence,
# the greedy loop of forwardRows, Alg 1)


def _dspark_model(r=16, w2_std=0.02, **kw):
    dims = scaled(TINY, r=r, **kw)
    return dims, gen.Model(dims, gains="random", stds={"markov.w2": w2_std}).materialise()


def test_dspark_w2_zero_reduces_to_the_parallel_drafter():
    """markov.w2 starts at zero (page 3's initialisation: the drafter then is
    plain parallel DFlash): every step's scores are the base logits, so the
    tokens are the plain forward's greedy ids, whatever w1 and the anchors."""
    dims, w = _dspark_model()
    w["markov.w2"] = np.zeros_like(w["markov.w2"])
    ctx, _, _ = tiny_context(dims, w, 12)
    anchors = np.array([5], np.int32)
    ids, ex = O.draft_forward(w, dims, ctx, anchors, False, return_all=True)
    tok, conf, lengths, extra = O.dspark_forward(w, dims, ctx, anchors, False)
    assert np.array_equal(tok, ids)
    assert rel(extra["base"].reshape(-1, dims.V), ex["logits"]) < 1e-14
    assert np.array_equal(lengths, [dims.gamma]) and np.all((conf > 0) & (conf < 1))


def _planted_chain(B=3, G=6, V=40, r=8, big=50.0, seed=0):
    """Base logits of small noise, w1 one-hot (row v = e_{v mod r}), w2 row j
    one-hot at succ[j] scaled by `big`: from token p the Markov bias favours
    succ[p mod r] by `big`, so the greedy chain is p -> succ[p mod r]."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((B, G, V)) * 0.1
    w1 = np.zeros((V, r))
    w1[np.arange(V), np.arange(V) % r] = 1.0
    succ = rng.permutation(V)[:r]
    w2 = np.zeros((r, V))
    w2[np.arange(r), succ] = big
    return base, w1, w2, succ


def test_dspark_follows_a_planted_markov_chain():
    B, G, V, r, d = 3, 6, 40, 8, 5
    base, w1, w2, succ = _planted_chain(B, G, V, r)
    anchors = np.array([3, 17, 38])
    cw, cb = np.zeros((d + r, 1)), np.zeros(1)
    block = np.zeros((B, G, d))
    tok, conf, lengths, scores = O.dspark_greedy(base, anchors, w1, w2, cw, cb, block)
    for b in range(B):
        p = anchors[b]
        for k in range(G):
            p = succ[p % r]
            assert tok[b, k] == p, (b, k)
    assert np.allclose(conf, 0.5) and np.array_equal(lengths, [G] * B)

    # planted mistake: a parallel head that conditions every step on the anchor
    # (no sequential dependence) proposes succ[anchor mod r] at every position
    def parallel(base, anchors, w1, w2):
        bias = w1[anchors] @ w2
        return np.argmax(base + bias[:, None, :], axis=-1)
    assert not np.array_equal(parallel(base, anchors, w1, w2), tok)


def test_dspark_argmax_ties_go_to_the_lowest_index():
    B, G, V, r, d = 1, 2, 12, 4, 3
    base = np.zeros((B, G, V))
    base[0, 0, [7, 2, 9]] = 1.0                 # a three-way tie at step 0 -> token 2
    w1 = np.zeros((V, r))
    w2 = np.zeros((r, V))
    tok, _, _, _ = O.dspark_greedy(base, np.array([0]), w1, w2, np.zeros((d + r, 1)), np.zeros(1),
                                   np.zeros((B, G, d)))
    assert tok[0, 0] == 2 and tok[0, 1] == 0     # step 1: all scores equal -> 0


def test_confidence_closed_forms():
    """conf_k = sigmoid([block_k; w1[previous]] conf.w + conf.b): with conf.w
    zero it is sigmoid(conf.b); with weight only on e1 coordinate j and
    one-hot e1 it is sigmoid(w_j + b) for previous tokens in class j; with
    weight only on block coordinate c it is sigmoid(block_k[c] w_c + b)."""
    B, G, V, r, d = 2, 5, 40, 8, 6
    base, w1, w2, succ = _planted_chain(B, G, V, r)
    anchors = np.array([3, 12])
    rng = np.random.default_rng(4)
    block = rng.standard_normal((B, G, d))
    b0 = 0.3
    _, conf, _, _ = O.dspark_greedy(base, anchors, w1, w2, np.zeros((d + r, 1)), np.array([b0]), block)
    assert np.allclose(conf, 1.0 / (1.0 + math.exp(-b0)), rtol=0, atol=1e-15)
    cw = np.zeros((d + r, 1))
    cw[d + 5, 0] = 2.0
    tok, conf, _, _ = O.dspark_greedy(base, anchors, w1, w2, cw, np.array([b0]), block)
    prev = np.concatenate([anchors[:, None], tok[:, :-1]], axis=1)     # the token each step conditions on
    want = np.where(prev % r == 5, 1.0 / (1.0 + math.exp(-(2.0 + b0))), 1.0 / (1.0 + math.exp(-b0)))
    assert np.allclose(conf, want, rtol=0, atol=1e-15)
    cw = np.zeros((d + r, 1))
    cw[2, 0] = -1.5
    _, conf, _, _ = O.dspark_greedy(base, anchors, w1, w2, cw, np.array([b0]), block)
    assert np.allclose(conf, 1.0 / (1.0 + np.exp(-(block[:, :, 2] * -1.5 + b0))), rtol=0, atol=1e-15)


def test_alg1_pruning_cuts_at_the_first_low_confidence_step():
    """Alg 1: position 0 is always kept; the first step k >= 1 whose confidence
    is below thresholds[k] (or min_conf) cuts the row to length k, and a later
    confident step does not undo the cut; without thresholds nothing is cut."""
    B, G, V, r, d = 4, 6, 40, 8, 6
    base, w1, w2, succ = _planted_chain(B, G, V, r)
    anchors = np.array([1, 2, 3, 4])
    block = np.zeros((B, G, d))
    # confidence by step through the block rows: conf_k = sigmoid(block[b, k, 0])
    cw = np.zeros((d + r, 1))
    cw[0, 0] = 1.0
    logit = np.array([[5, 5, 5, 5, 5, 5],
                      [5, -5, 5, 5, 5, 5],       # cut at 1
                      [-5, 5, 5, -5, 5, -5],     # position 0 is kept whatever its confidence; cut at 3
                      [5, 5, 5, 5, 5, -5]], float)   # cut at the last step
    block[:, :, 0] = logit
    run = lambda **kw: O.dspark_greedy(base, anchors, w1, w2, cw, np.zeros(1), block, **kw)
    _, conf, lengths, _ = run(min_conf=0.5)
    assert list(lengths) == [6, 1, 3, 5]
    _, _, lengths, _ = run()
    assert list(lengths) == [6, 6, 6, 6]
    _, _, lengths, _ = run(thresholds=[2.0] * G)       # every step below: cut at 1, never at 0
    assert list(lengths) == [1, 1, 1, 1]
    thr = [0.0, 0.0, 0.0, 0.999, 0.0, 0.0]            # per-step thresholds: only step 3 can cut
    _, _, lengths, _ = run(thresholds=thr)
    assert list(lengths) == [3, 3, 3, 3]
    tok_all, _, _, _ = run()
    tok_cut, _, _, _ = run(min_conf=0.5)
    assert np.array_equal(tok_all, tok_cut)           # pruning changes the lengths, never the tokens


@pytest.mark.parametrize("G", [1, 4, 7])
def test_verify_with_lengths_exhaustive(G):
    """A pruned block of length l proposes only its first l drafts: accepted
    is the agreeing prefix capped at l, committed = accepted + 1."""
    rng = np.random.default_rng(13)
    V = 50
    for bits in range(2 ** G):
        pattern = [(bits >> k) & 1 == 1 for k in range(G)]
        prefix = next((k for k in range(G) if not pattern[k]), G)
        T, draft, t = _planted_verify_inputs(G, V, pattern, rng)
        for l in range(1, G + 1):
            acc, com, ids, nxt = O.verify_greedy(T, draft, lengths=np.array([l]))
            assert acc[0] == min(prefix, l) and com[0] == acc[0] + 1
            assert nxt[0] == t[acc[0]] and list(ids[0, :acc[0] + 1]) == list(t[:acc[0] + 1])
