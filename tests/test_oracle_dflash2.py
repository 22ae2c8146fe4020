"""Pins for the oracle's DFlash2 variant (page "Inco Hacks Native: DFlash 2
Speculation": section 1, a sliding-window drafter; section 3, the target
verifies the block): rotary positions, the context window and verification
from the target's hidden states.

The pages fix neither the window nor the rotation, so what the variant
computes is this library's reading (rotate-half pairs, angle position *
theta^(-2i/hd), context row t at position t, block row k at len + k, the
last `window` context keys). These tests pin the oracle to that reading by
hand-computed values, the algebra of rotations (norms, composition, relative
position) and reductions to the plain drafter; the reading itself is
"parity unpinned" against the pages.
"""

import math

import numpy as np
import pytest

from oracle import dflash_oracle as O
from synth import gen, TINY, scaled

D2 = scaled(TINY, name="d2_pin", window=20, rope_theta=1e4)


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(1e-300, np.max(np.abs(b))))


# ----------------------------------------------------------------------------
# rotary positions


def test_rope_hand_values():
    # one pair (hd 2, frequency theta^0 = 1): [1, 0] at position 1 is [cos 1, sin 1]
    x = np.array([[[1.0, 0.0]]])
    assert np.allclose(O.rope(x, [1], 1e4), [[[math.cos(1.0), math.sin(1.0)]]], rtol=0, atol=1e-15)
    # [0, 1] turns the other way round: [-sin p, cos p]
    assert np.allclose(O.rope(np.array([[[0.0, 1.0]]]), [2], 1e4), [[[-math.sin(2.0), math.cos(2.0)]]], atol=1e-15)
    # hd 4: pair 1 (dims 1 and 3) turns at theta^(-2/4) = 0.1 for theta 100; position 10 -> angle 1
    y = O.rope(np.array([[[0.0, 1.0, 0.0, 0.0]]]), [10], 100.0)
    assert np.allclose(y, [[[0.0, math.cos(1.0), 0.0, math.sin(1.0)]]], atol=1e-15)
    # pair 0 of the same row turns at frequency 1: angle 10
    y = O.rope(np.array([[[1.0, 0.0, 0.0, 0.0]]]), [10], 100.0)
    assert np.allclose(y, [[[math.cos(10.0), 0.0, math.sin(10.0), 0.0]]], atol=1e-15)


def test_rope_identities():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 3, 64))
    pos = rng.integers(0, 20000, 6)
    # no rotation at position 0 and without a base
    assert np.array_equal(O.rope(x, np.zeros(6, int), 1e6), x)
    assert O.rope(x, pos, 0.0) is x
    y = O.rope(x, pos, 1e6)
    # each pair keeps its length
    n0 = x[..., :32] ** 2 + x[..., 32:] ** 2
    n1 = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert rel(n1, n0) < 1e-13
    # turns compose: p1 then p2 is p1 + p2
    p2 = rng.integers(0, 20000, 6)
    assert rel(O.rope(y, p2, 1e6), O.rope(x, pos + p2, 1e6)) < 1e-11


def test_rope_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((1, 1, 128)), rng.standard_normal((1, 1, 128))
    base = float(np.sum(O.rope(q, [700], 1e6) * O.rope(k, [300], 1e6)))
    for s in (1, 77, 4096, 100000):
        sh = float(np.sum(O.rope(q, [700 + s], 1e6) * O.rope(k, [300 + s], 1e6)))
        assert abs(sh - base) <= 1e-10 * max(1.0, abs(base))
    # and does depend on it
    other = float(np.sum(O.rope(q, [701], 1e6) * O.rope(k, [300], 1e6)))
    assert abs(other - base) > 1e-6


# ----------------------------------------------------------------------------
# a layer with rotary positions and a window


def _ctx_from(d, w, H_list, shift=0):
    """Context of the given H_ctx rows, keys turned at positions shift + t."""
    ctx = O.Context(d.nl, len(H_list), d.hkv, d.hd)
    for b, Hc in enumerate(H_list):
        for i in range(d.nl):
            K, V = O.context_kv(Hc, w[f"bb.{i}.attn_norm"], w[f"bb.{i}.k"], w[f"bb.{i}.v"], d.hkv, d.hd, d.eps,
                                False, positions=shift + np.arange(Hc.shape[0]), theta=d.rope_theta)
            ctx.append(i, b, K, V)
    return ctx


def _setup(d, lengths, seed=3):
    w = gen.Model(d, gains="random").materialise()
    rng = np.random.default_rng(seed)
    Hs = [rng.standard_normal((L, d.d)) for L in lengths]
    H_d = rng.standard_normal((len(lengths), d.gamma, d.d))
    return w, Hs, H_d


def test_layer_is_invariant_to_a_common_position_shift():
    d = scaled(D2, window=0)
    w, Hs, H_d = _setup(d, [32, 9])
    ref = O.draft_layer(H_d, _ctx_from(d, w, Hs), 0, w, d, False)
    for s in (1, 1000, 50000):
        ctx = _ctx_from(d, w, Hs, shift=s)
        out = O.draft_layer(H_d, ctx, 0, w, d, False, start=[32 + s, 9 + s])
        assert rel(out, ref) < 1e-10, s
    # a block that moves against its context changes the layer (the test can fail)
    out = O.draft_layer(H_d, _ctx_from(d, w, Hs), 0, w, d, False, start=[33, 10])
    assert rel(out, ref) > 1e-6


def test_rotation_reaches_the_scores():
    d = scaled(D2, window=0)
    w, Hs, H_d = _setup(d, [32])
    plain = scaled(d, rope_theta=0.0)
    a = O.draft_layer(H_d, _ctx_from(d, w, Hs), 0, w, d, False)
    b = O.draft_layer(H_d, _ctx_from(plain, w, Hs), 0, w, plain, False)
    assert rel(a, b) > 1e-4


def test_window_keeps_the_last_keys():
    d = D2                                        # window 20
    w, Hs, H_d = _setup(d, [32, 9, 20])
    full = _ctx_from(d, w, Hs)
    out = O.draft_layer(H_d, full, 0, w, d, False)
    # the same as the whole-context layer over only the last 20 rows (keys keep their
    # positions; the block stays at len + k)
    cut = O.Context(d.nl, 3, d.hkv, d.hd)
    for i in range(d.nl):
        for b in range(3):
            cut.append(i, b, full.k[i][b][-20:], full.v[i][b][-20:])
    ref = O.draft_layer(H_d, cut, 0, w, scaled(d, window=0), False, start=[32, 9, 20])
    assert rel(out, ref) < 1e-13
    # windows at or past the context length change nothing; a shorter one does
    for win in (32, 33, 10 ** 6):
        assert rel(O.draft_layer(H_d, full, 0, w, scaled(d, window=win), False),
                   O.draft_layer(H_d, full, 0, w, scaled(d, window=0), False)) < 1e-13
    assert rel(out, O.draft_layer(H_d, full, 0, w, scaled(d, window=0), False)) > 1e-6


def test_window_one_attends_the_last_row_and_the_block():
    d = scaled(D2, window=1, rope_theta=0.0)
    w, Hs, H_d = _setup(d, [12])
    full = _ctx_from(d, w, Hs)
    ctx1 = O.Context(d.nl, 1, d.hkv, d.hd)
    for i in range(d.nl):
        ctx1.append(i, 0, full.k[i][0][-1:], full.v[i][0][-1:])
    assert rel(O.draft_layer(H_d, full, 0, w, d, False),
               O.draft_layer(H_d, ctx1, 0, w, scaled(d, window=0), False)) < 1e-13


def test_append_turns_new_keys_at_their_positions():
    # appending in two pieces gives the keys of one append (positions continue)
    d = D2
    w, Hs, _ = _setup(d, [32])
    one = O.Context(d.nl, 1, d.hkv, d.hd)
    O.append_context(one, w, d, Hs[0], [list(range(32))], [32], False)
    two = O.Context(d.nl, 1, d.hkv, d.hd)
    O.append_context(two, w, d, Hs[0][:13], [list(range(13))], [13], False)
    O.append_context(two, w, d, Hs[0][13:], [list(range(19))], [19], False)
    for i in range(d.nl):
        assert rel(two.k[i][0], one.k[i][0]) < 1e-13
        assert rel(two.v[i][0], one.v[i][0]) < 1e-13
    # and the keys are the rotated ones (row t at position t)
    K, _ = O.context_kv(Hs[0], w["bb.0.attn_norm"], w["bb.0.k"], w["bb.0.v"], d.hkv, d.hd, d.eps, False)
    assert rel(one.k[0][0], O.rope(K, np.arange(32), d.rope_theta)) < 1e-13


# ----------------------------------------------------------------------------
# verification from the target's hidden states


def plant_hidden(E_out, tokens, scale=4.0):
    """Hidden rows along the planted tokens' head rows: each row's greedy token
    is its planted one (its logit is scale * |E_t|, every other logit at most
    scale * |E_v| * cos, far smaller for random head rows)."""
    E = O.dense(E_out)
    rows = E[tokens.reshape(-1)]
    h = scale * rows / np.linalg.norm(rows, axis=1, keepdims=True)
    return h.reshape(tokens.shape + (E.shape[1],))


@pytest.mark.parametrize("wdtype", ["f32", "bf16", "int4g64"])
def test_verify_from_hidden_realises_planted_schedules(wdtype):
    G = 7
    d = scaled(TINY, wdtype=wdtype, gamma=G, V=700, H=256)
    E_out = gen.make_weight(d, "E_out", seed=5)
    rng = np.random.default_rng(2)
    B = G + 1
    t = rng.integers(0, d.V, size=(B, G + 1))
    accept = np.arange(B) % (G + 1)               # every accept length once
    draft = t[:, :G].copy()
    for b in range(B):
        if accept[b] < G:
            draft[b, accept[b]] = (t[b, accept[b]] + 1) % d.V
    hidden = plant_hidden(E_out, t)
    logits = hidden @ O.dense(E_out).T
    s = np.sort(logits, axis=-1)
    assert np.min(s[..., -1] - s[..., -2]) > 0.1     # every target token decided
    acc, com, ids, nxt = O.verify_from_hidden(hidden, E_out, draft.astype(np.int32))
    assert np.array_equal(acc, accept)
    assert np.array_equal(com, accept + 1)
    assert np.array_equal(nxt, t[np.arange(B), accept])
    for b in range(B):
        assert list(ids[b, :accept[b] + 1]) == list(t[b, :accept[b] + 1])
        assert np.all(ids[b, accept[b] + 1:] == -1)
    # a length cap stops the prefix there
    lens = np.full(B, 2, np.int32)
    acc2, _, _, _ = O.verify_from_hidden(hidden, E_out, draft.astype(np.int32), lengths=lens)
    assert np.array_equal(acc2, np.minimum(accept, 2))
