"""CPU oracle for the DFlash KV-injection block drafter.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the library's
product path never does, and it shares no code with the HIP kernels.

Plain numpy in float64, written from the pages' definition of the method:

  * Eq 2 (page "@mlx-bun/inference 0.0.0-stage -> 1.0.0", dflash.ts header and
    #buildContext): H_ctx = RMSNorm(W_c [H^l1; ...; H^lm]) over every context
    row, the m tapped target hidden states concatenated on the feature axis.
  * Eq 3 (same page, #layer and projectContextRows): every draft layer i
    normalises BOTH the block and the context with its own attn_norm, forms
    Q = W_Q n_block, K = [W_K n_ctx ; W_K n_block], V likewise, and runs
    attention of the block rows over [context ++ block] with no mask (the
    block is bidirectional; is_causal is false, page "A Refusal Is Not A
    Failure", section "What the port taught, besides that"). The context is
    read-only memory re-projected by each layer; it is never updated.
  * #buildBlock: row 0 of the block is the anchor's embedding (borrowed from
    the target) through tok_proj plus block_pos[0]; rows k >= 1 are
    mask_emb[k-1] + block_pos[k].
  * #layer FFN: H += (act(n2 W_gate) * (n2 W_up)) W_down with n2 = RMSNorm(H;
    ff_norm); the residual adds follow the attention output projection and
    the FFN.
  * #backbone / #baseLogits: Y = RMSNorm(H; out_norm) W_out, cast to the
    embedding dtype, scored by the borrowed target LM head; forwardRows takes
    the greedy argmax of each row (row k proposes the (k+1)-th token after
    the anchor).
  * #markov, #confidence and the greedy loop of forwardRows (page 3): the
    DSpark sequential head adds w1[previous token] w2 to each block row's base
    logits before the argmax, one row after the other; the confidence head is
    sigmoid([block row; w1[previous]] conf.w + conf.b), and Alg 1 cuts a row's
    draft where it falls below the step's threshold.
  * Greedy verification (page "Inco Hacks Native: DFlash 2 Speculation",
    section 3, log lines "accepted=7 committed=8" and "accepted=5
    committed=6" for block 8): accepted = longest prefix of drafts equal to
    the target's argmax, committed = accepted + 1.

  * The DFlash2 variant (page "Inco Hacks Native: DFlash 2 Speculation",
    section 1: a sliding-window drafter; section 3: the target verifies the
    block): rotary positions on Q and K, attention over only the last
    `window` context keys, and verification that scores the target's own
    hidden states with the borrowed LM head instead of given logits.

Readings where the pages are silent (each listed in the design notes):
  RMSNorm is x * (mean(x^2) + eps)^-1/2 * g with eps = 1e-6; attention scale
  is hd^-1/2, with no positional rotation unless the variant's rope_theta is
  set; query head h reads kv head
  h // (hq / hkv); argmax ties resolve to the lowest index; the FFN
  activation is the tanh-form GELU or SiLU per the workload; the rows
  appended to the context each round are the `committed` verified rows.
  DFlash2 variant (the pages give neither the window nor the rotation): the
  rotation pairs dims i and i + hd/2 of a head (the rotate-half layout of
  the Qwen family the drafter pairs with) at the angle position *
  rope_theta^(-2i/hd); context row t sits at position t and block row k at
  position len + k (the block continues the context: row 0 holds the
  anchor, the token after the last retained row); the window keeps the last
  `window` context keys for every block row (0 = the whole context); the
  verify hidden states are the target's final hidden rows, already normed,
  that the borrowed LM head scores.

Modes:
  pure      float64 throughout (the fp32 workloads are compared to this).
  faithful  float64, but rounded to bfloat16 (nearest-even) at the points
            the GPU contract rounds: every input of a weight product (the
            normalised block, context and FFN inputs, the attention output,
            the FFN product, the out-norm output), the Q/K/V projections, the
            context K/V cache and the out-projection result Y; with rotary
            positions, Q and K are rounded once more after their rotation.

Weights are in the synthetic generator's storage formats: float32 arrays,
uint16 bfloat16 bit patterns, or 4-bit groups dict(codes, scales, biases)
with w = scale * q + bias, groups of 64 along the reduction axis, 8 codes
per uint32 low nibble first. Matrices are [out, in]; a product is x @ W.T.
"""

import math

import numpy as np

GROUP = 64


# ----------------------------------------------------------------------------
# number formats


def bf16(x):
    """Round float64 values to bfloat16 precision (8 significant bits),
    nearest with ties to even, returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                      # x = mant * 2^expo, 0.5 <= |mant| < 1
    return np.ldexp(np.rint(mant * 256.0), expo - 8)


def decode_bf16(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dequant_int4(w, rows=None):
    """4-bit groups -> float64 [N, K] (optionally only the given rows):
    element k of a row is scale[k // 64] * q_k + bias[k // 64], where q_k is
    nibble k % 8 (lowest first) of code word k // 8."""
    codes, scales, biases = w["codes"], w["scales"], w["biases"]
    if rows is not None:
        codes, scales, biases = codes[rows], scales[rows], biases[rows]
    N, K8 = codes.shape
    # little-endian bytes of a code word: byte j holds nibbles 2j (low) and 2j + 1 (high)
    by = np.ascontiguousarray(codes, dtype="<u4").view(np.uint8).reshape(N, K8 * 4)
    q = np.empty((N, K8 * 4, 2), dtype=np.uint8)
    q[:, :, 0] = by & 15
    q[:, :, 1] = by >> 4
    q = q.reshape(N, K8 * 8 // GROUP, GROUP).astype(np.float64)
    s = decode_bf16(scales)[:, :, None]
    b = decode_bf16(biases)[:, :, None]
    return (s * q + b).reshape(N, K8 * 8)


# Whole-matrix decodes are kept (read-only) for the stored arrays they came
# from, so repeated forwards over one model decode each weight once. Stored
# weights are treated as immutable: a changed weight is a new array.
_DENSE_LIMIT = 8 << 30
_dense_memo = {}
_dense_bytes = [0]


def _decode(w, rows):
    if isinstance(w, dict):
        return dequant_int4(w, rows)
    w = np.asarray(w)
    if rows is not None:
        w = w[rows]
    if w.dtype == np.uint16:
        return decode_bf16(w)
    return w.astype(np.float64)


def dense(w, rows=None):
    """Any stored weight -> float64 array (whole matrices: a read-only view
    shared between calls)."""
    if rows is not None:
        return _decode(w, rows)
    hit = _dense_memo.get(id(w))
    if hit is not None and hit[0] is w:
        return hit[1]
    a = _decode(w, None)
    a.setflags(write=False)
    if _dense_bytes[0] + a.nbytes > _DENSE_LIMIT:
        _dense_memo.clear()
        _dense_bytes[0] = 0
    _dense_memo[id(w)] = (w, a)
    _dense_bytes[0] += a.nbytes
    return a


def n_rows(w):
    return w["codes"].shape[0] if isinstance(w, dict) else np.asarray(w).shape[0]


# ----------------------------------------------------------------------------
# elementwise pieces


def rmsnorm(x, g, eps):
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis (page 3, the
    rmsNorm calls in #buildContext, #layer and #backbone)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def gelu_tanh(x):
    """Tanh-form GELU, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def silu(x):
    return x / (1.0 + np.exp(-x))


ACTS = {"gelu_tanh": gelu_tanh, "silu": silu}


def _r(x, faithful):
    return bf16(x) if faithful else x


def softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# Eq 2: context projection


def context_project(taps, W_c, g_ctx, eps):
    """taps: m arrays [n, H] -> H_ctx [n, d] (page 3, #buildContext, Eq 2)."""
    X = np.concatenate([dense(t) for t in taps], axis=1)
    P = X @ dense(W_c).T
    return rmsnorm(P, dense(g_ctx), eps)


# ----------------------------------------------------------------------------
# Eq 3, context half: per-layer K/V of the context


def rope_inv_freq(hd, theta):
    """Angular frequency of each rotated pair: theta^(-2i/hd), i < hd/2."""
    return float(theta) ** (-2.0 * np.arange(hd // 2) / hd)


def rope(x, positions, theta):
    """Rotary positions (DFlash2 variant; the pairing is this library's
    reading): x [n, heads, hd] at positions [n]; dims i and i + hd/2 of each
    head turn by the angle position * theta^(-2i/hd). theta 0: no rotation."""
    if not theta:
        return x
    hd = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(hd, theta)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., : hd // 2], x[..., hd // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def context_kv(H_ctx, g_attn, W_k, W_v, hkv, hd, eps, faithful, positions=None, theta=0.0):
    """One layer's context keys/values [n, hkv, hd] (page 3,
    projectContextRows: the layer's own attn_norm, then its own W_K, W_V);
    with rotary positions, each key turned at its row's position."""
    n = _r(rmsnorm(H_ctx, dense(g_attn), eps), faithful)
    K = _r(n @ dense(W_k).T, faithful)
    V = _r(n @ dense(W_v).T, faithful)
    rows = H_ctx.shape[0]
    K = K.reshape(rows, hkv, hd)
    if theta:
        K = _r(rope(K, positions, theta), faithful)
    return K, V.reshape(rows, hkv, hd)


class Context:
    """Retained per-layer context K/V of B sequences (page 3: the context
    projection is independent of the block and is retained across rounds)."""

    def __init__(self, nl, B, hkv, hd):
        self.k = [[np.zeros((0, hkv, hd)) for _ in range(B)] for _ in range(nl)]
        self.v = [[np.zeros((0, hkv, hd)) for _ in range(B)] for _ in range(nl)]

    def length(self, b):
        return self.k[0][b].shape[0]

    def append(self, layer, b, K, V):
        self.k[layer][b] = np.concatenate([self.k[layer][b], K], axis=0)
        self.v[layer][b] = np.concatenate([self.v[layer][b], V], axis=0)

    def truncate(self, b, length):
        for i in range(len(self.k)):
            self.k[i][b] = self.k[i][b][:length]
            self.v[i][b] = self.v[i][b][:length]


def append_context(ctx, weights, dims, H_ctx, seq_rows, counts, faithful):
    """Append rows of H_ctx to the retained context. seq_rows[b] is the list
    of H_ctx row indices proposed for sequence b; only the first counts[b]
    of them are appended (the verified ones)."""
    for i in range(dims.nl):
        for b, rows in enumerate(seq_rows):
            take = list(rows)[: int(counts[b])]
            if not take:
                continue
            theta = getattr(dims, "rope_theta", 0.0)
            rot = {"positions": ctx.k[i][b].shape[0] + np.arange(len(take)), "theta": theta} if theta else {}
            K, V = context_kv(H_ctx[take], weights[f"bb.{i}.attn_norm"], weights[f"bb.{i}.k"],
                              weights[f"bb.{i}.v"], dims.hkv, dims.hd, dims.eps, faithful, **rot)
            ctx.append(i, b, K, V)


# ----------------------------------------------------------------------------
# the block


def block_init(anchor_ids, E_in, W_tok, mask_emb, block_pos, gamma, faithful):
    """H_d [B, gamma, d] (page 3, #buildBlock; the embedding is the target's)."""
    e = _r(dense(E_in, rows=np.asarray(anchor_ids, dtype=np.int64)), faithful)   # [B, H]
    P = dense(block_pos)
    B = e.shape[0]
    H = np.empty((B, gamma, P.shape[1]))
    H[:, 0] = e @ dense(W_tok).T + P[0]
    if gamma > 1:
        H[:, 1:] = dense(mask_emb) + P[1:]
    return H


def attention(Q, K, V, scale):
    """Non-causal attention. Q [R, hq, hd]; K, V [Lk, hkv, hd] -> [R, hq, hd].
    Query head h reads key/value head h // (hq // hkv)."""
    R, hq, hd = Q.shape
    hkv = K.shape[1]
    group = hq // hkv
    O = np.empty_like(Q)
    for h in range(hq):
        g = h // group
        S = scale * (Q[:, h] @ K[:, g].T)
        O[:, h] = softmax_rows(S) @ V[:, g]
    return O


def draft_layer(H_d, ctx, layer, weights, dims, faithful, attn=attention, start=None):
    """One KV-injection layer over all sequences (page 3, #layer, Eq 3).
    H_d [B, gamma, d] -> new H_d. ctx.k[layer][b] is read, never written.
    DFlash2 variant: block row k of sequence b sits at position start[b] + k
    (start defaults to the retained context's length) and only the last
    dims.window context keys are attended (0: all)."""
    B, G, d = H_d.shape
    hq, hkv, hd = dims.hq, dims.hkv, dims.hd
    w = lambda n: weights[f"bb.{layer}.{n}"]
    Wq, Wk, Wv, Wo = dense(w("q")), dense(w("k")), dense(w("v")), dense(w("o"))
    Wg, Wu, Wd = dense(w("gate")), dense(w("up")), dense(w("down"))
    g_attn, g_ffn = dense(w("attn_norm")), dense(w("ff_norm"))
    act = ACTS[dims.act]
    theta, window = getattr(dims, "rope_theta", 0.0), getattr(dims, "window", 0)
    out = np.empty_like(H_d)
    for b in range(B):
        x = H_d[b]
        n = _r(rmsnorm(x, g_attn, dims.eps), faithful)
        Q = _r(n @ Wq.T, faithful).reshape(G, hq, hd)
        Kb = _r(n @ Wk.T, faithful).reshape(G, hkv, hd)
        Vb = _r(n @ Wv.T, faithful).reshape(G, hkv, hd)
        Kc, Vc = ctx.k[layer][b], ctx.v[layer][b]
        if theta:
            pos = (Kc.shape[0] if start is None else int(start[b])) + np.arange(G)
            Q, Kb = _r(rope(Q, pos, theta), faithful), _r(rope(Kb, pos, theta), faithful)
        if window > 0:
            Kc, Vc = Kc[max(0, Kc.shape[0] - window):], Vc[max(0, Vc.shape[0] - window):]
        K = np.concatenate([Kc, Kb], axis=0)
        V = np.concatenate([Vc, Vb], axis=0)
        O = _r(attn(Q, K, V, hd ** -0.5).reshape(G, hq * hd), faithful)
        x = x + O @ Wo.T
        n2 = _r(rmsnorm(x, g_ffn, dims.eps), faithful)
        A = _r(act(n2 @ Wg.T) * (n2 @ Wu.T), faithful)
        out[b] = x + A @ Wd.T
    return out


def out_project(H_d, g_out, W_out, eps, faithful):
    """Y = RMSNorm(H_d; out_norm) W_out, cast to the embedding dtype
    (page 3, #backbone then #baseLogits)."""
    y = _r(rmsnorm(H_d, dense(g_out), eps), faithful)
    return _r(y @ dense(W_out).T, faithful)


# ----------------------------------------------------------------------------
# LM head and argmax


def lm_head_argmax(Y, E_out, chunk=16384, want_logits=False):
    """Greedy ids of Y [M, H] under the borrowed head E_out [V, H]:
    argmax_v Y . E_out[v], lowest index among equal maxima.
    Returns (ids [M], max logit [M], logits [M, V] or None)."""
    Y = np.asarray(Y, dtype=np.float64)
    M = Y.shape[0]
    V = n_rows(E_out)
    best = np.full(M, -np.inf)
    arg = np.zeros(M, dtype=np.int64)
    logits = np.empty((M, V)) if want_logits else None
    for v0 in range(0, V, chunk):
        rows = np.arange(v0, min(V, v0 + chunk))
        s = Y @ dense(E_out, rows=rows).T
        if want_logits:
            logits[:, rows] = s
        j = np.argmax(s, axis=1)              # first (lowest) index of the chunk's maximum
        val = s[np.arange(M), j]
        better = val > best                   # strictly greater: an earlier chunk keeps ties
        best = np.where(better, val, best)
        arg = np.where(better, v0 + j, arg)
    return arg.astype(np.int32), best, logits


def argmax_lowest(x):
    """Row argmax with ties to the lowest index."""
    return np.argmax(np.asarray(x), axis=-1).astype(np.int32)


# ----------------------------------------------------------------------------
# greedy verification


def verify_greedy(target_logits, draft_ids, lengths=None):
    """target_logits [B, gamma+1, V], draft_ids [B, gamma] ->
    accepted [B], committed [B], ids [B, gamma+1] (-1 padded), next anchor [B].

    t[b, j] is the target's greedy token at verify row j; draft k is checked
    against row k; accepted is the longest agreeing prefix; the committed
    tokens are t[b, 0..accepted] (the verified drafts plus the target's own
    next token), so committed = accepted + 1, and t[b, accepted] is the next
    anchor. With lengths [B] (a confidence-pruned block, page 3's Alg 1: only
    the first lengths[b] drafts are proposed) the prefix stops there too."""
    t = argmax_lowest(target_logits)
    B, G = draft_ids.shape
    accepted = np.zeros(B, dtype=np.int32)
    for b in range(B):
        limit = G if lengths is None else int(lengths[b])
        a = 0
        while a < limit and int(draft_ids[b, a]) == int(t[b, a]):
            a += 1
        accepted[b] = a
    committed = accepted + 1
    ids = np.full((B, G + 1), -1, dtype=np.int32)
    for b in range(B):
        ids[b, : committed[b]] = t[b, : committed[b]]
    nxt = t[np.arange(B), accepted].astype(np.int32)
    return accepted, committed.astype(np.int32), ids, nxt


def verify_from_hidden(target_hidden, E_out, draft_ids, lengths=None):
    """Greedy verification from the target's own hidden states (DFlash2
    variant: the target verifies the block, page "Inco Hacks Native: DFlash 2
    Speculation", section 3): target_hidden [B, gamma+1, H] are the target's
    final hidden rows at the verify positions; the borrowed LM head scores
    them (logits = hidden E_out^T) and the greedy rule above decides."""
    B, W, H = target_hidden.shape
    _, _, logits = lm_head_argmax(target_hidden.reshape(B * W, H), E_out, want_logits=True)
    return verify_greedy(logits.reshape(B, W, -1), draft_ids, lengths)


# ----------------------------------------------------------------------------
# DSpark sequential head, confidence head and confidence-scheduled pruning


def block_rows(H_d, g_out, eps, faithful):
    """The backbone's output rows, RMSNorm(H_d; out_norm) (page 3, #backbone:
    `block`); rounded to bf16 in faithful mode, where they are the out
    projection's input."""
    return _r(rmsnorm(H_d, dense(g_out), eps), faithful)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def dspark_greedy(base, anchors, w1, w2, conf_w, conf_b, block, thresholds=None, min_conf=None):
    """Greedy drafting with the Markov sequential head and the confidence head
    (page 3, #markov, #confidence and the greedy loop of forwardRows).

    base [B, gamma, V]: the base logits of the block rows (#baseLogits);
    anchors [B]; w1 = markov.w1 [V, r]; w2 = markov.w2 [r, V];
    conf_w = conf.w [d + r, 1]; conf_b = conf.b [1]; block [B, gamma, d].

    Step k = 0 .. gamma-1, starting from previous = the anchors:
      e1 = w1[previous]                                  [B, r]
      scores = base[:, k] + e1 w2                        [B, V]
      token_k = argmax(scores), lowest index on ties; previous = token_k
      conf_k = sigmoid([block[:, k]; e1] conf_w + conf_b)
    Pruning (Alg 1, pages' single-user form): for k >= 1, with threshold
    thresholds[k] (else min_conf), a row whose conf_k falls below it is cut to
    length k; the first cut of a row stands, and position 0 is always kept.
    The page stops the loop once every row is cut; the tokens of the kept
    positions do not depend on that, and here every step runs.

    Returns tokens [B, gamma], conf [B, gamma], lengths [B] and the scores
    [B, gamma, V] of every step."""
    base = np.asarray(base, dtype=np.float64)
    B, G, V = base.shape
    W1, W2 = dense(w1), dense(w2)
    cw = dense(conf_w).reshape(-1)
    cb = float(dense(conf_b).reshape(-1)[0])
    pruning = thresholds is not None or min_conf is not None
    previous = np.asarray(anchors, dtype=np.int64)
    tokens = np.zeros((B, G), dtype=np.int32)
    conf = np.zeros((B, G))
    scores = np.zeros((B, G, V))
    lengths = np.full(B, G, dtype=np.int32)
    cut = np.zeros(B, dtype=bool)
    for k in range(G):
        e1 = W1[previous]
        scores[:, k] = base[:, k] + e1 @ W2
        tok = argmax_lowest(scores[:, k])
        tokens[:, k] = tok
        joined = np.concatenate([np.asarray(block[:, k], dtype=np.float64), e1], axis=1)
        conf[:, k] = sigmoid(joined @ cw + cb)
        if pruning and k > 0:
            threshold = thresholds[k] if thresholds is not None else min_conf
            newly = (~cut) & (conf[:, k] < threshold)
            lengths[newly] = k
            cut |= newly
        previous = tok.astype(np.int64)
    return tokens, conf, lengths, scores


def dspark_forward(weights, dims, ctx, anchor_ids, faithful, thresholds=None, min_conf=None):
    """forwardRows with the DSpark heads over the retained context: the
    backbone (block init, every layer, out_norm), the base logits through the
    borrowed head, then dspark_greedy. Returns (tokens, conf, lengths, extra)
    with extra = {"block", "Y", "base", "scores"}."""
    H = block_init(anchor_ids, weights["E_in"], weights["tok_proj"], weights["mask_emb"],
                   weights["block_pos"], dims.gamma, faithful)
    for i in range(dims.nl):
        H = draft_layer(H, ctx, i, weights, dims, faithful)
    blk = block_rows(H, weights["out_norm"], dims.eps, faithful)
    Y = _r(blk @ dense(weights["out_proj"]).T, faithful)
    B, G = H.shape[0], dims.gamma
    _, _, logits = lm_head_argmax(Y.reshape(B * G, -1), weights["E_out"], want_logits=True)
    base = logits.reshape(B, G, -1)
    tokens, conf, lengths, scores = dspark_greedy(base, anchor_ids, weights["markov.w1"], weights["markov.w2"],
                                                  weights["conf.w"], weights["conf.b"], blk, thresholds, min_conf)
    return tokens, conf, lengths, {"block": blk, "Y": Y, "base": base, "scores": scores}


# ----------------------------------------------------------------------------
# composition


def draft_forward(weights, dims, ctx, anchor_ids, faithful, return_all=False, start=None):
    """Block init, every layer, out projection, LM head argmax (page 3,
    forwardRows with the retained context). Returns draft ids [B, gamma]
    (and the intermediates when return_all). start: the block's first
    position per sequence under rotary positions (default: context length)."""
    H = block_init(anchor_ids, weights["E_in"], weights["tok_proj"], weights["mask_emb"],
                   weights["block_pos"], dims.gamma, faithful)
    layers = [H]
    for i in range(dims.nl):
        H = draft_layer(H, ctx, i, weights, dims, faithful, start=start)
        layers.append(H)
    Y = out_project(H, weights["out_norm"], weights["out_proj"], dims.eps, faithful)
    B, G = H.shape[0], dims.gamma
    ids, best, logits = lm_head_argmax(Y.reshape(B * G, -1), weights["E_out"], want_logits=return_all)
    ids = ids.reshape(B, G)
    if return_all:
        return ids, {"H": layers, "Y": Y, "logits": logits, "max_logit": best.reshape(B, G)}
    return ids
