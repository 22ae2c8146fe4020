"""Seeded synthetic inputs for the DFlash block drafter.

This module only *constructs inputs*: drafter weights, tapped target hidden
states, anchor tokens, accept schedules and planted target logits. It holds
none of the drafter's arithmetic (no norm, projection, attention, argmax or
verification), so both the CPU oracle and the GPU path may consume what it
produces.

Random numbers come from SplitMix64 (S. Vigna's published generator: the state
advances by the golden-ratio increment 0x9E3779B97F4A7C15 and each output is
the state passed through the 30/27/31 xor-shift-multiply finaliser). A stream
is keyed by (seed, crc32(tensor name)); element k of a stream is the k-th
output from that key, so any slice of any tensor can be generated alone and
the values do not depend on chunking. Uniforms are (top-53-bits + 1) * 2^-53
in (0, 1]; normals are Box-Muller pairs (cos, sin) over consecutive uniforms.

Weight distributions follow the workload definition: every projection, the
mask embeddings, the block positions and both borrowed embedding tables are
N(0, 0.02); norm gains are 1.0 (the page-3 initialisation of dflash.ts) or,
for tests that must catch a dropped or shared norm, 1 + U(-0.5, 0.5). Taps are
N(0, 1). The 4-bit format draws codes uniformly from {0..15} with per-group
bf16 scale 0.02/sqrt(21.25)*(0.75+0.5u) and bias -7.5*scale (mean ~0,
std ~0.02), 64 codes per group along the reduction axis, 8 codes per uint32,
low nibble first.

Storage formats returned:
  "f32"      numpy float32 array
  "bf16"     numpy uint16 array of bfloat16 bit patterns
  "int4g64"  dict(codes=uint32 [N, K/8], scales=uint16 [N, K/64],
                  biases=uint16 [N, K/64])
Matrices are stored [out, in] (reduction axis contiguous).
"""

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Dims, GROUP, WDTYPE_F32, WDTYPE_BF16, WDTYPE_INT4G64

SEED_WEIGHTS = 0
SEED_TAPS = 1
SEED_ANCHORS = 2
SEED_LOGITS = 3
SEED_LENGTHS = 4

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_S30, _S27, _S31, _S11 = np.uint64(30), np.uint64(27), np.uint64(31), np.uint64(11)

_CHUNK = 1 << 18
_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _finalise(z):
    z ^= z >> _S30
    z *= _MIX1
    z ^= z >> _S27
    z *= _MIX2
    z ^= z >> _S31
    return z


def stream_key(seed: int, name: str) -> np.uint64:
    """Key of the stream for tensor `name` under `seed` (one SplitMix64 step)."""
    tid = zlib.crc32(name.encode("utf-8"))
    z = np.array([((seed & 0xFFFFFFFF) << 32) | tid], dtype=np.uint64)
    z += _GOLDEN
    return _finalise(z)[0]


def raw64(key: np.uint64, start: int, count: int) -> np.ndarray:
    """Outputs start..start+count-1 of the SplitMix64 sequence with state `key`."""
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    z = k * _GOLDEN
    z += key
    return _finalise(z)


def _uniform_from_raw(r: np.ndarray) -> np.ndarray:
    return ((r >> _S11).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)


def uniforms(key, start: int, count: int) -> np.ndarray:
    return _uniform_from_raw(raw64(key, start, count))


def _normals_serial(key, start: int, count: int) -> np.ndarray:
    p0 = start // 2
    p1 = (start + count + 1) // 2
    r = raw64(key, 2 * p0, 2 * (p1 - p0))
    u = _uniform_from_raw(r)
    u1, u2 = u[0::2], u[1::2]
    rad = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * (p1 - p0), dtype=np.float64)
    out[0::2] = rad * np.cos(th)
    out[1::2] = rad * np.sin(th)
    off = start - 2 * p0
    return out[off:off + count]


def _parallel(fn, count: int, dtype) -> np.ndarray:
    out = np.empty(count, dtype=dtype)
    if count <= _CHUNK:
        out[:] = fn(0, count)
        return out

    def work(s):
        n = min(_CHUNK, count - s)
        out[s:s + n] = fn(s, n)

    with ThreadPoolExecutor(_WORKERS) as ex:
        list(ex.map(work, range(0, count, _CHUNK)))
    return out


def normals(seed: int, name: str, count: int, start: int = 0) -> np.ndarray:
    key = stream_key(seed, name)
    return _parallel(lambda s, n: _normals_serial(key, start + s, n), count, np.float64)


def _stored_chunk(kind, seed, name, std, fp32, start, s, n):
    key = stream_key(seed, name)
    if kind == "codes":
        return (raw64(key, start + s, n) >> np.uint64(60)).astype(np.uint8)
    x = (_normals_serial(key, start + s, n) * std).astype(np.float32)
    return x if fp32 else f32_to_bf16_bits(x)


def _generate(kind, seed, name, std, fp32, start, count, dtype):
    return _parallel(lambda s, n: _stored_chunk(kind, seed, name, std, fp32, start, s, n), count, dtype)


def scaled_normals_stored(seed: int, name: str, count: int, std: float, fp32: bool, start: int = 0):
    """std * N(0,1) in the storage type (float32, or bf16 bits), chunk by chunk
    so that no full-size float64 temporary is ever allocated."""
    return _generate("normal", seed, name, std, fp32, start, count, np.float32 if fp32 else np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# weights


def weight_names(dims: Dims):
    names = []
    for i in range(dims.nl):
        names += [f"bb.{i}.{w}" for w in ("attn_norm", "q", "k", "v", "o", "ff_norm", "gate", "up", "down")]
    names += ["W_c", "ctx_norm", "tok_proj", "mask_emb", "block_pos", "out_norm", "out_proj", "E_in", "E_out"]
    if dims.r > 0:
        names += HEAD_NAMES
    return names


# the DSpark sequential head and confidence head (page 3 names and shapes: markov.w1 [V, r],
# markov.w2 [r, V], conf.w [d + r, 1], conf.b [1]); stored bf16 (f32 for f32 models), never 4-bit
HEAD_NAMES = ["markov.w1", "markov.w2", "conf.w", "conf.b"]


def weight_shape(dims: Dims, name: str):
    d, H, F = dims.d, dims.H, dims.F
    head = {"markov.w1": (dims.V, dims.r), "markov.w2": (dims.r, dims.V), "conf.w": (d + dims.r, 1),
            "conf.b": (1,)}
    if name in head:
        return head[name]
    qw, kw = dims.hq * dims.hd, dims.kv_width
    leaf = name.split(".")[-1]
    table = {
        "attn_norm": (d,), "ff_norm": (d,), "ctx_norm": (d,), "out_norm": (d,),
        "q": (qw, d), "k": (kw, d), "v": (kw, d), "o": (d, qw),
        "gate": (F, d), "up": (F, d), "down": (d, F),
        "W_c": (d, dims.m * H), "tok_proj": (d, H), "out_proj": (H, d),
        "mask_emb": (max(dims.gamma - 1, 0), d), "block_pos": (dims.gamma, d),
        "E_in": (dims.V, H), "E_out": (dims.V, H),
    }
    return table[leaf]


def is_gain(name: str) -> bool:
    return name.split(".")[-1] in ("attn_norm", "ff_norm", "ctx_norm", "out_norm")


def is_matrix(name: str) -> bool:
    return name.split(".")[-1] in ("q", "k", "v", "o", "gate", "up", "down", "W_c", "tok_proj",
                                   "out_proj", "E_in", "E_out")


def _store_dense(x64: np.ndarray, fp32: bool) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if fp32 else f32_to_bf16_bits(x32)


def _int4_matrix(seed: int, name: str, shape):
    N, K = shape
    assert K % GROUP == 0, f"{name}: reduction width {K} is not a multiple of {GROUP}"
    count = N * K
    q = _generate("codes", seed, name + "#codes", 0.0, False, 0, count, np.uint8)
    q = q.reshape(N, K // 8, 8).astype(np.uint32)
    packed = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        packed |= q[:, :, j] << np.uint32(4 * j)
    ng = N * (K // GROUP)
    u = uniforms(stream_key(seed, name + "#scale"), 0, ng)
    scale_bits = f32_to_bf16_bits((0.02 / math.sqrt(21.25) * (0.75 + 0.5 * u)).astype(np.float32))
    bias_bits = f32_to_bf16_bits((-7.5 * bf16_bits_to_f32(scale_bits).astype(np.float64)).astype(np.float32))
    return {"codes": packed, "scales": scale_bits.reshape(N, K // GROUP),
            "biases": bias_bits.reshape(N, K // GROUP)}


def make_weight(dims: Dims, name: str, seed: int = SEED_WEIGHTS, gains: str = "ones", std: float = 0.02):
    shape = weight_shape(dims, name)
    fp32 = dims.wdtype == WDTYPE_F32
    if is_gain(name):
        if gains == "ones":
            g = np.ones(shape, dtype=np.float64)
        else:
            g = 1.0 + (uniforms(stream_key(seed, name), 0, shape[0]) - 0.5)
        return _store_dense(g, fp32)
    if is_matrix(name) and dims.wdtype == WDTYPE_INT4G64:
        return _int4_matrix(seed, name, shape)
    count = int(np.prod(shape))
    return scaled_normals_stored(seed, name, count, std, fp32).reshape(shape)


class Model(dict):
    """Lazily generated weight set: model[name] generates on first access.
    stds overrides the N(0, 0.02) scale of chosen weights (e.g. a DSpark head
    whose Markov bias competes with the base logits)."""

    def __init__(self, dims: Dims, seed: int = SEED_WEIGHTS, gains: str = "ones", stds=None):
        super().__init__()
        self.dims, self.seed, self.gains = dims, seed, gains
        self.stds = dict(stds or {})

    def __missing__(self, name):
        w = make_weight(self.dims, name, self.seed, self.gains, self.stds.get(name, 0.02))
        self[name] = w
        return w

    def materialise(self):
        for n in weight_names(self.dims):
            self[n]
        return self


# ----------------------------------------------------------------------------
# per-round inputs


def make_taps(dims: Dims, start_row: int, rows: int, stream: str = "ctx", seq: int = 0,
              seed: int = SEED_TAPS):
    """m tap buffers [rows, H] for rows start_row..start_row+rows-1 of a stream."""
    out = []
    for j in range(dims.m):
        x = scaled_normals_stored(seed, f"tap.{j}.{stream}.{seq}", rows * dims.H, 1.0, dims.fp32,
                                  start=start_row * dims.H)
        out.append(x.reshape(rows, dims.H))
    return out


def make_anchors(dims: Dims, round_idx: int, seed: int = SEED_ANCHORS) -> np.ndarray:
    u = uniforms(stream_key(seed, "anchor"), round_idx * dims.B, dims.B)
    return np.minimum((u * dims.V).astype(np.int64), dims.V - 1).astype(np.int32)


def accept_schedule(dims: Dims, round_idx: int, seed: int = SEED_LOGITS) -> np.ndarray:
    """Accepted-prefix length each sequence's planted logits will produce."""
    if dims.name == "tiny":
        return np.full(dims.B, round_idx % (dims.gamma + 1), dtype=np.int32)
    u = uniforms(stream_key(seed, "accept"), round_idx * dims.B, dims.B)
    return np.minimum((u * (dims.gamma + 1)).astype(np.int64), dims.gamma).astype(np.int32)


def plant_target_tokens(dims: Dims, draft_ids: np.ndarray, accept: np.ndarray, round_idx: int,
                        seed: int = SEED_LOGITS) -> np.ndarray:
    """The target's greedy tokens [B, gamma+1] that stop the agreement with
    `draft_ids` after exactly accept[b] tokens (the tokens plant_target_logits
    raises): the drafts up to accept[b], then a token other than the draft at
    accept[b], then seeded tokens."""
    B, G, V = dims.B, dims.gamma, dims.V
    W = G + 1
    picks = uniforms(stream_key(seed, "target_pick"), round_idx * B * W, B * W).reshape(B, W)
    t = np.empty((B, W), dtype=np.int64)
    for b in range(B):
        a = int(accept[b])
        for j in range(W):
            if j < a:
                t[b, j] = int(draft_ids[b, j])
            else:
                t[b, j] = min(int(picks[b, j] * V), V - 1)
                if j == a and j < G and t[b, j] == int(draft_ids[b, j]):
                    t[b, j] = (t[b, j] + 1) % V
    return t


def plant_target_logits(dims: Dims, draft_ids: np.ndarray, accept: np.ndarray, round_idx: int,
                        seed: int = SEED_LOGITS) -> np.ndarray:
    """Target logits [B, gamma+1, V] (float32) whose greedy agreement with
    `draft_ids` stops after exactly accept[b] tokens.

    Rows start as N(0,1). Row j < a gets draft[j] raised to (row max + 1); row
    a < gamma gets some token other than draft[a] raised the same way; every
    later row (and the bonus row) gets a random token raised. Every row's top
    entry therefore leads the runner-up by at least 1.
    """
    B, G, V = dims.B, dims.gamma, dims.V
    W = G + 1
    T = normals(seed, "target_logits", B * W * V, start=round_idx * B * W * V)
    T = T.astype(np.float32).reshape(B, W, V)
    t = plant_target_tokens(dims, draft_ids, accept, round_idx, seed)
    for b in range(B):
        for j in range(W):
            T[b, j, t[b, j]] = np.float32(T[b, j].max()) + np.float32(1.0)
    return T


def context_lengths(dims: Dims, seed: int = SEED_LENGTHS) -> np.ndarray:
    if dims.L_max is None:
        return np.full(dims.B, dims.L, dtype=np.int32)
    u = uniforms(stream_key(seed, "ctx_len"), 0, dims.B)
    span = dims.L_max - dims.L + 1
    return (dims.L + np.minimum((u * span).astype(np.int64), span - 1)).astype(np.int32)
