"""Python binding of libdflash.so (include/dflash.h).

Argument marshalling only: ctypes mirrors of the C structs, wrappers with the
same names as the C calls that pass torch tensors' device pointers and the
current HIP stream, and helpers that upload weights into the layouts the
library expects (fused QKV rows, fused gate/up rows). Every step of the
drafter runs in the library's HIP kernels; there is no fallback. If the
library is missing the import fails loudly.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB_PATH selects another build of the library (tuning variants)
LIB_PATH = os.environ.get("DFLASH_LIB_PATH") or os.path.join(_HERE, "libdflash.so")

DFLASH_OK, DFLASH_DECLINED, DFLASH_EINVAL, DFLASH_ENOSPC, DFLASH_EHIP = 0, 1, -1, -2, -3
DFLASH_F32, DFLASH_BF16, DFLASH_INT4G64 = 0, 1, 2
DFLASH_ACT_GELU_TANH, DFLASH_ACT_SILU = 0, 1

EXPORTS = ["dflash_workspace_bytes", "dflash_query", "dflash_status_string", "dflash_invocations",
           "dflash_context_project", "dflash_ctx_kv_append", "dflash_draft_layer", "dflash_draft_forward",
           "dflash_lm_head_argmax", "dflash_lm_head_workspace_bytes", "dflash_verify_greedy",
           "dflash_verify_workspace_bytes", "dflash_kv_prefill_workspace_bytes", "dflash_trace_begin",
           "dflash_trace_end", "dflash_lm_head_workgroups", "dflash_wall_clock_hz", "dflash_wall_clock_hz_reported", "dflash_verify_greedy_noalloc",
           "dflash_verify_noalloc_max_bytes", "dflash_dspark_workspace_bytes", "dflash_draft_forward_dspark",
           "dflash_verify_greedy_lengths", "dflash_draft_round", "dflash_round_workspace_bytes",
           "dflash_verify_from_hidden", "dflash_verify_hidden_workspace_bytes", "dflash_lm_head_workspace_bytes_for",
           "dflash_int4_prefill_workspace_bytes"]
DFLASH_TRACE_LM_HEAD, DFLASH_TRACE_ATTENTION, DFLASH_TRACE_PROJECTIONS = 1, 2, 4


class DflashError(RuntimeError):
    pass


class dflash_dims(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("m", ctypes.c_int32), ("d", ctypes.c_int32), ("nl", ctypes.c_int32),
                ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("hd", ctypes.c_int32), ("F", ctypes.c_int32),
                ("V", ctypes.c_int32), ("gamma", ctypes.c_int32), ("eps", ctypes.c_float),
                ("act", ctypes.c_int32), ("wdtype", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_theta", ctypes.c_float)]


class dflash_weight(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class dflash_layer(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("w_qkv", dflash_weight), ("w_o", dflash_weight),
                ("ffn_norm", ctypes.c_void_p), ("w_gate_up", dflash_weight), ("w_down", dflash_weight)]


class dflash_model(ctypes.Structure):
    _fields_ = [("dims", dflash_dims), ("w_c", dflash_weight), ("ctx_norm", ctypes.c_void_p),
                ("tok_proj", dflash_weight), ("mask_emb", ctypes.c_void_p), ("block_pos", ctypes.c_void_p),
                ("out_norm", ctypes.c_void_p), ("out_proj", dflash_weight), ("embed_in", dflash_weight),
                ("lm_head", dflash_weight), ("layers", ctypes.POINTER(dflash_layer))]


class dflash_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("cap", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class dflash_dspark_head(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("w1", ctypes.c_void_p), ("w2t", ctypes.c_void_p),
                ("conf_w", ctypes.c_void_p), ("conf_b", ctypes.c_void_p)]


class dflash_trace_record(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 64), ("kind", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("offset", ctypes.c_int64), ("bytes", ctypes.c_double), ("ctx_row_bytes", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_diffusion_draft_tap_amd.build` "
                          "(the drafter has no non-HIP path)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    lib.dflash_workspace_bytes.argtypes = [P(dflash_dims), I32, I32]
    lib.dflash_workspace_bytes.restype = SZ
    lib.dflash_kv_prefill_workspace_bytes.argtypes = [P(dflash_dims), I32]
    lib.dflash_kv_prefill_workspace_bytes.restype = SZ
    lib.dflash_int4_prefill_workspace_bytes.argtypes = [P(dflash_dims), I32]
    lib.dflash_int4_prefill_workspace_bytes.restype = SZ
    lib.dflash_query.argtypes = [P(dflash_dims)]
    lib.dflash_query.restype = ctypes.c_int
    lib.dflash_status_string.argtypes = [ctypes.c_int]
    lib.dflash_status_string.restype = ctypes.c_char_p
    lib.dflash_invocations.argtypes = []
    lib.dflash_invocations.restype = ctypes.c_uint64
    lib.dflash_context_project.argtypes = [P(dflash_model), P(VP), ctypes.c_int64, I32, VP, VP, SZ, VP]
    lib.dflash_context_project.restype = ctypes.c_int
    lib.dflash_ctx_kv_append.argtypes = [P(dflash_model), VP, I32, VP, VP, P(dflash_kv), VP, SZ, VP]
    lib.dflash_ctx_kv_append.restype = ctypes.c_int
    lib.dflash_draft_layer.argtypes = [P(dflash_model), I32, VP, P(dflash_kv), I32, VP, SZ, VP]
    lib.dflash_draft_layer.restype = ctypes.c_int
    lib.dflash_draft_forward.argtypes = [P(dflash_model), VP, P(dflash_kv), I32, VP, VP, VP, VP, SZ, VP]
    lib.dflash_draft_forward.restype = ctypes.c_int
    lib.dflash_lm_head_argmax.argtypes = [P(dflash_weight), VP, I32, I32, VP, VP, VP, SZ, VP]
    lib.dflash_lm_head_argmax.restype = ctypes.c_int
    lib.dflash_lm_head_workspace_bytes.argtypes = [I32, I32]
    lib.dflash_lm_head_workspace_bytes.restype = SZ
    lib.dflash_lm_head_workspace_bytes_for.argtypes = [P(dflash_weight), I32, I32]
    lib.dflash_lm_head_workspace_bytes_for.restype = SZ
    lib.dflash_verify_greedy.argtypes = [VP, VP, I32, I32, I32, VP, VP, VP, VP, VP, SZ, VP]
    lib.dflash_verify_greedy.restype = ctypes.c_int
    lib.dflash_verify_workspace_bytes.argtypes = [I32, I32, I32]
    lib.dflash_verify_workspace_bytes.restype = SZ
    lib.dflash_verify_greedy_noalloc.argtypes = [VP, VP, I32, I32, I32, VP, VP, VP, VP, VP]
    lib.dflash_verify_greedy_noalloc.restype = ctypes.c_int
    lib.dflash_dspark_workspace_bytes.argtypes = [P(dflash_dims), I32, I32, I32]
    lib.dflash_dspark_workspace_bytes.restype = SZ
    lib.dflash_draft_forward_dspark.argtypes = [P(dflash_model), P(dflash_dspark_head), VP, P(dflash_kv), I32, VP,
                                                ctypes.c_float, VP, VP, VP, VP, VP, SZ, VP]
    lib.dflash_draft_forward_dspark.restype = ctypes.c_int
    lib.dflash_verify_greedy_lengths.argtypes = [VP, VP, VP, I32, I32, I32, VP, VP, VP, VP, VP, SZ, VP]
    lib.dflash_verify_greedy_lengths.restype = ctypes.c_int
    lib.dflash_draft_round.argtypes = [P(dflash_model), P(VP), ctypes.c_int64, I32, VP, VP, P(dflash_kv), I32, VP, VP,
                                       VP, VP, VP, SZ, VP]
    lib.dflash_draft_round.restype = ctypes.c_int
    lib.dflash_round_workspace_bytes.argtypes = [P(dflash_dims), I32, I32]
    lib.dflash_round_workspace_bytes.restype = SZ
    lib.dflash_verify_from_hidden.argtypes = [P(dflash_model), VP, I32, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
    lib.dflash_verify_from_hidden.restype = ctypes.c_int
    lib.dflash_verify_hidden_workspace_bytes.argtypes = [P(dflash_dims), I32]
    lib.dflash_verify_hidden_workspace_bytes.restype = SZ
    lib.dflash_verify_noalloc_max_bytes.argtypes = []
    lib.dflash_verify_noalloc_max_bytes.restype = SZ
    lib.dflash_trace_begin.argtypes = [I32, VP, ctypes.c_int64]
    lib.dflash_trace_begin.restype = None
    lib.dflash_trace_end.argtypes = [P(dflash_trace_record), I32]
    lib.dflash_trace_end.restype = I32
    lib.dflash_lm_head_workgroups.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.dflash_lm_head_workgroups.restype = ctypes.c_int32
    lib.dflash_wall_clock_hz.argtypes = []
    lib.dflash_wall_clock_hz.restype = ctypes.c_double
    lib.dflash_wall_clock_hz_reported.argtypes = []
    lib.dflash_wall_clock_hz_reported.restype = ctypes.c_double
    return lib


lib = _load()


def status_string(code):
    return lib.dflash_status_string(int(code)).decode()


def check(code, what=""):
    """Raise on errors; return the code (OK or DECLINED) otherwise."""
    if code < 0:
        raise DflashError(f"{what}: {status_string(code)} ({code})")
    return code


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------------------
# dims and weights


_WD = {"f32": DFLASH_F32, "bf16": DFLASH_BF16, "int4g64": DFLASH_INT4G64}
_ACT = {"gelu_tanh": DFLASH_ACT_GELU_TANH, "silu": DFLASH_ACT_SILU}


def make_dims(d):
    """dflash_dims from any object with the drafter geometry attributes."""
    return dflash_dims(H=d.H, m=d.m, d=d.d, nl=d.nl, hq=d.hq, hkv=d.hkv, hd=d.hd, F=d.F, V=d.V, gamma=d.gamma,
                       eps=float(d.eps), act=_ACT[d.act], wdtype=_WD[d.wdtype], window=int(getattr(d, "window", 0)),
                       rope_theta=float(getattr(d, "rope_theta", 0.0)))


def _to_dev(a, device):
    if isinstance(a, torch.Tensor):
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


class Weight:
    """A matrix on the device in one of the library's formats."""

    def __init__(self, stored, device):
        if isinstance(stored, dict):
            self.dtype = DFLASH_INT4G64
            self.rows = stored["codes"].shape[0]
            self.cols = stored["codes"].shape[1] * 8
            self.data = _to_dev(stored["codes"], device)
            self.scales = _to_dev(stored["scales"], device)
            self.biases = _to_dev(stored["biases"], device)
        elif isinstance(stored, torch.Tensor):
            if stored.dtype not in (torch.bfloat16, torch.float32) or stored.dim() != 2:
                raise DflashError("device weights are 2-D bfloat16 or float32 tensors")
            self.dtype = DFLASH_BF16 if stored.dtype == torch.bfloat16 else DFLASH_F32
            self.rows, self.cols = stored.shape
            self.data = _to_dev(stored, device)
            self.scales = self.biases = None
        else:
            a = np.asarray(stored)
            self.dtype = DFLASH_BF16 if a.dtype == np.uint16 else DFLASH_F32
            if a.dtype not in (np.uint16, np.float32):
                a = a.astype(np.float32)
            self.rows, self.cols = a.shape
            self.data = _to_dev(a, device)
            self.scales = self.biases = None

    def c(self):
        return dflash_weight(dtype=self.dtype, rows=self.rows, cols=self.cols, data=_ptr(self.data),
                             scales=_ptr(self.scales), biases=_ptr(self.biases))


def cat_rows(parts):
    """Concatenate stored matrices along the output axis (fused layouts)."""
    if isinstance(parts[0], dict):
        return {k: np.concatenate([p[k] for p in parts], axis=0) for k in ("codes", "scales", "biases")}
    if isinstance(parts[0], torch.Tensor):
        return torch.cat(parts, dim=0)
    return np.concatenate([np.asarray(p) for p in parts], axis=0)


class DeviceModel:
    """Drafter weights on the device plus the dflash_model descriptor.

    `weights` maps the drafter's parameter names (bb.{i}.{attn_norm,q,k,v,o,
    ff_norm,gate,up,down}, W_c, ctx_norm, tok_proj, mask_emb, block_pos,
    out_norm, out_proj, E_in, E_out) to stored arrays ([out, in] matrices)."""

    def __init__(self, dims, weights, device="cuda"):
        self.dims = dims
        self.cdims = make_dims(dims)
        dev = torch.device(device)
        self._keep = []

        def vec(name):
            w = weights[name]
            t = _to_dev(w if isinstance(w, torch.Tensor) else np.asarray(w), dev)
            self._keep.append(t)
            return t

        self.w_c = Weight(weights["W_c"], dev)
        self.tok_proj = Weight(weights["tok_proj"], dev)
        self.out_proj = Weight(weights["out_proj"], dev)
        self.embed_in = Weight(weights["E_in"], dev)
        self.lm_head = self.embed_in if weights["E_out"] is weights["E_in"] else Weight(weights["E_out"], dev)
        self.ctx_norm, self.out_norm = vec("ctx_norm"), vec("out_norm")
        self.block_pos = vec("block_pos")
        self.mask_emb = vec("mask_emb") if dims.gamma > 1 else None
        self.layers = []
        for i in range(dims.nl):
            g = lambda n: weights[f"bb.{i}.{n}"]
            L = {
                "attn_norm": vec(f"bb.{i}.attn_norm"),
                "ffn_norm": vec(f"bb.{i}.ff_norm"),
                "w_qkv": Weight(cat_rows([g("q"), g("k"), g("v")]), dev),
                "w_o": Weight(g("o"), dev),
                "w_gate_up": Weight(cat_rows([g("gate"), g("up")]), dev),
                "w_down": Weight(g("down"), dev),
            }
            self.layers.append(L)
        n = max(1, dims.nl)
        self._c_layers = (dflash_layer * n)()
        for i, L in enumerate(self.layers):
            self._c_layers[i] = dflash_layer(attn_norm=_ptr(L["attn_norm"]), w_qkv=L["w_qkv"].c(),
                                             w_o=L["w_o"].c(), ffn_norm=_ptr(L["ffn_norm"]),
                                             w_gate_up=L["w_gate_up"].c(), w_down=L["w_down"].c())
        self.c = dflash_model(dims=self.cdims, w_c=self.w_c.c(), ctx_norm=_ptr(self.ctx_norm),
                              tok_proj=self.tok_proj.c(), mask_emb=_ptr(self.mask_emb),
                              block_pos=_ptr(self.block_pos), out_norm=_ptr(self.out_norm),
                              out_proj=self.out_proj.c(), embed_in=self.embed_in.c(), lm_head=self.lm_head.c(),
                              layers=ctypes.cast(self._c_layers, ctypes.POINTER(dflash_layer)))

    @property
    def act_dtype(self):
        return torch.float32 if self.dims.wdtype == "f32" else torch.bfloat16


class KVCache:
    """Retained context K/V: k [nl, B, hkv, cap, hd]; v [nl, B, hkv, cap/32, hd, 32]
    for bf16 models (32-key chunks, head-dim major inside a chunk), [nl, B, hkv, hd,
    cap] for f32 models; len int32 [B]. cap is rounded up to a multiple of 32."""

    def __init__(self, dims, B, cap, device="cuda"):
        dt = torch.float32 if dims.wdtype == "f32" else torch.bfloat16
        cap = (cap + 31) // 32 * 32
        nl = max(1, dims.nl)
        self.k = torch.zeros((nl, B, dims.hkv, cap, dims.hd), dtype=dt, device=device)
        vshape = (nl, B, dims.hkv, dims.hd, cap) if dt == torch.float32 else (nl, B, dims.hkv, cap // 32, dims.hd, 32)
        self.v = torch.zeros(vshape, dtype=dt, device=device)
        self.len = torch.zeros(B, dtype=torch.int32, device=device)
        self.B, self.cap = B, cap
        self.c = dflash_kv(k=_ptr(self.k), v=_ptr(self.v), len=_ptr(self.len), B=B, cap=cap,
                           dtype=DFLASH_F32 if dt == torch.float32 else DFLASH_BF16)


def workspace(dims, B, cap, device="cuda"):
    n = lib.dflash_workspace_bytes(ctypes.byref(make_dims(dims)), B, cap)
    if n == 0:
        raise DflashError("invalid dims for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# the calls (same names as the C ABI)


def dflash_query(dims):
    return lib.dflash_query(ctypes.byref(make_dims(dims) if not isinstance(dims, dflash_dims) else dims))


def dflash_invocations():
    return int(lib.dflash_invocations())


def dflash_context_project(model, taps, h_ctx, ws=None, stream=None):
    n = taps[0].shape[0]
    arr = (ctypes.c_void_p * len(taps))(*[_ptr(t) for t in taps])
    ld = taps[0].stride(0)
    return lib.dflash_context_project(ctypes.byref(model.c), arr, ld, n, _ptr(h_ctx), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream))


def dflash_ctx_kv_append(model, h_ctx, row_offsets, counts, kv, ws=None, stream=None):
    n = h_ctx.shape[0]
    return lib.dflash_ctx_kv_append(ctypes.byref(model.c), _ptr(h_ctx), n, _ptr(row_offsets), _ptr(counts),
                                    ctypes.byref(kv.c), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream))


def dflash_draft_layer(model, layer, h_block, kv, B, ws, stream=None):
    return lib.dflash_draft_layer(ctypes.byref(model.c), layer, _ptr(h_block), ctypes.byref(kv.c), B, _ptr(ws),
                                  ws.numel(), _stream(stream))


def dflash_draft_forward(model, anchor_ids, kv, B, draft_ids, ws, y_out=None, max_logit=None, stream=None):
    return lib.dflash_draft_forward(ctypes.byref(model.c), _ptr(anchor_ids), ctypes.byref(kv.c), B,
                                    _ptr(draft_ids), _ptr(y_out), _ptr(max_logit), _ptr(ws), ws.numel(),
                                    _stream(stream))


def dflash_lm_head_argmax(weight, y, ids, ws, max_logit=None, stream=None):
    cw = weight.c() if isinstance(weight, Weight) else weight
    ydt = DFLASH_F32 if y.dtype == torch.float32 else DFLASH_BF16
    return lib.dflash_lm_head_argmax(ctypes.byref(cw), _ptr(y), ydt, y.shape[0], _ptr(ids), _ptr(max_logit),
                                     _ptr(ws), ws.numel(), _stream(stream))


class DsparkHead:
    """The DSpark heads on the device: markov.w1 [V, r], markov.w2 [r, V]
    (uploaded transposed, [V, r]), conf.w [d + r, 1], conf.b [1]; stored
    arrays of the weights' storage format (bf16 bits, or float32 for f32
    models)."""

    def __init__(self, weights, device="cuda"):
        w1 = weights["markov.w1"]
        w2 = weights["markov.w2"]
        self.r = int(np.asarray(w1).shape[1]) if not isinstance(w1, torch.Tensor) else int(w1.shape[1])
        self.w1 = _to_dev(w1, device)
        w2t = w2.t().contiguous() if isinstance(w2, torch.Tensor) else np.ascontiguousarray(np.asarray(w2).T)
        self.w2t = _to_dev(w2t, device)
        self.conf_w = _to_dev(weights["conf.w"], device).reshape(-1).contiguous()
        self.conf_b = _to_dev(weights["conf.b"], device).reshape(-1).contiguous()
        self.c = dflash_dspark_head(r=self.r, w1=_ptr(self.w1), w2t=_ptr(self.w2t), conf_w=_ptr(self.conf_w),
                                    conf_b=_ptr(self.conf_b))


def dspark_workspace(dims, r, B, cap, device="cuda"):
    n = lib.dflash_dspark_workspace_bytes(ctypes.byref(make_dims(dims)), r, B, cap)
    if n == 0:
        raise DflashError("invalid dims for a DSpark workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dflash_draft_forward_dspark(model, head, anchor_ids, kv, B, draft_ids, ws, thresholds=None, min_conf=0.0,
                                conf=None, lengths=None, y_out=None, stream=None):
    return lib.dflash_draft_forward_dspark(ctypes.byref(model.c), ctypes.byref(head.c), _ptr(anchor_ids),
                                           ctypes.byref(kv.c), B, _ptr(thresholds), float(min_conf),
                                           _ptr(draft_ids), _ptr(conf), _ptr(lengths), _ptr(y_out), _ptr(ws),
                                           ws.numel(), _stream(stream))


def dflash_verify_greedy_lengths(target_logits, draft_ids, lengths, accepted, committed, ids, ws, next_anchor=None,
                                 stream=None):
    B, W, V = target_logits.shape
    return lib.dflash_verify_greedy_lengths(_ptr(target_logits), _ptr(draft_ids), _ptr(lengths), B, W - 1, V,
                                            _ptr(accepted), _ptr(committed), _ptr(ids), _ptr(next_anchor),
                                            _ptr(ws), ws.numel(), _stream(stream))


def verify_hidden_workspace(dims, B, device="cuda"):
    n = lib.dflash_verify_hidden_workspace_bytes(ctypes.byref(make_dims(dims)), B)
    if n == 0:
        raise DflashError("invalid dims for a verify-from-hidden workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dflash_verify_from_hidden(model, target_hidden, draft_ids, accepted, committed, ids, ws, lengths=None,
                              next_anchor=None, stream=None):
    B = target_hidden.shape[0]
    return lib.dflash_verify_from_hidden(ctypes.byref(model.c), _ptr(target_hidden), B, _ptr(draft_ids),
                                         _ptr(lengths), _ptr(accepted), _ptr(committed), _ptr(ids),
                                         _ptr(next_anchor), _ptr(ws), ws.numel(), _stream(stream))


def round_workspace(dims, B, cap, device="cuda"):
    n = lib.dflash_round_workspace_bytes(ctypes.byref(make_dims(dims)), B, cap)
    if n == 0:
        raise DflashError("invalid dims for a round workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dflash_draft_round(model, taps, row_offsets, counts, kv, B, anchor_ids, draft_ids, ws, y_out=None, max_logit=None,
                       stream=None):
    n = taps[0].shape[0]
    arr = (ctypes.c_void_p * len(taps))(*[_ptr(t) for t in taps])
    return lib.dflash_draft_round(ctypes.byref(model.c), arr, taps[0].stride(0), n, _ptr(row_offsets), _ptr(counts),
                                  ctypes.byref(kv.c), B, _ptr(anchor_ids), _ptr(draft_ids), _ptr(y_out),
                                  _ptr(max_logit), _ptr(ws), ws.numel(), _stream(stream))


def kv_prefill_workspace(dims, n, device="cuda"):
    """Workspace with which a K/V append of n >= 64 rows stages every layer's
    normalised rows as bf16 before its matrix-core GEMM."""
    nb = lib.dflash_kv_prefill_workspace_bytes(ctypes.byref(make_dims(dims)), n)
    if nb == 0:
        raise DflashError("invalid dims or row count for a prefill workspace")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def int4_prefill_workspace(dims, n, device="cuda"):
    """The workspace with which an int4 model's context projection and K/V append of n >= 64
    rows run on matrix cores (their weights expanded into bf16 high and low parts)."""
    nb = lib.dflash_int4_prefill_workspace_bytes(ctypes.byref(make_dims(dims)), n)
    if nb == 0:
        raise DflashError("no int4 prefill workspace for these dims or row count")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def lm_head_workspace(V, M, device="cuda"):
    return torch.empty(lib.dflash_lm_head_workspace_bytes(V, M), dtype=torch.uint8, device=device)


def lm_head_workspace_for(weight, y_dtype, M, device="cuda"):
    """The workspace for the head's fastest path (its matrix-core path, where it has one)."""
    cw = weight.c() if isinstance(weight, Weight) else weight
    ydt = DFLASH_F32 if y_dtype == torch.float32 else DFLASH_BF16
    return torch.empty(lib.dflash_lm_head_workspace_bytes_for(ctypes.byref(cw), ydt, M), dtype=torch.uint8,
                       device=device)


def dflash_verify_greedy(target_logits, draft_ids, accepted, committed, ids, ws, next_anchor=None, stream=None):
    B, W, V = target_logits.shape
    return lib.dflash_verify_greedy(_ptr(target_logits), _ptr(draft_ids), B, W - 1, V, _ptr(accepted),
                                    _ptr(committed), _ptr(ids), _ptr(next_anchor), _ptr(ws), ws.numel(),
                                    _stream(stream))


def dflash_verify_greedy_noalloc(target_logits, draft_ids, accepted, committed, ids, next_anchor=None,
                                 stream=None):
    B, W, V = target_logits.shape
    return lib.dflash_verify_greedy_noalloc(_ptr(target_logits), _ptr(draft_ids), B, W - 1, V, _ptr(accepted),
                                            _ptr(committed), _ptr(ids), _ptr(next_anchor), _stream(stream))


def verify_workspace(B, gamma, V, device="cuda"):
    return torch.empty(lib.dflash_verify_workspace_bytes(B, gamma, V), dtype=torch.uint8, device=device)


def dflash_trace_begin(kinds, stamps):
    """Trace the launches of `kinds` (DFLASH_TRACE_* bits): their workgroups
    write wall-clock (start, end) pairs into `stamps`, an int64 device tensor."""
    assert stamps.dtype == torch.int64 and stamps.is_cuda and stamps.is_contiguous()
    lib.dflash_trace_begin(int(kinds), _ptr(stamps), stamps.numel())


def dflash_trace_end(capacity=4096):
    """Stop tracing; the records of the traced launches as dicts (kernel,
    kind, workgroups, offset, bytes, ctx_row_bytes), in enqueue order."""
    recs = (dflash_trace_record * capacity)()
    n = lib.dflash_trace_end(recs, capacity)
    return [{"kernel": r.kernel.decode(), "kind": r.kind, "workgroups": r.workgroups, "offset": r.offset,
             "bytes": r.bytes, "ctx_row_bytes": r.ctx_row_bytes} for r in recs[:min(n, capacity)]]


def dflash_lm_head_workgroups(V, H, dtype, M, y_dtype=None):
    """(workgroups per launch, launches) of the LM head over M rows. dtype: a
    DFLASH_* weight format or a workload weight name ("f32", "bf16", "int4g64");
    y_dtype: the rows' format (default: fp32 rows for an f32 head, bf16 otherwise)."""
    if isinstance(dtype, str):
        dtype = _WD[dtype]
    if y_dtype is None:
        y_dtype = DFLASH_F32 if dtype == DFLASH_F32 else DFLASH_BF16
    n = ctypes.c_int32(0)
    w = lib.dflash_lm_head_workgroups(V, H, dtype, M, y_dtype, ctypes.byref(n))
    return w, n.value


def dflash_wall_clock_hz():
    return lib.dflash_wall_clock_hz()


def dflash_wall_clock_hz_reported():
    return lib.dflash_wall_clock_hz_reported()


def traced_durations_s(stamps, records):
    """Duration (seconds) of every traced launch: its last workgroup end minus
    its first workgroup start, read from the stamp buffer."""
    a = stamps.cpu().numpy().astype(np.int64)
    hz = lib.dflash_wall_clock_hz()
    if hz <= 0:
        raise DflashError("the runtime reports no wall-clock rate")
    out = []
    for r in records:
        x = a[r["offset"]:r["offset"] + 2 * r["workgroups"]].reshape(-1, 2)
        out.append((int(x[:, 1].max()) - int(x[:, 0].min())) / hz)
    return out
