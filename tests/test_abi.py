"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and validates arguments on the host before enqueueing
anything (invalid -> EINVAL, unsupported -> DECLINED, short workspace ->
ENOSPC). Pointers passed here are never dereferenced by the library: every
call below is rejected before any device work."""

import ctypes
import os
import re

import pytest

from block_diffusion_draft_tap_amd import binding as bd
from synth import TINY, DEFAULT, WIDE, WIDE4, BATCHED, DFLASH2, scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(bd.lib, n), n
    assert set(names) == set(bd.EXPORTS)


def test_status_strings():
    for code in (0, 1, -1, -2, -3):
        assert bd.status_string(code)
    assert "declined" in bd.status_string(1)


@pytest.mark.parametrize("cfg", [TINY, DEFAULT, WIDE, WIDE4, BATCHED, DFLASH2], ids=lambda c: c.name)
def test_query_valid_dims_without_device_declines(cfg):
    # consistent dims: OK on an MI355X, DECLINED where there is no gfx950 device
    rc = bd.dflash_query(cfg)
    assert rc in (bd.DFLASH_OK, bd.DFLASH_DECLINED)
    assert bd.lib.dflash_workspace_bytes(ctypes.byref(bd.make_dims(cfg)), cfg.B, cfg.L + 64) > 0


def test_query_rejects_inconsistent_and_unsupported_dims():
    d = bd.make_dims(DEFAULT)
    d.d = 1000                     # d != hq * hd
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_EINVAL
    d = bd.make_dims(DEFAULT)
    d.hkv = 3                      # hq % hkv != 0
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_EINVAL
    d = bd.make_dims(scaled(DEFAULT, hd=256, hq=4, hkv=4))
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_DECLINED      # head dim not served
    d = bd.make_dims(DEFAULT)
    d.wdtype = 7
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_DECLINED
    d = bd.make_dims(scaled(DEFAULT, gamma=70))
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_DECLINED      # verify width > 64
    # the block's keys form one 32-key attention unit: gamma 32 is served (where a gfx950
    # device is), 33 is declined for every weight format, MHA or grouped heads alike
    for wd in ("f32", "bf16", "int4g64"):
        for hq, hkv in ((8, 8), (8, 1)):
            ok = bd.make_dims(scaled(DEFAULT, gamma=32, hq=hq, hkv=hkv, wdtype=wd))
            if hq // hkv * 32 <= 48:
                assert bd.lib.dflash_query(ctypes.byref(ok)) in (bd.DFLASH_OK, bd.DFLASH_DECLINED)
            big = bd.make_dims(scaled(DEFAULT, gamma=33, hq=hq, hkv=hkv, wdtype=wd))
            assert bd.lib.dflash_query(ctypes.byref(big)) == bd.DFLASH_DECLINED, (wd, hq, hkv)
    d = bd.make_dims(DEFAULT)
    d.eps = -1.0
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_EINVAL
    assert bd.lib.dflash_workspace_bytes(None, 1, 10) == 0
    assert bd.lib.dflash_query(None) == bd.DFLASH_EINVAL


def test_kv_prefill_workspace_size():
    # every layer's normalised rows as bf16, rounded up to 256 bytes; 0 when invalid
    f = bd.lib.dflash_kv_prefill_workspace_bytes
    for cfg, n in ((DEFAULT, 2048), (BATCHED, 192011), (scaled(DEFAULT, nl=1, hq=4, hkv=4, d=512), 65)):
        exact = cfg.nl * n * cfg.d * 2
        got = f(ctypes.byref(bd.make_dims(cfg)), n)
        assert got >= exact and got - exact < 256 and got % 256 == 0, (cfg.name, n, got)
    assert f(ctypes.byref(bd.make_dims(DEFAULT)), 0) == 0
    assert f(ctypes.byref(bd.make_dims(DEFAULT)), -5) == 0
    assert f(None, 100) == 0
    bad = bd.make_dims(DEFAULT)
    bad.d = 1000                   # d != hq * hd
    assert f(ctypes.byref(bad), 100) == 0


def test_kill_switch_declines(monkeypatch):
    monkeypatch.setenv("DFLASH_DISABLE", "1")
    assert bd.dflash_query(DEFAULT) == bd.DFLASH_DECLINED


class _FakeModel:
    """A dflash_model whose device pointers are dummies (never dereferenced)."""

    def __init__(self, dims):
        P = 1 << 20
        self.dims = dims
        w = lambda r, c, dt=None: bd.dflash_weight(
            dtype=bd._WD[dims.wdtype] if dt is None else dt, rows=r, cols=c, data=P, scales=P, biases=P)
        qkv = (dims.hq + 2 * dims.hkv) * dims.hd
        self.layers = (bd.dflash_layer * dims.nl)()
        for i in range(dims.nl):
            self.layers[i] = bd.dflash_layer(attn_norm=P, w_qkv=w(qkv, dims.d), w_o=w(dims.d, dims.d), ffn_norm=P,
                                             w_gate_up=w(2 * dims.F, dims.d), w_down=w(dims.d, dims.F))
        self.c = bd.dflash_model(dims=bd.make_dims(dims), w_c=w(dims.d, dims.m * dims.H), ctx_norm=P,
                                 tok_proj=w(dims.d, dims.H), mask_emb=P, block_pos=P, out_norm=P,
                                 out_proj=w(dims.H, dims.d), embed_in=w(dims.V, dims.H),
                                 lm_head=w(dims.V, dims.H),
                                 layers=ctypes.cast(self.layers, ctypes.POINTER(bd.dflash_layer)))
        self.kv = bd.dflash_kv(k=P, v=P, len=P, B=1, cap=64,
                               dtype=bd.DFLASH_F32 if dims.wdtype == "f32" else bd.DFLASH_BF16)


def test_forward_argument_validation():
    fm = _FakeModel(DEFAULT)
    P = 1 << 20
    lib = bd.lib
    # null model / anchors
    assert lib.dflash_draft_forward(None, P, ctypes.byref(fm.kv), 1, P, None, None, P, 1 << 30, None) == bd.DFLASH_EINVAL
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), None, ctypes.byref(fm.kv), 1, P, None, None, P, 1 << 30,
                                    None) == bd.DFLASH_EINVAL
    # workspace too small
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), P, ctypes.byref(fm.kv), 1, P, None, None, P, 16,
                                    None) == bd.DFLASH_ENOSPC
    # more sequences than the cache holds
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), P, ctypes.byref(fm.kv), 2, P, None, None, P, 1 << 30,
                                    None) == bd.DFLASH_EINVAL
    # wrong weight shape
    fm.c.tok_proj.rows = 7
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), P, ctypes.byref(fm.kv), 1, P, None, None, P, 1 << 30,
                                    None) == bd.DFLASH_EINVAL
    fm.c.tok_proj.rows = DEFAULT.d
    # kv dtype must match the model
    fm.kv.dtype = bd.DFLASH_F32
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), P, ctypes.byref(fm.kv), 1, P, None, None, P, 1 << 30,
                                    None) == bd.DFLASH_EINVAL
    fm.kv.dtype = bd.DFLASH_BF16
    # weight data and norm gains are read as 16-byte vectors: other alignments are declined
    fm.c.out_norm = P + 8
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), P, ctypes.byref(fm.kv), 1, P, None, None, P, 1 << 30,
                                    None) == bd.DFLASH_DECLINED
    fm.c.out_norm = P
    fm.c.w_c.data = P + 4
    assert lib.dflash_draft_forward(ctypes.byref(fm.c), P, ctypes.byref(fm.kv), 1, P, None, None, P, 1 << 30,
                                    None) == bd.DFLASH_DECLINED
    fm.c.w_c.data = P
    # a valid request reaches the device gate: served on gfx950, declined without one
    rc = lib.dflash_draft_layer(ctypes.byref(fm.c), 9, P, ctypes.byref(fm.kv), 1, P, 1 << 30, None)
    assert rc == bd.DFLASH_EINVAL  # layer index out of range


def test_verify_and_head_validation():
    lib = bd.lib
    P = 1 << 20
    assert lib.dflash_verify_greedy(None, P, 1, 7, 100, P, P, P, None, P, 1 << 20, None) == bd.DFLASH_EINVAL
    assert lib.dflash_verify_greedy(P, P, 1, 70, 100, P, P, P, None, P, 1 << 20, None) == bd.DFLASH_DECLINED
    assert lib.dflash_verify_greedy(P, P, 1, 7, 100, P, P, P, None, P, 4, None) == bd.DFLASH_ENOSPC
    assert lib.dflash_verify_greedy(P + 4, P, 1, 7, 100, P, P, P, None, P, 1 << 20, None) == bd.DFLASH_DECLINED
    assert lib.dflash_verify_workspace_bytes(1, 7, 151936) > 0
    # the variant without a workspace: the same checks, and requests beyond its fixed
    # scratch are refused before any enqueue
    mx = lib.dflash_verify_noalloc_max_bytes()
    assert mx == 1 << 20
    assert lib.dflash_verify_greedy_noalloc(None, P, 1, 7, 100, P, P, P, None, None) == bd.DFLASH_EINVAL
    assert lib.dflash_verify_greedy_noalloc(P, P, 1, 70, 100, P, P, P, None, None) == bd.DFLASH_DECLINED
    assert lib.dflash_verify_greedy_noalloc(P + 4, P, 1, 7, 100, P, P, P, None, None) == bd.DFLASH_DECLINED
    big_b = 4000                                           # 4000 x 8 rows x 38 splits x 8 B > 1 MiB
    assert lib.dflash_verify_workspace_bytes(big_b, 7, 151936) > mx
    assert lib.dflash_verify_greedy_noalloc(P, P, big_b, 7, 151936, P, P, P, None, None) == bd.DFLASH_ENOSPC
    w = bd.dflash_weight(dtype=bd.DFLASH_BF16, rows=1000, cols=256, data=P, scales=None, biases=None)
    assert lib.dflash_lm_head_argmax(ctypes.byref(w), P, bd.DFLASH_BF16, 5, P, None, P, 8, None) == bd.DFLASH_ENOSPC
    assert lib.dflash_lm_head_argmax(ctypes.byref(w), P, 9, 5, P, None, P, 1 << 20, None) == bd.DFLASH_EINVAL
    w.dtype = bd.DFLASH_INT4G64   # 4-bit without scales
    assert lib.dflash_lm_head_argmax(ctypes.byref(w), P, bd.DFLASH_BF16, 5, P, None, P, 1 << 20,
                                     None) == bd.DFLASH_EINVAL


def test_dspark_and_length_verify_validation():
    fm = _FakeModel(DEFAULT)
    lib = bd.lib
    P = 1 << 20
    head = bd.dflash_dspark_head(r=256, w1=P, w2t=P, conf_w=P, conf_b=P)
    args = lambda h, mc=0.0, ws=1 << 30: (ctypes.byref(fm.c), h, P, ctypes.byref(fm.kv), 1, None, mc, P, None, None,
                                          None, P, ws, None)
    assert lib.dflash_draft_forward_dspark(*args(None)) == bd.DFLASH_EINVAL
    assert lib.dflash_draft_forward_dspark(*args(ctypes.byref(head), float("nan"))) == bd.DFLASH_EINVAL
    assert lib.dflash_draft_forward_dspark(*args(ctypes.byref(head), 0.0, 16)) == bd.DFLASH_ENOSPC
    bad = bd.dflash_dspark_head(r=12, w1=P, w2t=P, conf_w=P, conf_b=P)      # rows of 12 bf16: not 16-byte
    assert lib.dflash_draft_forward_dspark(*args(ctypes.byref(bad))) == bd.DFLASH_DECLINED
    bad = bd.dflash_dspark_head(r=256, w1=P, w2t=None, conf_w=P, conf_b=P)
    assert lib.dflash_draft_forward_dspark(*args(ctypes.byref(bad))) == bd.DFLASH_EINVAL
    dims = ctypes.byref(bd.make_dims(DEFAULT))
    n = lib.dflash_dspark_workspace_bytes(dims, 256, 1, 2112)
    # the forward's own workspace plus the base logits of the block rows at least
    assert n >= lib.dflash_workspace_bytes(dims, 1, 2112) + DEFAULT.gamma * DEFAULT.V * 4
    assert lib.dflash_dspark_workspace_bytes(dims, 0, 1, 2112) == 0
    # the length-capped verify: lengths are required; otherwise the plain verify's checks
    assert lib.dflash_verify_greedy_lengths(P, P, None, 1, 7, 100, P, P, P, None, P, 1 << 20, None) == bd.DFLASH_EINVAL
    assert lib.dflash_verify_greedy_lengths(P, P, P, 1, 70, 100, P, P, P, None, P, 1 << 20, None) == bd.DFLASH_DECLINED
    assert lib.dflash_verify_greedy_lengths(P, P, P, 1, 7, 100, P, P, P, None, P, 4, None) == bd.DFLASH_ENOSPC


def test_dflash2_dims_and_hidden_verify_validation():
    # the variant's fields: a window and a rotary base, zero for the plain drafter
    for w, theta in ((2048, 1e6), (1, 1e4), (0, 0.0)):
        d = bd.make_dims(scaled(DFLASH2, window=w, rope_theta=theta))
        assert bd.lib.dflash_query(ctypes.byref(d)) in (bd.DFLASH_OK, bd.DFLASH_DECLINED)
    d = bd.make_dims(DFLASH2)
    d.window = -1
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_EINVAL
    d = bd.make_dims(DFLASH2)
    d.rope_theta = -1.0
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_EINVAL
    d.rope_theta = float("nan")
    assert bd.lib.dflash_query(ctypes.byref(d)) == bd.DFLASH_EINVAL
    # a window shrinks the attention's partial results, never below the plain drafter's need
    # for short caches
    plain = bd.make_dims(scaled(DFLASH2, window=0, rope_theta=0.0))
    assert 0 < bd.lib.dflash_workspace_bytes(ctypes.byref(bd.make_dims(DFLASH2)), 1, 8256) \
        <= bd.lib.dflash_workspace_bytes(ctypes.byref(plain), 1, 8256)
    # verify from hidden states: the workspace holds the target ids and the head's partials
    dims = ctypes.byref(bd.make_dims(DFLASH2))
    n = bd.lib.dflash_verify_hidden_workspace_bytes(dims, 3)
    assert n >= 3 * (DFLASH2.gamma + 1) * 4 * 3
    assert bd.lib.dflash_verify_hidden_workspace_bytes(dims, 0) == 0
    assert bd.lib.dflash_verify_hidden_workspace_bytes(None, 3) == 0
    fm = _FakeModel(DFLASH2)
    P = 1 << 20
    lib = bd.lib
    v = lambda hid, B, ws, wsb: lib.dflash_verify_from_hidden(ctypes.byref(fm.c), hid, B, P, None, P, P, P, None, ws,
                                                               wsb, None)
    assert v(None, 1, P, n) == bd.DFLASH_EINVAL
    assert v(P, 0, P, n) == bd.DFLASH_EINVAL
    assert v(P + 2, 1, P, n) == bd.DFLASH_DECLINED          # hidden rows read as 16-byte vectors
    assert v(P, 3, P, n - 1) == bd.DFLASH_ENOSPC
    assert v(P, 3, None, n) == bd.DFLASH_ENOSPC


def test_append_and_project_validation():
    fm = _FakeModel(TINY)
    lib = bd.lib
    P = 1 << 20
    taps = (ctypes.c_void_p * TINY.m)(P, P)
    assert lib.dflash_context_project(ctypes.byref(fm.c), taps, TINY.H, -1, P, None, 0, None) == bd.DFLASH_EINVAL
    assert lib.dflash_context_project(ctypes.byref(fm.c), taps, TINY.H - 1, 4, P, None, 0, None) == bd.DFLASH_EINVAL
    bad = (ctypes.c_void_p * TINY.m)(P + 2, P)
    assert lib.dflash_context_project(ctypes.byref(fm.c), bad, TINY.H, 4, P, None, 0, None) == bd.DFLASH_DECLINED
    assert lib.dflash_ctx_kv_append(ctypes.byref(fm.c), P, 4, None, None, ctypes.byref(fm.kv), None, 0,
                                    None) == bd.DFLASH_EINVAL
