"""GPU parity of the DFlash2 variant's verification from the target's hidden
states (page "Inco Hacks Native: DFlash 2 Speculation", section 3: the target
verifies the block): the borrowed LM head scores the target's hidden rows and
the greedy prefix rule decides, against the CPU oracle on the same inputs.

The hidden rows are planted along the head rows of chosen target tokens, so
every target argmax is decided by a wide margin (checked on the oracle's
logits) and the expected acceptance is known. The drafter's rotary positions
and context window run through every test of the parity suite (the d2_* cases
there).
"""

import numpy as np
import pytest
import torch

import block_diffusion_draft_tap_amd as dfa
from block_diffusion_draft_tap_amd import binding as bd
from gpu_common import log
from oracle import dflash_oracle as O
from test_gpu_parity import get

pytestmark = pytest.mark.gpu


def plant_hidden(E_out, tokens, scale=4.0):
    E = O.dense(E_out)
    rows = E[tokens.reshape(-1)]
    h = scale * rows / np.linalg.norm(rows, axis=1, keepdims=True)
    return h.reshape(tokens.shape + (E.shape[1],))


@pytest.mark.parametrize("name", ["d2_tiny", "d2_gqa", "d2_wide4", "d2_batched"])
@pytest.mark.parametrize("nseq", [8, 24])
def test_verify_from_hidden(name, nseq):
    """nseq sequences (24: more than 16 verify rows in all, the head's matrix-core
    path for bf16 models), every accept length, with and without length caps."""
    s = get(name)
    d = s.dims
    G = d.gamma
    rng = np.random.default_rng(nseq)
    t = rng.integers(0, d.V, size=(nseq, G + 1))
    accept = np.arange(nseq) % (G + 1)
    draft = t[:, :G].copy()
    for b in range(nseq):
        if accept[b] < G:
            draft[b, accept[b]] = (t[b, accept[b]] + 1 + rng.integers(0, d.V - 1)) % d.V
    hidden = plant_hidden(s.w["E_out"], t)
    if d.wdtype != "f32":
        hidden = O.bf16(hidden)                 # the target hands over bf16 rows
    logits = hidden.reshape(-1, d.H) @ O.dense(s.w["E_out"]).T
    srt = np.sort(logits, axis=1)
    assert np.min(srt[:, -1] - srt[:, -2]) > 0.05   # every target token decided by far
    hid_d = torch.from_numpy(hidden.astype(np.float32)).cuda().to(s.dm.act_dtype).contiguous()
    draft_d = torch.from_numpy(draft.astype(np.int32)).cuda()
    ws = dfa.verify_hidden_workspace(d, nseq)
    for lens in (None, (np.arange(nseq) % G + 1).astype(np.int32)):
        acc_o, com_o, ids_o, nxt_o = O.verify_from_hidden(hidden, s.w["E_out"], draft.astype(np.int32), lengths=lens)
        if lens is None:
            assert np.array_equal(acc_o, accept)
        acc = torch.empty(nseq, dtype=torch.int32, device="cuda")
        com, nxt = torch.empty_like(acc), torch.empty_like(acc)
        ids = torch.empty(nseq, G + 1, dtype=torch.int32, device="cuda")
        lens_d = None if lens is None else torch.from_numpy(lens).cuda()
        bd.check(dfa.dflash_verify_from_hidden(s.dm, hid_d, draft_d, acc, com, ids, ws, lengths=lens_d,
                                               next_anchor=nxt), "verify_from_hidden")
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_o)
        assert np.array_equal(com.cpu().numpy(), com_o)
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        assert np.array_equal(nxt.cpu().numpy(), nxt_o)
    log(f"[{name}] verify from hidden states, {nseq} sequences: accepted {acc_o.tolist()}")
