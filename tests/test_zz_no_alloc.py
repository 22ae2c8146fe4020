"""The verify entry point without a workspace against the one with a
workspace, through the C ABI: two calls in a row, the second with a smaller
input (the device scratch array keeps the first call's partial results), each
bit-exact against the workspace entry point and against the oracle."""

import numpy as np
import pytest
import torch

from block_diffusion_draft_tap_amd import binding as bd
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


def _planted(B, G, V, seed):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, V, size=(B, G + 1))
    draft = np.empty((B, G), dtype=np.int32)
    for b in range(B):
        a = int(rng.integers(0, G + 1))            # accepted prefix of this sequence
        for k in range(G):
            draft[b, k] = t[b, k] if k < a else (t[b, k] + 1 + rng.integers(0, V - 1)) % V
    T = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    T[np.arange(B)[:, None], np.arange(G + 1)[None, :], t] = T.max(axis=2) + 1.0
    return T, draft


def _outputs(B, G):
    z = lambda *s: torch.full(s, -7, dtype=torch.int32, device="cuda")
    return z(B), z(B), z(B, G + 1), z(B)


def test_verify_noalloc_matches_workspace_entry_point():
    for (B, G, V) in ((16, 7, 151936), (3, 4, 5001)):    # the second call is smaller
        T, draft = _planted(B, G, V, seed=B * 1000 + V)
        T_d, dr_d = torch.from_numpy(T).cuda(), torch.from_numpy(draft).cuda()
        assert bd.lib.dflash_verify_workspace_bytes(B, G, V) <= bd.lib.dflash_verify_noalloc_max_bytes()
        acc, com, ids, nxt = _outputs(B, G)
        ws = bd.verify_workspace(B, G, V)
        bd.check(bd.dflash_verify_greedy(T_d, dr_d, acc, com, ids, ws, next_anchor=nxt), "verify")
        acc2, com2, ids2, nxt2 = _outputs(B, G)
        rc = bd.lib.dflash_verify_greedy_noalloc(T_d.data_ptr(), dr_d.data_ptr(), B, G, V, acc2.data_ptr(),
                                                 com2.data_ptr(), ids2.data_ptr(), nxt2.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
        assert rc == bd.DFLASH_OK, bd.status_string(rc)
        torch.cuda.synchronize()
        for a, b in ((acc, acc2), (com, com2), (ids, ids2), (nxt, nxt2)):
            assert torch.equal(a, b)
        acc_o, com_o, ids_o, nxt_o = O.verify_greedy(T, draft)
        assert np.array_equal(acc2.cpu().numpy(), acc_o) and np.array_equal(com2.cpu().numpy(), com_o)
        assert np.array_equal(ids2.cpu().numpy(), ids_o) and np.array_equal(nxt2.cpu().numpy(), nxt_o)
