"""The fused decode step without a workspace (sparsekv_select_attend_noalloc,
scratch held by the library) against the same step with a caller workspace
(sparsekv_select_attend), on two calls in a row, the second on a smaller
input, through the C ABI.  Selection and counts must be identical and the
attention within the parity tolerance; the oracle also checks the first
call's selection and output."""
import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D

from gpu_helpers import ATTN_TOL, DEV, say

pytestmark = pytest.mark.gpu


def _upload(st):
    kv = S.kv_to_device(st.kv, DEV)
    q = S.to_device(st.q, DEV, True)
    lo = S.to_device(st.lo.astype(np.int32), DEV)
    hi = S.to_device(st.hi.astype(np.int32), DEV)
    return kv, q, lo, hi


def _outputs(kv, G, k):
    B, H, L = kv.B, kv.H, kv.L_max
    return (torch.empty((B, H, L), dtype=torch.float32, device=DEV),
            torch.full((B, H, k), -7, dtype=torch.int32, device=DEV),
            torch.full((B, H), -7, dtype=torch.int32, device=DEV),
            torch.full((B, H * G, kv.d_v), float("nan"), dtype=torch.float32, device=DEV))


def test_noalloc_matches_workspace_call_twice_second_smaller():
    cases = [W.make_gqa_paged(tag=301, B=4, H=4, G=4, L=8192, k=512, sink=4, local=64),
             W.make_gqa_paged(tag=302, B=2, H=2, G=2, L=4096, k=256, sink=4, local=32)]
    for i, st in enumerate(cases):
        say("noalloc call", i, st.name, "G", st.G, "k", st.k)
        kv, q, lo, hi = _upload(st)
        assert S.sparsekv_select_attend_noalloc_bytes(kv, st.G) <= S.NOALLOC_SCRATCH_BYTES
        sc, idx, cnt, out = _outputs(kv, st.G, st.k)
        S.sparsekv_select_attend_noalloc(kv, q, st.G, lo, hi, st.k, st.scale, sc, idx, cnt, out)
        rsc, ridx, rcnt, rout = S.sparsekv_select_attend(kv, q, st.G, lo, hi, st.k, st.scale)
        torch.cuda.synchronize()
        assert torch.equal(idx, ridx) and torch.equal(cnt, rcnt)
        assert torch.equal(sc, rsc)
        err = float((out - rout).abs().max().item())
        assert err <= ATTN_TOL, err
        say("  max |noalloc - workspace| =", err)
        if i == 0:
            ref = D.step(st)
            got = idx.cpu().numpy()
            for b in range(st.kv.B):
                for h in range(st.kv.H):
                    assert got[b, h].tolist() == sorted(ref["idx"][b, h].tolist()), (b, h)
            assert float(np.abs(out.cpu().numpy() - ref["out"]).max()) <= ATTN_TOL


def test_noalloc_repeated_calls_do_not_carry_state():
    """The scratch keeps the last call's contents: the call must clear what
    has to start at zero, so repeating it gives the same result."""
    st = W.make_gqa_paged(tag=303, B=2, H=4, G=4, L=4096, k=256, sink=4, local=64)
    kv, q, lo, hi = _upload(st)
    first = None
    for rep in range(3):
        sc, idx, cnt, out = _outputs(kv, st.G, st.k)
        S.sparsekv_select_attend_noalloc(kv, q, st.G, lo, hi, st.k, st.scale, sc, idx, cnt, out)
        torch.cuda.synchronize()
        if first is None:
            first = (idx.clone(), out.clone())
        else:
            assert torch.equal(idx, first[0]) and torch.equal(out, first[1]), rep
