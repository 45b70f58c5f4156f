"""GPU parity of the compressed path over a multi-step decode with the Update
Buffer (sparsekv_update_buffer + sparsekv_retrieve + sparsekv_gather_attend)
against the oracle's decode loop: every step's flushes, retrieved ids and
candidate counts identical, attention within 2e-3 on sampled steps, and the
grown index (ids, codes, w, histogram, positions) identical to the oracle's
at the end."""
import dataclasses

import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D
from oracle import lloyd
from oracle import update as U

from gpu_helpers import ATTN_TOL, DEV, say

pytestmark = pytest.mark.gpu


def _decode(p, L0, steps, update, attend_every):
    lv, th = lloyd.codebook_f32(8)
    cb = S.new_codebook(torch.from_numpy(p.signs).to(DEV))
    kvn = p.kv()
    kvn.seq_len = np.array([L0], np.int32)
    kv = S.kv_to_device(kvn, DEV)
    cap = p.L - p.sink - p.local
    index = S.new_index(p.H, cap, device=DEV)
    S.sparsekv_encode(cb, kv, 0, p.sink, L0 - p.local, index)
    ref = U.prefill_index(p, L0, lv, th)
    n = L0 - p.sink - p.local
    # one workspace for the whole loop, sized for the largest index it serves
    big = dataclasses.replace(index, n=cap)
    ws = S.workspace(S.retrieve_workspace_size(big, p.G, p.beta, p.k_final), DEV)
    qs = W.paris_step_queries(p, steps)
    lo = torch.tensor([p.sink], dtype=torch.int32, device=DEV)
    hi = torch.tensor([p.sink + n], dtype=torch.int32, device=DEV)
    total_flushes = 0
    for i in range(steps):
        seq = L0 + 1 + i
        kv.seq_len.fill_(seq)
        f = S.sparsekv_update_buffer(cb, kv, 0, seq, p.sink, p.local, update, index)
        ref, n, f_ref, res = U.decode_step(p, ref, n, seq, qs[i], lv, th, update)
        assert f == f_ref and index.n == n, (i, f, f_ref, index.n, n)
        total_flushes += f
        if f:
            hi.fill_(p.sink + n)
            say("  step", i, "flushed", f, "n", n)
        q = S.to_device(qs[i], DEV, bf16=True)
        idx, n_cand, _ = S.sparsekv_retrieve(cb, index, q, p.G, p.rho, p.beta, p.k_final, ws=ws)
        got_idx, got_nc = idx.cpu().numpy(), n_cand.cpu().numpy()
        for h in range(p.H):
            k = int(got_nc[h])
            assert k == res["idx"][h].size, (i, h)
            assert np.array_equal(np.sort(got_idx[h][:k]), np.sort(res["idx"][h])), (i, h)
            assert np.all(got_idx[h][k:] == -1)
        if i % attend_every == 0 or f:
            out = S.sparsekv_gather_attend(kv, q.view(1, p.H * p.G, p.d), p.G,
                                           idx.view(1, p.H, -1), p.k_final, lo, hi, p.scale)
            out = out.cpu().numpy()[0]
            kvn.seq_len = np.array([seq], np.int32)
            for h in range(p.H):
                o_ref = D.attend_row(kvn, qs[i].reshape(1, p.H * p.G, p.d), p.G, 0, h,
                                     res["idx"][h], p.sink, p.sink + n, p.scale)
                err = np.abs(out[h * p.G:(h + 1) * p.G] - o_ref).max()
                assert err <= ATTN_TOL, (i, h, err)
    torch.cuda.synchronize()
    assert index.n == n
    for key, got in (("ids", index.ids[:, :n]), ("codes", index.codes[:, :n]),
                     ("hist", index.hist), ("pos", index.pos[:n])):
        assert np.array_equal(got.cpu().numpy(), ref[key]), key
    w = index.w[:, :n].cpu().numpy()
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32))
    return total_flushes


def test_decode_loop_with_update_buffer():
    """Prefill 2048 tokens, then 300 decode steps with a 128-token buffer:
    two flushes, every step retrieved from the index as it stands."""
    p = W.make_paris(tag=71, H=2, G=4, L=4096, sink=4, local=64, rho=0.2, beta=0.2)
    say("paris decode", p.name, "L0 2048 steps 300 update 128")
    assert _decode(p, 2048, 300, 128, attend_every=50) == 2


def test_decode_loop_candidate_slices_grow():
    """With beta = 1 every entry is a candidate, and the flush takes C from
    32760 to 32776: the top-k over the candidates goes from one workgroup per
    row to the sliced path and its per-slice table grows (32 -> 33 entries
    per head), moving what follows it in the workspace -- the regions kept
    zero between calls stay at fixed offsets."""
    p = W.make_paris(tag=72, H=8, G=1, L=33000, sink=4, local=32, rho=1.0, beta=1.0)
    say("paris decode", p.name, "L0 32796 steps 24 update 16")
    assert _decode(p, 32796, 24, 16, attend_every=12) == 1


def test_update_buffer_rejects_bad_arguments():
    p = W.make_paris(tag=73, H=1, G=1, L=600, sink=4, local=32)
    cb = S.new_codebook(torch.from_numpy(p.signs).to(DEV))
    kv = S.kv_to_device(p.kv(), DEV)
    index = S.new_index(p.H, 100, device=DEV)
    S.sparsekv_encode(cb, kv, 0, 4, 50, index)
    with pytest.raises(S.SkvError) as e:        # length below the retrieval end
        S.sparsekv_update_buffer(cb, kv, 0, 40, 4, 32, 16, index)
    assert e.value.status == S.SKV_EINVAL
    with pytest.raises(S.SkvError) as e:        # update < 1
        S.sparsekv_update_buffer(cb, kv, 0, 200, 4, 32, 0, index)
    assert e.value.status == S.SKV_EINVAL
    with pytest.raises(S.SkvError) as e:        # the flush would overflow the index
        S.sparsekv_update_buffer(cb, kv, 0, 600, 4, 32, 16, index)
    assert e.value.status == S.SKV_EINVAL and index.n == 46
    assert S.sparsekv_update_buffer(cb, kv, 0, 60, 4, 32, 16, index) == 0
