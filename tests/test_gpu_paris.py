"""GPU parity of ParisKV compressed-code retrieval (encode bit-exact; votes,
candidates, rerank estimates and the final top-k identical) against the fp32
oracle, plus attention over the retrieved set."""
import dataclasses

import numpy as np
import pytest
import torch

import sparse_top_kv_indexer_amd as S
import workloads as W
from oracle import dense as D
from oracle import lloyd
from oracle import paris as P

from gpu_helpers import ATTN_TOL, DEV, say

pytestmark = pytest.mark.gpu


def _gpu_index(p, cb):
    kv = S.kv_to_device(p.kv(), DEV)
    index = S.new_index(p.H, p.n + 7, device=DEV)
    S.sparsekv_encode(cb, kv, 0, p.sink, p.L - p.local, index)
    torch.cuda.synchronize()
    return kv, index


def _codebook(p):
    cb = S.new_codebook(torch.from_numpy(p.signs).to(DEV))
    lv, th = lloyd.codebook_f32(8)
    assert cb.levels.view(np.uint32).tolist() == lv.view(np.uint32).tolist()
    return cb, lv, th


@pytest.mark.parametrize("L,tag", [(3000, 11), (9000, 12)])
def test_encode_bit_exact(L, tag):
    p = W.make_paris(tag=tag, H=2, G=4, L=L, sink=4, local=64)
    say("encode", p.name, "n", p.n)
    cb, lv, th = _codebook(p)
    _, index = _gpu_index(p, cb)
    ref = P.build_index(p, lv, th)
    n = p.n
    assert index.n == n
    ids = index.ids[:, :n].cpu().numpy()
    codes = index.codes[:, :n].cpu().numpy()
    w = index.w[:, :n].cpu().numpy()
    assert np.array_equal(ids, ref["ids"])
    assert np.array_equal(codes, ref["codes"])
    bad = (w.view(np.uint32) != ref["w"].view(np.uint32))
    assert not bad.any(), (int(bad.sum()), w[bad][:4], ref["w"][bad][:4])
    assert np.array_equal(index.hist.cpu().numpy(), ref["hist"])
    assert np.array_equal(index.pos[:n].cpu().numpy(), ref["pos"])


def test_encode_appends_in_pieces():
    """Two appends give the same index as one."""
    p = W.make_paris(tag=13, H=2, G=4, L=5000, sink=4, local=64)
    cb, lv, th = _codebook(p)
    kv = S.kv_to_device(p.kv(), DEV)
    index = S.new_index(p.H, p.n, device=DEV)
    mid = 1234
    S.sparsekv_encode(cb, kv, 0, p.sink, mid, index)
    S.sparsekv_encode(cb, kv, 0, mid, p.L - p.local, index)
    ref = P.build_index(p, lv, th)
    assert index.n == p.n
    assert np.array_equal(index.ids.cpu().numpy(), ref["ids"])
    assert np.array_equal(index.w.cpu().numpy().view(np.uint32), ref["w"].view(np.uint32))
    assert np.array_equal(index.hist.cpu().numpy(), ref["hist"])
    with pytest.raises(S.SkvError):
        S.sparsekv_encode(cb, kv, 0, 4, 10, index)          # index is full


def _check_retrieval(p, ref, idx, n_cand, tr):
    votes, cand, est = (tr["votes"].cpu().numpy(), tr["cand"].cpu().numpy(),
                        tr["est"].cpu().numpy())
    idx, n_cand = idx.cpu().numpy(), n_cand.cpu().numpy()
    for h in range(p.H):
        assert np.array_equal(votes[h], ref["S"][h]), h
        assert np.array_equal(cand[h], ref["cand"][h]), h
        assert np.array_equal(est[h].view(np.uint32), ref["est"][h].view(np.uint32)), h
        assert n_cand[h] == len(ref["idx"][h])
        assert idx[h][: n_cand[h]].tolist() == sorted(ref["idx"][h].tolist()), h
        assert np.all(idx[h][n_cand[h]:] == -1)


@pytest.mark.parametrize("L,tag,beta,k_final", [(6000, 21, 0.05, 100), (20000, 22, 0.02, 100),
                                                (3000, 23, 1.0, 64), (9000, 29, 1.0, 5000)])
def test_retrieve_identical(L, tag, beta, k_final):
    p = W.make_paris(tag=tag, H=2, G=4, L=L, sink=4, local=64, beta=beta, rho=beta,
                     k_final=k_final)
    say("retrieve", p.name, "n", p.n, "beta", beta)
    cb, lv, th = _codebook(p)
    _, index = _gpu_index(p, cb)
    q = S.to_device(p.q, DEV, bf16=True)
    idx, n_cand, tr = S.sparsekv_retrieve(cb, index, q, p.G, p.rho, p.beta, p.k_final, trace=True)
    torch.cuda.synchronize()
    ref_index = P.build_index(p, lv, th)
    ref = P.retrieve(p, ref_index, lv)
    votes, cand, est = (tr["votes"].cpu().numpy(), tr["cand"].cpu().numpy(),
                        tr["est"].cpu().numpy())
    idx, n_cand = idx.cpu().numpy(), n_cand.cpu().numpy()
    true = P.exact_top(p, 100)
    for h in range(p.H):
        assert np.array_equal(votes[h], ref["S"][h]), h
        assert np.array_equal(cand[h], ref["cand"][h]), h
        assert np.array_equal(est[h].view(np.uint32), ref["est"][h].view(np.uint32)), h
        got = idx[h][: n_cand[h]]
        assert n_cand[h] == len(ref["idx"][h])
        assert got.tolist() == sorted(ref["idx"][h].tolist()), h
        assert np.all(idx[h][n_cand[h]:] == -1)
        say("  h", h, "recall@100", P.recall_at(got, true[h]))


@pytest.mark.parametrize("G,L,tag,beta,rho", [(1, 17000, 24, 0.03, 0.1), (3, 26000, 25, 0.02, 0.02),
                                              (2, 9000, 26, 0.2, 0.5)])
def test_retrieve_group_sizes_and_chunk_tails(G, L, tag, beta, rho):
    """G < 4 leaves bytes of the packed tier table unused; n spans several
    8192-entry vote chunks with a ragged last one."""
    p = W.make_paris(tag=tag, H=3, G=G, L=L, sink=4, local=64, beta=beta, rho=rho, k_final=100)
    say("retrieve", p.name, "G", G, "n", p.n, "beta", beta, "rho", rho)
    cb, lv, th = _codebook(p)
    _, index = _gpu_index(p, cb)
    q = S.to_device(p.q, DEV, bf16=True)
    idx, n_cand, tr = S.sparsekv_retrieve(cb, index, q, p.G, p.rho, p.beta, p.k_final, trace=True)
    torch.cuda.synchronize()
    ref = P.retrieve(p, P.build_index(p, lv, th), lv)
    _check_retrieval(p, ref, idx, n_cand, tr)


def test_retrieve_repeated_on_one_workspace():
    """Calls that share a workspace: the vote totals are left zero by every
    call, so a second call (another query, a smaller beta) on the same
    workspace gives its own exact result."""
    p = W.make_paris(tag=27, H=2, G=4, L=20000, sink=4, local=64, beta=0.05, rho=0.05)
    cb, lv, th = _codebook(p)
    _, index = _gpu_index(p, cb)
    ref_index = P.build_index(p, lv, th)
    ws = S.workspace(S.retrieve_workspace_size(index, p.G, 0.05, p.k_final), DEV)
    for call, (tag_q, beta) in enumerate([(27, 0.05), (28, 0.02), (27, 0.05)]):
        pq = W.make_paris(tag=tag_q, H=2, G=4, L=20000, sink=4, local=64, beta=beta, rho=beta)
        pc = dataclasses.replace(p, q=pq.q, beta=beta, rho=beta)
        say("call", call, "query tag", tag_q, "beta", beta)
        q = S.to_device(pc.q, DEV, bf16=True)
        idx, n_cand, tr = S.sparsekv_retrieve(cb, index, q, pc.G, pc.rho, pc.beta, pc.k_final,
                                              trace=True, ws=ws)
        torch.cuda.synchronize()
        _check_retrieval(pc, P.retrieve(pc, ref_index, lv), idx, n_cand, tr)
    # kept zero between calls: the vote totals [H][98] i32, then the top-k
    # histograms [H][4096] u32 and list counters (one 256-byte line per head)
    al = lambda x: (x + 255) // 256 * 256
    w = ws.view(torch.uint8).cpu().numpy()
    assert not w[: al(p.H * 98 * 4) + al(p.H * 4096 * 4) + p.H * 256].any()


def test_attention_over_retrieved_set():
    p = W.make_paris(tag=31, H=2, G=4, L=12000, sink=4, local=512)
    cb, lv, th = _codebook(p)
    kv, index = _gpu_index(p, cb)
    q = S.to_device(p.q, DEV, bf16=True)
    idx, n_cand, _ = S.sparsekv_retrieve(cb, index, q, p.G, p.rho, p.beta, p.k_final)
    lo = torch.tensor([p.sink], dtype=torch.int32, device=DEV)
    hi = torch.tensor([p.L - p.local], dtype=torch.int32, device=DEV)
    out = S.sparsekv_gather_attend(kv, q.view(1, p.H * p.G, p.d), p.G, idx.view(1, p.H, -1),
                                   p.k_final, lo, hi, p.scale)
    out = out.cpu().numpy()[0]
    ref = P.retrieve(p, P.build_index(p, lv, th), lv)
    kvn = p.kv()
    qn = p.q.reshape(1, p.H * p.G, p.d)
    for h in range(p.H):
        o = D.attend_row(kvn, qn, p.G, 0, h, ref["idx"][h], p.sink, p.L - p.local, p.scale)
        err = np.abs(out[h * p.G:(h + 1) * p.G] - o).max()
        assert err <= ATTN_TOL, (h, err)


@pytest.mark.slow
def test_full_size_against_stored_oracle_results():
    """The full compressed-code workload (8 x 1,048,576 keys): GPU encode and
    retrieval against the oracle's results stored by
    tests/golden/make_paris_full.py (votes, candidate set and rerank
    estimates by hash, final ids, attention outputs)."""
    import hashlib
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "paris_full_expected.json")))
    p = W.make_paris()
    assert p.n == gold["n"]
    cb, lv, th = _codebook(p)
    assert lv.view(np.uint32).tolist() == gold["levels_bits"]
    kv, index = _gpu_index(p, cb)
    q = S.to_device(p.q, DEV, bf16=True)
    idx, n_cand, tr = S.sparsekv_retrieve(cb, index, q, p.G, p.rho, p.beta, p.k_final, trace=True)
    lo = torch.tensor([p.sink], dtype=torch.int32, device=DEV)
    hi = torch.tensor([p.L - p.local], dtype=torch.int32, device=DEV)
    out = S.sparsekv_gather_attend(kv, q.view(1, p.H * p.G, p.d), p.G, idx.view(1, p.H, -1),
                                   p.k_final, lo, hi, p.scale)
    torch.cuda.synchronize()
    sha = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    idx, n_cand, out = idx.cpu().numpy(), n_cand.cpu().numpy(), out.cpu().numpy()[0]
    hist = index.hist.cpu().numpy()
    for h, g in enumerate(gold["heads"]):
        say("head", h)
        assert sha(hist[h].astype(np.int32)) == g["index_hist_sha256"]
        for e, smp in g["samples"].items():
            e = int(e)
            assert index.ids[h, e].cpu().numpy().tolist() == smp["ids"]
            assert index.codes[h, e].cpu().numpy().tolist() == smp["codes"]
            assert index.w[h, e].cpu().numpy().view(np.uint32).tolist() == smp["w_bits"]
        votes = tr["votes"][h].cpu().numpy()
        assert np.bincount(votes, minlength=97).tolist() == g["vote_hist"]
        assert sha(votes) == g["votes_sha256"]
        assert sha(tr["cand"][h].cpu().numpy().astype(np.int32)) == g["cand_sha256"]
        assert sha(tr["est"][h].cpu().numpy().astype(np.float32)) == g["est_sha256"]
        assert n_cand[h] == g["n_cand"]
        assert idx[h][: n_cand[h]].tolist() == g["idx"]
        err = np.abs(out[h * p.G:(h + 1) * p.G] - np.array(g["out"])).max()
        assert err <= ATTN_TOL, (h, err)
        say("  recall@100 (oracle and GPU)", g["recall_at_100"])


@pytest.mark.slow
@pytest.mark.parametrize("rho", [0.05, 0.10])
def test_full_size_larger_tier_budgets_against_stored_oracle_results(rho):
    """The full workload retrieved with tier budgets rho = 0.05 and 0.10
    (beta = 0.02 unchanged): votes, candidates and estimates by hash and the
    final ids equal the oracle's stored by tests/golden/make_paris_full.py, so
    recall@100 is the oracle's."""
    import hashlib
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "paris_full_expected.json")))
    heads = gold["by_rho"][repr(rho)]
    p = W.make_paris()
    cb, lv, th = _codebook(p)
    kv, index = _gpu_index(p, cb)
    q = S.to_device(p.q, DEV, bf16=True)
    idx, n_cand, tr = S.sparsekv_retrieve(cb, index, q, p.G, rho, p.beta, p.k_final, trace=True)
    torch.cuda.synchronize()
    sha = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    idx, n_cand = idx.cpu().numpy(), n_cand.cpu().numpy()
    for h, g in enumerate(heads):
        assert sha(tr["votes"][h].cpu().numpy()) == g["votes_sha256"], h
        assert sha(tr["cand"][h].cpu().numpy().astype(np.int32)) == g["cand_sha256"], h
        assert sha(tr["est"][h].cpu().numpy().astype(np.float32)) == g["est_sha256"], h
        assert idx[h][: n_cand[h]].tolist() == g["idx"], h
    say("  rho", rho, "mean recall@100 (oracle and GPU)",
        sum(g["recall_at_100"] for g in heads) / len(heads))
