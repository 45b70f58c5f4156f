"""The streaming-read yardsticks (libskv_yardstick) read every byte once:
each workgroup's folded word equals the XOR of the 16-byte units it owns,
computed here on the host -- for the grid-stride probe (plain and
non-temporal loads) unit u belongs to workgroup (u // 256) % n_wg; for the
4 KB-piece probe the piece at position i of the order belongs to wave
i % (4 n_wg), that is workgroup (i % (4 n_wg)) // 4."""
import numpy as np
import pytest
import torch

from sparse_top_kv_indexer_amd import yardstick as Y

from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("n_units,n_wg", [(1, 1), (1000, 3), (256 * 37 + 5, 8), (1 << 16, 64)])
def test_read_probe_folds_every_word(n_units, n_wg, nt):
    rng = np.random.default_rng(n_units)
    host = rng.integers(0, 2 ** 32, size=(n_units, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    got = Y.read_probe(buf, n_wg, nontemporal=nt).cpu().numpy().view(np.uint32)
    owner = (np.arange(n_units) // 256) % n_wg
    for g in range(n_wg):
        words = host[owner == g].ravel()
        exp = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
        assert got[g] == exp, g


@pytest.mark.parametrize("n_pieces,n_wg", [(1, 1), (37, 2), (1000, 5)])
def test_read_pieces_folds_every_piece_in_its_order(n_pieces, n_wg):
    rng = np.random.default_rng(n_pieces)
    host = rng.integers(0, 2 ** 32, size=(n_pieces, 1024), dtype=np.uint64).astype(np.uint32)
    order = rng.permutation(n_pieces).astype(np.int32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    got = Y.read_pieces(buf, torch.from_numpy(order).to(DEV), n_wg).cpu().numpy().view(np.uint32)
    owner = (np.arange(n_pieces) % (4 * n_wg)) // 4
    for g in range(n_wg):
        words = host[order[owner == g]].ravel()
        exp = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
        assert got[g] == exp, g
