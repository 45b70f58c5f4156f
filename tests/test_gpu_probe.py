"""The streaming-read yardstick (skv_read_probe, libskv_yardstick) reads every byte once:
each workgroup's folded word equals the XOR of the 16-byte units it owns
(unit u belongs to workgroup (u // 256) % n_wg), computed here on the host."""
import numpy as np
import pytest
import torch

from sparse_top_kv_indexer_amd import yardstick as Y

from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_units,n_wg", [(1, 1), (1000, 3), (256 * 37 + 5, 8), (1 << 16, 64)])
def test_read_probe_folds_every_word(n_units, n_wg):
    rng = np.random.default_rng(n_units)
    host = rng.integers(0, 2 ** 32, size=(n_units, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    got = Y.read_probe(buf, n_wg).cpu().numpy().view(np.uint32)
    owner = (np.arange(n_units) // 256) % n_wg
    for g in range(n_wg):
        words = host[owner == g].ravel()
        exp = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
        assert got[g] == exp, g
