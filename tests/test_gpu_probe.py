"""The streaming-read probe (kvc_read_probe, a measurement aid): every workgroup's word is the
xor of the 32-bit words of its contiguous share of the buffer, read forwards or backwards, for
shares that do not fill the last load batch and for grids whose last workgroups get nothing."""
import numpy as np
import pytest
import torch

from compressed_decode_attention_gqa_amd import kvc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_vec,grid", [(1000, 1), (1000, 3), (4099, 7), (5, 8), (70000, 64)])
@pytest.mark.parametrize("reverse", [False, True])
def test_read_probe_reads_each_share_once(n_vec, grid, reverse):
    rng = np.random.default_rng(n_vec + grid)
    words = rng.integers(0, 1 << 32, size=4 * n_vec, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.full((grid,), -1, dtype=torch.int32, device="cuda")
    kvc.kvc_read_probe(buf, grid, sink, reverse=reverse)
    got = sink.cpu().numpy().view(np.uint32)
    per = (n_vec + grid - 1) // grid
    for b in range(grid):
        lo, hi = min(n_vec, b * per), min(n_vec, (b + 1) * per)
        want = np.bitwise_xor.reduce(words[4 * lo:4 * hi]) if hi > lo else np.uint32(0)
        assert got[b] == want, (b, lo, hi)
