"""The benchmark's HBM stream probe (libkvsel_probe.so, not part of the
method) on the GPU: the copy mode copies exactly, and the read mode's
per-workgroup folds XOR to the XOR of every 16-byte word of the source, for a
buffer larger than one pass of the grid and for one smaller than a single
workgroup's share."""
import numpy as np
import pytest
import torch

from sparse_decode_attention_window_amd import _probe as probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [(1 << 23) + 48, 48])
def test_hbm_probe_copy_and_read_fold(nbytes):
    print(f"[probe] nbytes {nbytes}", flush=True)
    g = torch.Generator().manual_seed(nbytes % 1000)
    src_h = torch.randint(-(2 ** 31), 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    src = src_h.cuda()
    dst = torch.full_like(src, -1)
    probe.probe_stream(probe.PROBE_COPY, src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src_h)

    fold = torch.full((probe.PROBE_BLOCKS * 4,), -1, dtype=torch.int32, device="cuda")
    probe.probe_stream(probe.PROBE_READ, src, fold, nbytes)
    torch.cuda.synchronize()
    words = fold.cpu().numpy().view(np.uint32).reshape(-1, 4)
    expect = np.bitwise_xor.reduce(src_h.numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(np.bitwise_xor.reduce(words, axis=0), expect)
