"""The measurement probes compute what they claim: the read probe folds the
whole buffer (XOR of its sink = XOR of the buffer's 32-bit words), the copy
probe copies it, and the matrix-core probe's sums equal the closed form
4 * iters for inputs of 1/16 (sft.h, measurement probes)."""
import numpy as np
import pytest
import torch

from sparse_full_weight_amd import _lib

pytestmark = pytest.mark.gpu


def test_probe_read_folds_every_word():
    n = (1 << 20) + 4 * 37          # not a multiple of the grid's stride
    host = np.random.default_rng(1).integers(0, 2 ** 32, size=n, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(_lib.sft_probe_grid() * 256, dtype=torch.int32, device="cuda")
    _lib.prepare_probe_read(buf, sink)()
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)


def test_probe_copy_copies():
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, ((1 << 20) + 12,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    _lib.prepare_probe_copy(src, dst)()
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_mfma_closed_form():
    out = torch.zeros(_lib.sft_probe_grid() * 256, dtype=torch.float32, device="cuda")
    _lib.prepare_probe_mfma(1000, out)()
    torch.cuda.synchronize()
    assert torch.all(out == 4000.0)
