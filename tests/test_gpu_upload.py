"""GPU tests of sft_plan_upload: the step's plan, written by the host into
pinned memory, reaches the device byte for byte through the upload kernel on
the caller's stream, for sizes with and without a 4-byte tail, in stream
order with the kernels that read it; bad arguments are refused before any
launch.  Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost
of the Active Set", section 2.6 and Figure 2 (masks shipped to the GPU once
per step).
"""
import numpy as np
import pytest
import torch

from sparse_full_weight_amd import _lib, synth

pytestmark = pytest.mark.gpu


def _pinned_words(n, seed):
    g = synth.rng(seed)
    return torch.from_numpy(g.integers(-2**31, 2**31 - 1, size=n, dtype=np.int64).astype(np.int32)).pin_memory()


@pytest.mark.parametrize("words", [1, 3, 4, 5, 1100, 65536 * 4 + 7])
def test_upload_copies_every_byte(gpu_lib, words):
    src = _pinned_words(words, 500 + words)
    dst = torch.full((words + 8,), -1, dtype=torch.int32, device="cuda")
    _lib.sft_plan_upload(dst, src, 4 * words)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:words], src.numpy())
    assert np.all(got[words:] == -1), "write past the copied bytes"


def test_upload_of_a_prefix_and_zero_bytes(gpu_lib):
    src = _pinned_words(1000, 601)
    dst = torch.full((1000,), 7, dtype=torch.int32, device="cuda")
    _lib.sft_plan_upload(dst, src, 0)
    _lib.sft_plan_upload(dst, src, 4 * 333)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:333], src.numpy()[:333]) and np.all(got[333:] == 7)


def test_upload_in_stream_order_on_a_second_stream(gpu_lib):
    # the upload and a kernel reading its result on another stream, repeated
    # with new host contents each time after the stream has passed the call
    s = torch.cuda.Stream()
    src = _pinned_words(4096, 602)
    dst = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for it in range(5):
        src.copy_(torch.arange(4096, dtype=torch.int32) * (it + 3))
        with torch.cuda.stream(s):
            _lib.sft_plan_upload(dst, src, stream=s)
            tot = dst.to(torch.int64).sum()
        s.synchronize()
        assert int(tot) == (it + 3) * 4095 * 4096 // 2


def test_upload_rejects_bad_arguments(gpu_lib):
    dst = torch.zeros(64, dtype=torch.int32, device="cuda")
    pinned = _pinned_words(64, 603)
    with pytest.raises(TypeError):
        _lib.sft_plan_upload(dst, torch.zeros(64, dtype=torch.int32))          # pageable host memory
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_plan_upload(dst, pinned, 6)                                   # not whole words
    assert e.value.code == _lib.SFT_ESHAPE
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_plan_upload(dst[1:], pinned, 16)                              # dst not 16-byte aligned
    assert e.value.code == _lib.SFT_EALIGN
    with pytest.raises(ValueError):
        _lib.sft_plan_upload(dst, pinned, 4 * 65)                              # beyond the tensors
    # the library's own check: pageable host memory is refused, nothing launched
    host = np.zeros(64, np.int32)
    if host.ctypes.data % 16 == 0:
        rc = _lib.lib().sft_plan_upload(dst.data_ptr(), host.ctypes.data, 64, None)
        assert rc == _lib.SFT_EINVAL
        # and the refusal leaves no error behind for the next runtime call
        torch.zeros(16, device="cuda").add_(1)
        torch.cuda.synchronize()
