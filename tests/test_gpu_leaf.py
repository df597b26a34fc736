"""GPU parity of the SparseLeaf calls (blog post "SparseLeaf: synaptic sparse
fine-tuning"): the gradients of K selected connections (sft_leaf_grad)
against the oracle's fp64 dot products, within the masked-dW tolerance and
bit for bit on integer-valued inputs; the coordinate Adam step
(sft_leaf_adam) bit for bit against the oracle given the same gradients."""
import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import _lib, synth
from tests.gpu_helpers import adam_dev, bf16_dev, dev, dw_close, host_u16

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _coords(m, n, K, seed):
    g = synth.rng(seed)
    flat = np.sort(g.choice(m * n, size=K, replace=False))
    return (flat // n).astype(np.int32), (flat % n).astype(np.int32)


def _case(T, m, n, K, seed, integer=False):
    if integer:
        D = synth.integer_bf16((T, m), -3, 3, seed)
        X = synth.integer_bf16((T, n), -3, 3, seed + 1)
    else:
        D = synth.normal_bf16((T, m), 0.01, seed)
        X = synth.normal_bf16((T, n), 1.0, seed + 1)
    rows, cols = _coords(m, n, K, seed + 2)
    return D, X, rows, cols


def _run(cases):
    mats = []
    for D, X, rows, cols in cases:
        mats.append(_lib.LeafMat(bf16_dev(D), bf16_dev(X), dev(rows), dev(cols),
                                 torch.full((max(rows.size, 1),), float("nan"), dtype=torch.float32, device="cuda")
                                 [: rows.size]))
    ws = torch.zeros(max(_lib.sft_leaf_grad_workspace(mats) // 4, 1), dtype=torch.int32, device="cuda")
    _lib.sft_leaf_grad(mats, ws)
    torch.cuda.synchronize()
    return [m.grad.cpu().numpy() for m in mats], mats, ws


def _close(got, want):
    if want.size:
        dw_close(got[None, :], want[None, :])


def test_leaf_grad_matches_oracle():
    # ragged token count (not a multiple of any LDS batch), several shapes in
    # one call, one matrix with more coordinates than one pass holds
    T = 300
    cases = [_case(T, 64, 40, 500, 10), _case(T, 264, 128, 3000, 20), _case(T, 512, 520, 40000, 30),
             _case(T, 8, 8, 64, 40)]
    got, _, _ = _run(cases)
    for g, (D, X, rows, cols) in zip(got, cases):
        _close(g, oracle.leaf_grad(D, X, rows, cols))


@pytest.mark.parametrize("K,width", [(10000, 12), (15000, 16), (19000, 20), (23000, 24), (27000, 28)])
def test_leaf_grad_every_kernel_width(K, width):
    # one 256 x 256 matrix per call: the planner takes the width (coordinates
    # per lane and pass, of 12, 16, 20, 24, 28) with the least slot work, which
    # for (width - 4) * 1024 < K <= width * 1024 is `width` (one pass; the
    # next smaller width would take two)
    case = _case(70, 256, 256, K, 200 + width)
    got, _, _ = _run([case])
    D, X, rows, cols = case
    _close(got[0], oracle.leaf_grad(D, X, rows, cols))


def test_leaf_grad_integer_inputs_bit_exact():
    T = 257
    cases = [_case(T, 96, 72, 2000, 50, integer=True), _case(T, 512, 520, 36000, 60, integer=True)]
    got, _, _ = _run(cases)
    for g, (D, X, rows, cols) in zip(got, cases):
        assert np.array_equal(g, oracle.leaf_grad(D, X, rows, cols))


def test_leaf_grad_widest_rows_and_repeat():
    # m + n = 15104 (the MLP shapes of a 7B layer): two tokens per LDS batch;
    # a second call gives the same bits
    cases = [_case(37, 11008, 4096, 1500, 70), _case(37, 4096, 11008, 1500, 80)]
    got, mats, ws = _run(cases)
    for g, (D, X, rows, cols) in zip(got, cases):
        _close(g, oracle.leaf_grad(D, X, rows, cols))
    _lib.sft_leaf_grad(mats, ws)
    torch.cuda.synchronize()
    for g, m in zip(got, mats):
        assert np.array_equal(g.view(np.uint32), m.grad.cpu().numpy().view(np.uint32))


def test_leaf_grad_one_token_and_no_tokens_and_empty():
    one = [_case(1, 40, 24, 200, 90), _case(1, 16, 16, 0, 91)]
    got, _, _ = _run(one)
    D, X, rows, cols = one[0]
    assert np.array_equal(got[0], oracle.leaf_grad(D, X, rows, cols))   # bf16 x bf16 is exact in fp32
    zero = [_case(0, 40, 24, 200, 92)]
    got, _, _ = _run(zero)
    assert np.array_equal(got[0], np.zeros(200, np.float32))


def test_leaf_grad_rejects_bad_shapes():
    D, X, rows, cols = _case(16, 12, 16, 10, 95)
    m = _lib.LeafMat(bf16_dev(D), bf16_dev(X), dev(rows), dev(cols), torch.zeros(10, device="cuda"))
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_leaf_grad_workspace([m])
    assert e.value.code == _lib.SFT_EINVAL or e.value.code == _lib.SFT_ESHAPE
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_leaf_grad([m], torch.zeros(1024, dtype=torch.int32, device="cuda"))
    assert e.value.code == _lib.SFT_ESHAPE
    D, X, rows, cols = _case(16, 32768, 8, 10, 96)
    big = _lib.LeafMat(bf16_dev(D), bf16_dev(X), dev(rows), dev(cols), torch.zeros(10, device="cuda"))
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_leaf_grad([big], torch.zeros(1024, dtype=torch.int32, device="cuda"))
    assert e.value.code == _lib.SFT_ENOTSUP


def test_leaf_adam_matches_oracle_over_steps():
    Ks = [1, 700, 5000, 0, 33]
    rng = np.random.default_rng(100)
    hp = adam_dev(**HP)
    vecs, host = [], []
    for K in Ks:
        st = [np.zeros(K, np.float32) for _ in range(3)]
        bf = np.zeros(K, np.uint16)
        vecs.append(_lib.LeafVec(torch.zeros(max(K, 1), device="cuda")[:K], dev(st[0]), dev(st[1]), dev(st[2]),
                                 torch.zeros(max(K, 1), dtype=torch.int16, device="cuda")[:K]))
        host.append((st, bf))
    for step in range(1, 5):
        gs = []
        for K, v in zip(Ks, vecs):
            g = (rng.standard_normal(K) * 10.0 ** rng.uniform(-5, 0, K)).astype(np.float32)
            if K > 3:
                g[:3] = [0.0, -0.0, 1e-30]
            v.grad.copy_(torch.from_numpy(g))
            gs.append(g)
        _lib.sft_leaf_adam(vecs, step, hp)
        torch.cuda.synchronize()
        for i, (g, (st, bf), v) in enumerate(zip(gs, host, vecs)):
            oracle.leaf_adam(g, st[0], st[1], st[2], bf, step, **HP)
            for name, a, b in (("theta", v.theta, st[0]), ("m", v.m, st[1]), ("v", v.v, st[2])):
                assert np.array_equal(a.cpu().numpy().view(np.uint32), b.view(np.uint32)), (step, i, name)
            assert np.array_equal(host_u16(v.theta_bf16), bf), (step, i, "theta_bf16")


def test_leaf_adam_rejects_bad_step_and_decay():
    K = 8
    v = _lib.LeafVec(torch.zeros(K, device="cuda"), torch.zeros(K, device="cuda"), torch.zeros(K, device="cuda"),
                     torch.zeros(K, device="cuda"))
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_leaf_adam([v], 0, adam_dev(**HP))
    assert e.value.code == _lib.SFT_EINVAL
    with pytest.raises(_lib.SftError) as e:
        _lib.sft_leaf_adam([v], 1, adam_dev(weight_decay=0.01, **HP))
    assert e.value.code == _lib.SFT_EINVAL
