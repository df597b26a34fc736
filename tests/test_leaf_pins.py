"""Pins of the oracle's SparseLeaf functions (blog post "SparseLeaf: synaptic
sparse fine-tuning", sections "Weight gradients: write the selected results
directly" and "The optimizer"): the connection gradients against numpy's
float64 product of the whole matrices, exact integer cases, the diagonal
support and one-token outer products; the coordinate Adam step against its
closed first step and against torch.optim.Adam."""
import numpy as np
import pytest
import torch

import oracle
from sparse_full_weight_amd import synth


def _f32(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _coords(m, n, K, seed):
    g = synth.rng(seed)
    flat = np.sort(g.choice(m * n, size=K, replace=False))
    return (flat // n).astype(np.int32), (flat % n).astype(np.int32)


def test_leaf_grad_matches_full_product_at_the_coordinates():
    T, m, n = 96, 40, 56
    D = synth.normal_bf16((T, m), 0.01, 1)
    X = synth.normal_bf16((T, n), 1.0, 2)
    rows, cols = _coords(m, n, 300, 3)
    full = _f32(D).T @ _f32(X)
    want = full[rows, cols]
    got = oracle.leaf_grad(D, X, rows, cols)
    # both are fp64 sums rounded once; only the summation order differs
    assert np.allclose(got, want, rtol=1e-6, atol=1e-9)


def test_leaf_grad_integer_inputs_are_exact():
    T, m, n = 200, 24, 32
    D = synth.integer_bf16((T, m), -4, 4, 4)
    X = synth.integer_bf16((T, n), -4, 4, 5)
    rows, cols = _coords(m, n, 150, 6)
    want = (_f32(D).T @ _f32(X))[rows, cols].astype(np.float32)
    assert np.array_equal(oracle.leaf_grad(D, X, rows, cols), want)


def test_leaf_grad_diagonal_support_is_the_diagonal():
    T, m = 64, 48
    D = synth.normal_bf16((T, m), 0.01, 7)
    X = synth.normal_bf16((T, m), 1.0, 8)
    idx = np.arange(m, dtype=np.int32)
    want = np.einsum("ti,ti->i", _f32(D), _f32(X)).astype(np.float32)
    assert np.allclose(oracle.leaf_grad(D, X, idx, idx), want, rtol=1e-6, atol=1e-9)


def test_leaf_grad_one_token_is_the_outer_product():
    D = synth.normal_bf16((1, 10), 0.01, 9)
    X = synth.normal_bf16((1, 12), 1.0, 10)
    rows, cols = _coords(10, 12, 30, 11)
    want = (_f32(D)[0, rows] * _f32(X)[0, cols]).astype(np.float32)   # bf16 x bf16 is exact in fp32
    assert np.array_equal(oracle.leaf_grad(D, X, rows, cols), want)


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def test_leaf_adam_first_step_closed_form():
    # from zero state: m = (1-b1) g, v = (1-b2) g^2, mhat ~ g, vhat ~ g^2, so
    # theta = -lr * g / (|g| + eps) to within a few ulp
    g = np.array([1e-3, -2e-2, 5.0, -7e-5, 0.0], np.float32)
    th, m, v = (np.zeros(5, np.float32) for _ in range(3))
    bf = np.zeros(5, np.uint16)
    oracle.leaf_adam(g, th, m, v, bf, 1, **HP)
    want = -HP["lr"] * g.astype(np.float64) / (np.abs(g) + HP["eps"])
    assert np.allclose(th, want, rtol=1e-5, atol=0)
    assert th[4] == 0.0 and m[4] == 0.0 and v[4] == 0.0
    assert np.array_equal(bf, oracle.f32_to_bf16(th))


def test_leaf_adam_matches_torch_adam_over_steps():
    K = 257
    rng = np.random.default_rng(12)
    th, m, v = (np.zeros(K, np.float32) for _ in range(3))
    p = torch.zeros(K, dtype=torch.float32, requires_grad=True)
    opt = torch.optim.Adam([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"])
    for step in range(1, 8):
        g = (rng.standard_normal(K) * 10.0 ** rng.uniform(-4, 0, K)).astype(np.float32)
        oracle.leaf_adam(g, th, m, v, None, step, **HP)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        ref = p.detach().numpy()
        # torch folds the bias corrections differently: a few ulp of each step,
        # which is lr in size (theta near zero after cancellation keeps that
        # absolute error)
        assert np.allclose(th, ref, rtol=1e-5, atol=1e-6 * HP["lr"]), step


@pytest.mark.parametrize("step", [1, 5, 100])
def test_leaf_adam_zero_gradient_zero_state_stays_zero(step):
    th, m, v = (np.zeros(9, np.float32) for _ in range(3))
    oracle.leaf_adam(np.zeros(9, np.float32), th, m, v, None, step, **HP)
    assert not th.any() and not m.any() and not v.any()
