"""Pins for the oracle's backward pass (dQ, dK, dV).  CPU only.

The pages define only the forward; the backward is the gradient of that
definition.  It is pinned against three things other than itself: central
finite differences of the oracle's forward, autograd through a dense masked
softmax in fp64, and identities that the chain rule fixes.
"""
import numpy as np
import pytest
import torch

import oracle

SPECS = [
    "causal;window=5",
    "causal;window=3;stride=4;phase=1;global=2",
    "bidir;radius=2;stride=6;global=0:2",
    "causal;window=4;dilation=2",
    "blocks;block=4;radius=1;random=2;seed=3;global=0",
]


def _grid(shape, seed, step=2.0 ** -8):
    """N(0,1) values rounded to multiples of `step`, so x +- step is exact in
    fp32 and the finite differences see exactly the perturbation asked for."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) / step).round() * step


def _loss(spec, q, k, v, g):
    O, _, _ = oracle.forward_rows(spec, q, k, v)
    return float((O * g.double().numpy()).sum())


@pytest.mark.parametrize("spec", SPECS)
def test_backward_matches_finite_differences(spec):
    """L = sum(dO * O): dL/dx by central differences (step 2^-8) on a sample
    of elements of Q, K and V."""
    B, H, T, d = 1, 1, 12, 4
    q, k, v, g = (_grid((B, H, T, d), s) for s in (1, 2, 3, 4))
    dq, dk, dv = oracle.backward(spec, q, k, v, g)
    h = 2.0 ** -8
    rng = np.random.default_rng(0)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            t, c = int(rng.integers(T)), int(rng.integers(d))
            xp, xm = x.clone(), x.clone()
            xp[0, 0, t, c] += h
            xm[0, 0, t, c] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num = (_loss(spec, args_p["q"], args_p["k"], args_p["v"], g)
                   - _loss(spec, args_m["q"], args_m["k"], args_m["v"], g)) / (2 * h)
            assert abs(num - grad[0, 0, t, c]) <= 1e-4 * (1 + abs(num)), (name, t, c)


@pytest.mark.parametrize("spec", SPECS)
def test_backward_matches_autograd_of_dense_masked_softmax(spec):
    T, d = 23, 8
    q, k, v, g = (_grid((2, 2, T, d), s) for s in (5, 6, 7, 8))
    dq, dk, dv = oracle.backward(spec, q, k, v, g)
    mask = torch.from_numpy(oracle.dense_mask(spec, T))
    Q, K, V = (x.double().requires_grad_() for x in (q, k, v))
    s = torch.matmul(Q, K.transpose(-1, -2)) / np.sqrt(d)
    O = torch.matmul(torch.softmax(s.masked_fill(~mask, float("-inf")), -1), V)
    O.backward(g.double())
    for got, ref in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("spec", SPECS + ["causal", "bidir"])
def test_backward_identities(spec):
    """Each row's weights sum to one, so sum_j ds_ij = 0: the key gradients of
    a head sum to zero and the value gradients sum to the upstream ones."""
    q, k, v, g = (_grid((1, 3, 31, 8), s) for s in (9, 10, 11, 12))
    dq, dk, dv = oracle.backward(spec, q, k, v, g)
    assert np.abs(dk.sum(2)).max() < 1e-12
    assert np.allclose(dv.sum(2), g.double().numpy().sum(2), atol=1e-12)


def test_window_one_passes_values_through():
    """w = 1: every query reads only itself with weight 1, so O = V, dV = dO
    and the score gradients vanish."""
    q, k, v, g = (_grid((1, 2, 17, 8), s) for s in (13, 14, 15, 16))
    dq, dk, dv = oracle.backward("causal;window=1", q, k, v, g)
    assert np.array_equal(dv, g.double().numpy())
    assert not dq.any() and not dk.any()
