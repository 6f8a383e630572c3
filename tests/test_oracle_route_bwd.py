"""Pins for the oracle's router backward (CPU only): torch.autograd through
torch's softmax and gather, finite differences, and the shift invariance of
the softmax (every row of dlogits sums to zero)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _torch_grad(logits, idx, dS, renorm):
    lg = torch.tensor(logits.astype(np.float64), requires_grad=True)
    p = torch.softmax(lg, dim=1)
    w = torch.gather(p, 1, torch.as_tensor(idx, dtype=torch.int64))
    if renorm:
        w = w / w.sum(dim=1, keepdim=True)
    (w * torch.as_tensor(dS)).sum().backward()
    return lg.grad.numpy()


@pytest.mark.parametrize("T,E,k,renorm", [(50, 8, 2, False), (40, 32, 8, False), (30, 6, 3, True),
                                          (20, 4, 4, False), (25, 5, 1, True)])
def test_route_backward_matches_autograd(T, E, k, renorm):
    rng = np.random.default_rng(T * E + k)
    logits = (2 * rng.standard_normal((T, E))).astype(np.float32)
    dS = rng.standard_normal((T, k))
    idx, _ = O.route(logits, k, renorm)
    got = O.route_backward(logits, idx, dS, renorm)
    ref = _torch_grad(logits, idx, dS, renorm)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    # softmax is shift invariant: the gradient of every row sums to zero
    assert np.abs(got.sum(axis=1)).max() < 1e-13


def test_route_backward_finite_differences():
    rng = np.random.default_rng(7)
    T, E, k = 6, 8, 2
    logits = rng.standard_normal((T, E))
    dS = rng.standard_normal((T, k))
    idx, _ = O.route(logits.astype(np.float32), k)
    got = O.route_backward(logits.astype(np.float32), idx, dS)

    def loss(lg):   # the weights of the fixed chosen experts
        z = np.exp(lg - lg.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        return float((np.take_along_axis(p, idx.astype(np.int64), axis=1) * dS).sum())

    base = logits.astype(np.float32).astype(np.float64)
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            a, b = base.copy(), base.copy()
            a[t, e] += eps
            b[t, e] -= eps
            fd = (loss(a) - loss(b)) / (2 * eps)
            assert abs(fd - got[t, e]) < 1e-8


def test_route_backward_k_equals_e_without_renorm_sums_softmax_jacobian():
    # k = E, dS = 1 for every slot: sum_j w_j = 1 identically, so the gradient is 0
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((10, 5)).astype(np.float32)
    idx, _ = O.route(logits, 5)
    got = O.route_backward(logits, idx, np.ones((10, 5)))
    assert np.abs(got).max() < 1e-15
