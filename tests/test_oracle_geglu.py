"""Pins for the oracle's GeGLU variant (CPU only).

GELU is taken in its exact form x * Phi(x). Its values are pinned to
tabulated standard-normal CDF values, its derivative to torch.autograd of
torch's own GELU; the GeGLU expert MLP forward and backward are pinned to a
dense torch fp64 reference and to torch.autograd, and the identity-weight
closed form O = s * x * gelu(x) is checked with torch's GELU.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

F = torch.nn.functional

# standard normal CDF at a few points (printed in every statistics table)
PHI = {0.0: 0.5, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -0.5: 0.3085375387259869,
       -1.0: 0.15865525393145707, 3.0: 0.9986501019683699}


def test_gelu_matches_tabulated_normal_cdf():
    for v, phi in PHI.items():
        assert abs(O.gelu(np.array([v]))[0] - v * phi) < 1e-15


def test_gelu_and_its_gradient_match_torch():
    v = torch.linspace(-8, 8, 2001, dtype=torch.float64, requires_grad=True)
    y = F.gelu(v, approximate="none")
    y.sum().backward()
    np.testing.assert_allclose(O.gelu(v.detach().numpy()), y.detach().numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu_grad(v.detach().numpy()), v.grad.numpy(), rtol=1e-13, atol=1e-15)


def _torch_moe(x, idx, w, w1, w2, g=32):
    """Dense reference: O_t = sum_j w_tj * GeGLU-MLP_{e_tj}(x_t), torch fp64."""
    E, d, n2 = w1.shape
    n = n2 // 2
    cols = np.arange(n2).reshape(n // g, 2, g)
    gate_cols = torch.as_tensor(cols[:, 0, :].reshape(-1))
    up_cols = torch.as_tensor(cols[:, 1, :].reshape(-1))
    out = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            h = x[t] @ w1[e]
            a = F.gelu(h[gate_cols], approximate="none") * h[up_cols]
            out[t] = out[t] + w[t, j] * (a @ w2[e])
    return out


def _problem(T, E, d, n, seed, wstd):
    rng = np.random.default_rng(seed)
    x = O.round_bf16(rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = O.round_bf16(wstd * rng.standard_normal((E, d, 2 * n)))
    w2 = O.round_bf16(wstd * rng.standard_normal((E, n, d)))
    dout = O.round_bf16(rng.standard_normal((T, d)))
    return x, logits, w1, w2, dout


def test_geglu_forward_matches_torch_dense_reference():
    x, logits, w1, w2, _ = _problem(36, 4, 32, 64, 11, 0.2)
    r = O.forward(x, logits, w1, w2, k=2, rounding=False, act="geglu")
    ref = _torch_moe(torch.as_tensor(x), r["topk_idx"], torch.as_tensor(r["topk_w"]),
                     torch.as_tensor(w1), torch.as_tensor(w2)).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
    # the activation switch is real: SwiGLU gives a different layer
    rs = O.forward(x, logits, w1, w2, k=2, rounding=False, act="swiglu")
    assert np.abs(rs["out"] - r["out"]).max() > 1e-3


def test_geglu_backward_matches_autograd():
    x, logits, w1, w2, dout = _problem(40, 4, 32, 64, 12, 0.2)
    r = O.forward(x, logits, w1, w2, k=2, rounding=False, act="geglu")
    b = O.mlp_backward(r["x_perm"], w1, w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"],
                       r["offsets"], r["row_of"], r["src_of"], 2, rounding=False, act="geglu")
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(r["topk_w"], requires_grad=True)
    w1t = torch.tensor(w1, requires_grad=True)
    w2t = torch.tensor(w2, requires_grad=True)
    out = _torch_moe(xt, r["topk_idx"], wt, w1t, w2t)
    (out * torch.as_tensor(dout)).sum().backward()
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dW1"], w1t.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dW2"], w2t.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dS"], wt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_geglu_identity_weights_closed_form():
    """gate = up = [I_n; 0], W2_e = alpha_e [I_n | 0]  =>
    O_t = (sum_j w_tj alpha_{e_tj}) * x * gelu(x) on the first n dims."""
    T, E, k, d, n = 40, 4, 2, 96, 64
    rng = np.random.default_rng(13)
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    eye = np.zeros((d, n))
    eye[:n, :n] = np.eye(n)
    alpha = np.array([1.0, 2.0, 0.5, 4.0])
    w1 = np.stack([O.interleave(eye, eye)] * E)
    w2 = np.stack([a * eye.T for a in alpha])
    r = O.forward(x, logits, w1, w2, k=k, rounding=False, act="geglu")
    s = (r["topk_w"] * alpha[r["topk_idx"]]).sum(1, keepdims=True)
    xs = x[:, :n]
    ref = np.zeros((T, d))
    ref[:, :n] = s * xs * F.gelu(torch.as_tensor(xs), approximate="none").numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_zero_gate_gives_zero_activation(act):
    # silu(0) = gelu(0) = 0: a zero gate half makes A, Y and every dX exactly 0
    x, logits, w1, w2, dout = _problem(16, 3, 32, 32, 14, 0.2)
    g, u = O.deinterleave(w1)
    w1z = O.interleave(np.zeros_like(g), u)
    r = O.forward(x, logits, w1z, w2, k=2, rounding=False, act=act)
    assert np.all(r["A"] == 0) and np.all(r["out"] == 0)
