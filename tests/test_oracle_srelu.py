"""Pins for the oracle's sReLU variant (CPU only).

sReLU is read as the non-gated squared ReLU, A = relu(H)^2 with H = X W1_e of
width n. Its value and derivative are pinned to torch.autograd of
torch.relu(x) ** 2; the expert MLP forward and backward to a dense torch fp64
reference and to torch.autograd; identity weights give the closed form
O = s * relu(x)^2; a layer of non-positive pre-activations gives exact zeros.
"""
import numpy as np
import torch

from oracle import moe_oracle as O


def test_srelu_and_its_gradient_match_torch():
    v = torch.linspace(-6, 6, 1201, dtype=torch.float64, requires_grad=True)
    y = torch.relu(v) ** 2
    y.sum().backward()
    np.testing.assert_array_equal(O.srelu(v.detach().numpy()), y.detach().numpy())
    np.testing.assert_array_equal(O.srelu_grad(v.detach().numpy()), v.grad.numpy())
    assert O.srelu(np.array([-1.0, 0.0, 3.0])).tolist() == [0.0, 0.0, 9.0]


def _torch_moe(x, idx, w, w1, w2):
    """Dense reference: O_t = sum_j w_tj * relu(x_t W1_e)^2 W2_e, torch fp64."""
    out = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            a = torch.relu(x[t] @ w1[e]) ** 2
            out[t] = out[t] + w[t, j] * (a @ w2[e])
    return out


def _problem(T, E, d, n, seed, wstd):
    rng = np.random.default_rng(seed)
    x = O.round_bf16(rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = O.round_bf16(wstd * rng.standard_normal((E, d, n)))
    w2 = O.round_bf16(wstd * rng.standard_normal((E, n, d)))
    dout = O.round_bf16(rng.standard_normal((T, d)))
    return x, logits, w1, w2, dout


def test_srelu_forward_matches_torch_dense_reference():
    x, logits, w1, w2, _ = _problem(36, 4, 32, 48, 21, 0.2)
    r = O.forward(x, logits, w1, w2, k=2, rounding=False, act="srelu")
    assert r["H"].shape[1] == 48 and r["A"].shape[1] == 48
    ref = _torch_moe(torch.as_tensor(x), r["topk_idx"], torch.as_tensor(r["topk_w"]),
                     torch.as_tensor(w1), torch.as_tensor(w2)).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_srelu_backward_matches_autograd():
    x, logits, w1, w2, dout = _problem(40, 4, 32, 48, 22, 0.2)
    r = O.forward(x, logits, w1, w2, k=2, rounding=False, act="srelu")
    b = O.mlp_backward(r["x_perm"], w1, w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"],
                       r["offsets"], r["row_of"], r["src_of"], 2, rounding=False, act="srelu")
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


def test_srelu_rewritten_ds_equals_plain_ds():
    """The dS the GPU takes, <dO W2^T, relu(H)^2>, equals <dO, Y> (unrounded)."""
    x, logits, w1, w2, dout = _problem(30, 4, 32, 32, 23, 0.2)
    r = O.forward(x, logits, w1, w2, k=2, rounding=False, act="srelu")
    args = (r["x_perm"], w1, w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"], r["offsets"],
            r["row_of"], r["src_of"], 2)
    b = O.mlp_backward(*args, rounding=False, act="srelu")
    M_cap = r["x_perm"].shape[0]
    dy_u = O.permute(dout, r["row_of"], 2, M_cap)
    dap = np.zeros((M_cap, w2.shape[1]))
    for e, r0, r1 in O.expert_segments(r["counts"], r["offsets"]):
        dap[r0:r1] = dy_u[r0:r1] @ w2[e].T
    b2 = O.mlp_backward(*args, rounding=False, act="srelu", dap=dap)
    np.testing.assert_allclose(b2["dS"], b["dS"], rtol=1e-11, atol=1e-12)


def test_srelu_identity_weights_closed_form():
    """W1_e = [I_n; 0], W2_e = alpha_e [I_n | 0]  =>  O_t = (sum_j w_tj alpha_{e_tj}) relu(x)^2."""
    T, E, k, d, n = 40, 4, 2, 96, 64
    rng = np.random.default_rng(24)
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    eye = np.zeros((d, n))
    eye[:n, :n] = np.eye(n)
    alpha = np.array([1.0, 2.0, 0.5, 4.0])
    w1 = np.stack([eye] * E)
    w2 = np.stack([a * eye.T for a in alpha])
    r = O.forward(x, logits, w1, w2, k=k, rounding=False, act="srelu")
    s = (r["topk_w"] * alpha[r["topk_idx"]]).sum(1, keepdims=True)
    ref = np.zeros((T, d))
    ref[:, :n] = s * np.maximum(x[:, :n], 0.0) ** 2
    np.testing.assert_allclose(r["out"], ref, rtol=1e-13, atol=1e-15)


def test_nonpositive_preactivation_gives_exact_zeros():
    x, logits, w1, w2, dout = _problem(16, 3, 32, 32, 25, 0.2)
    x = np.abs(x)
    w1 = -np.abs(w1)                    # H <= 0 everywhere
    r = O.forward(x, logits, w1, w2, k=2, rounding=False, act="srelu")
    assert np.all(r["A"] == 0) and np.all(r["out"] == 0)
    b = O.mlp_backward(r["x_perm"], w1, w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"],
                       r["offsets"], r["row_of"], r["src_of"], 2, rounding=False, act="srelu")
    for key in ("dH", "dx", "dW1", "dW2", "dS"):
        assert np.all(b[key] == 0), key
