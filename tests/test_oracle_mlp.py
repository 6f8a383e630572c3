"""Pins for the oracle's expert MLP forward and backward (CPU only).

Library pins (torch fp64 dense MLP and torch.autograd), closed forms (zero and
identity weights), finite differences, the router-gradient identity from the
SonicMoE page, and layout invariance of the gate/up interleave.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _problem(T=48, E=4, k=2, d=64, n=64, seed=0, wstd=0.1, rounding=True):
    rng = np.random.default_rng(seed)
    x = O.round_bf16(rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = O.round_bf16(wstd * rng.standard_normal((E, d, 2 * n)))
    w2 = O.round_bf16(wstd * rng.standard_normal((E, n, d)))
    dout = O.round_bf16(rng.standard_normal((T, d)))
    return x, logits, w1, w2, dout


def _torch_moe(x, idx, w, w1, w2, g=32):
    """Dense reference: O_t = sum_j w_tj * SwiGLU-MLP_{e_tj}(x_t), torch fp64."""
    x = torch.as_tensor(x)
    w = torch.as_tensor(w)
    w1 = torch.as_tensor(w1)
    w2 = torch.as_tensor(w2)
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
            a = torch.nn.functional.silu(h[gate_cols]) * h[up_cols]
            out[t] = out[t] + w[t, j] * (a @ w2[e])
    return out


def test_single_expert_equals_dense_mlp():
    rng = np.random.default_rng(1)
    T, d, n = 20, 32, 64
    x = rng.standard_normal((T, d))
    w1 = 0.2 * rng.standard_normal((1, d, 2 * n))
    w2 = 0.2 * rng.standard_normal((1, n, d))
    logits = rng.standard_normal((T, 1)).astype(np.float32)
    r = O.forward(x, logits, w1, w2, k=1, rounding=False)
    gate, up = O.deinterleave(w1[0])
    xt = torch.as_tensor(x)
    ref = (torch.nn.functional.silu(xt @ torch.as_tensor(gate)) * (xt @ torch.as_tensor(up))) @ torch.as_tensor(w2[0])
    np.testing.assert_allclose(r["out"], ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(r["topk_w"] == 1.0)


def test_forward_matches_torch_dense_reference():
    x, logits, w1, w2, _ = _problem()
    r = O.forward(x, logits, w1, w2, k=2, rounding=False)
    ref = _torch_moe(x, r["topk_idx"], r["topk_w"], w1, w2).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
    # bf16 storage rounding stays within the parity tolerance of the exact result
    rr = O.forward(x, logits, w1, w2, k=2, rounding=True)
    assert O.max_abs_normalised_error(rr["out"], ref) < 1e-2


def test_zero_weights_give_exact_zeros():
    x, logits, w1, w2, dout = _problem()
    r = O.forward(x, logits, 0 * w1, w2, k=2)
    assert np.all(r["A"] == 0) and np.all(r["Y"] == 0) and np.all(r["out"] == 0)
    b = O.mlp_backward(r["x_perm"], 0 * w1, w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"],
                       r["offsets"], r["row_of"], r["src_of"], 2)
    for key in ("dS", "dH", "a_w", "dx_perm", "dx", "dW1", "dW2"):
        assert np.all(b[key] == 0), key
    # zero W2: only dW2 survives
    r = O.forward(x, logits, w1, 0 * w2, k=2)
    assert np.all(r["out"] == 0)
    b = O.mlp_backward(r["x_perm"], w1, 0 * w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"],
                       r["offsets"], r["row_of"], r["src_of"], 2)
    for key in ("dS", "dH", "dx_perm", "dx", "dW1"):
        assert np.all(b[key] == 0), key
    assert np.abs(b["dW2"]).max() > 0


def test_identity_weights_closed_form():
    """gate = up = [I_n; 0], W2_e = alpha_e [I_n | 0]  =>
    O_t = (sum_j w_tj alpha_{e_tj}) * x^2 sigmoid(x) on the first n dims."""
    T, E, k, d, n = 40, 4, 2, 96, 64
    rng = np.random.default_rng(3)
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    eye = np.zeros((d, n))
    eye[:n, :n] = np.eye(n)
    alpha = np.array([1.0, 2.0, 0.5, 4.0])
    w1 = np.stack([O.interleave(eye, eye)] * E)
    w2 = np.stack([a * eye.T for a in alpha])
    r = O.forward(x, logits, w1, w2, k=k, rounding=False)
    s = (r["topk_w"] * alpha[r["topk_idx"]]).sum(1, keepdims=True)
    xs = x[:, :n]
    ref = np.zeros((T, d))
    ref[:, :n] = s * xs * xs / (1 + np.exp(-xs))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("g", [1, 8, 64])
def test_interleave_granularity_is_layout_only(g):
    rng = np.random.default_rng(4)
    T, E, k, d, n = 30, 3, 2, 32, 64
    x = O.round_bf16(rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    gate = 0.1 * rng.standard_normal((E, d, n))
    up = 0.1 * rng.standard_normal((E, d, n))
    w2 = 0.1 * rng.standard_normal((E, n, d))
    r32 = O.forward(x, logits, O.interleave(gate, up, 32), w2, k, g=32, rounding=False)
    rg = O.forward(x, logits, O.interleave(gate, up, g), w2, k, g=g, rounding=False)
    np.testing.assert_allclose(rg["A"], r32["A"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(rg["out"], r32["out"], rtol=1e-14, atol=1e-15)
    # g = n is the plain [gate | up] concatenation
    cat = np.concatenate([gate, up], axis=2)
    assert np.array_equal(O.interleave(gate, up, n), cat)


def _oracle_grads(x, logits, w1, w2, dout, k, rounding):
    r = O.forward(x, logits, w1, w2, k=k, rounding=rounding)
    b = O.mlp_backward(r["x_perm"], w1, w2, r["H"], r["Y"], dout, r["topk_w"], r["counts"],
                       r["offsets"], r["row_of"], r["src_of"], k, rounding=rounding)
    return r, b


def test_backward_matches_autograd():
    x, logits, w1, w2, dout = _problem(T=40, E=4, k=2, d=32, n=64, seed=5, wstd=0.2)
    r, b = _oracle_grads(x, logits, w1, w2, dout, 2, rounding=False)
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


def test_backward_finite_differences():
    x, logits, w1, w2, dout = _problem(T=6, E=3, k=2, d=32, n=32, seed=6, wstd=0.3)
    r, b = _oracle_grads(x, logits, w1, w2, dout, 2, rounding=False)
    idx, w = r["topk_idx"], r["topk_w"]

    def loss(xv, w1v, w2v, wv):
        H, A, Y = O.mlp_forward(O.permute(xv, r["row_of"], 2, r["M_cap"]), w1v, w2v,
                                r["counts"], r["offsets"], rounding=False)
        return float((O.combine(Y, r["row_of"], 2, wv, rounding=False) * dout).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(6):
        t, c = rng.integers(6), rng.integers(32)
        xp, xm = x.copy(), x.copy()
        xp[t, c] += eps
        xm[t, c] -= eps
        fd = (loss(xp, w1, w2, w) - loss(xm, w1, w2, w)) / (2 * eps)
        assert abs(fd - b["dx"][t, c]) < 1e-6 * max(1, abs(fd))
        e, i, o = idx[t, 0], rng.integers(32), rng.integers(64)
        p, m = w1.copy(), w1.copy()
        p[e, i, o] += eps
        m[e, i, o] -= eps
        fd = (loss(x, p, w2, w) - loss(x, m, w2, w)) / (2 * eps)
        assert abs(fd - b["dW1"][e, i, o]) < 1e-6 * max(1, abs(fd))
        j = rng.integers(2)
        wp, wm = w.copy(), w.copy()
        wp[t, j] += eps
        wm[t, j] -= eps
        fd = (loss(x, w1, w2, wp) - loss(x, w1, w2, wm)) / (2 * eps)
        assert abs(fd - b["dS"][t, j]) < 1e-6 * max(1, abs(fd))


def test_router_gradient_rewrite_identity():
    """<dO_t, Y_row> (plain side) equals <dO_t W2^T, A_row> (rewritten side)."""
    x, logits, w1, w2, dout = _problem(T=64, E=5, k=3, d=64, n=32, seed=9)
    r, b = _oracle_grads(x, logits, w1, w2, dout, 3, rounding=False)
    rows = r["row_of"].reshape(-1)
    rhs = np.zeros(rows.size)
    for e, r0, r1 in O.expert_segments(r["counts"], r["offsets"]):
        da = b["dy_u"][r0:r1] @ w2[e].T
        rhs_rows = (da * r["A"][r0:r1]).sum(1)
        sel = (rows >= r0) & (rows < r1)
        rhs[sel] = rhs_rows[rows[sel] - r0]
    lhs = b["dS"].reshape(-1)
    np.testing.assert_allclose(rhs, lhs, rtol=1e-12, atol=1e-12 * np.abs(lhs).max())


def test_empty_expert_gets_exact_zero_weight_gradient():
    x, logits, w1, w2, dout = _problem(T=50, E=6, k=2, seed=12)
    logits[:, 5] = -1e4          # expert 5 is never chosen
    r, b = _oracle_grads(x, logits, w1, w2, dout, 2, rounding=True)
    assert r["counts"][5] == 0
    assert np.all(b["dW1"][5] == 0) and np.all(b["dW2"][5] == 0)
    assert r["offsets"][6] == r["offsets"][5]


def test_all_tokens_to_one_expert():
    """Constant logits, k = 1: every token goes to expert 0 with w = 1/E."""
    T, E, d, n = 33, 4, 32, 32
    rng = np.random.default_rng(13)
    x = O.round_bf16(rng.standard_normal((T, d)))
    w1 = 0.2 * rng.standard_normal((E, d, 2 * n))
    w2 = 0.2 * rng.standard_normal((E, n, d))
    logits = np.zeros((T, E), dtype=np.float32)
    r = O.forward(x, logits, w1, w2, k=1, rounding=False)
    assert list(r["counts"]) == [T, 0, 0, 0]
    single = O.forward(x, np.zeros((T, 1), np.float32), w1[:1], w2[:1], k=1, rounding=False)
    np.testing.assert_allclose(r["out"], single["out"] / E, rtol=1e-13, atol=1e-15)
    rn = O.forward(x, logits, w1, w2, k=1, renorm=True, rounding=False)
    np.testing.assert_allclose(rn["out"], single["out"], rtol=1e-13, atol=1e-15)
