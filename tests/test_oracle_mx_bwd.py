"""Pins for the oracle's MXFP8 backward (CPU only).

* the wgrad products over rows equal the block-scaled MX-GEMM definition of
  the forward (mx_gemm_rows) applied to the transposed operands, an
  independent formulation of the same sum;
* data that MXFP8 represents exactly (small integers, unit block scales)
  makes every MX gradient equal the bf16 path's gradient computed on the
  same values;
* on random data the MX gradients stay within the MXFP8 tolerance of the
  bf16 backward; zero upstream gradient gives exact zeros.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O

TOL_MX = 6e-2
# outputs behind two quantized GEMMs (Y after an MX FC1 and an MX FC2): the
# E4M3 rounding of both products adds, so twice the one-GEMM bound
TOL_MX_CHAIN = 1.2e-1


def _run(T=64, E=3, k=2, d=64, n=64, seed=0, wstd=0.2, scale=1.0):
    rng = np.random.default_rng(seed)
    x = O.round_bf16(scale * rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = O.round_bf16(wstd * rng.standard_normal((E, d, 2 * n)))
    w2 = O.round_bf16(wstd * rng.standard_normal((E, n, d)))
    dout = O.round_bf16(rng.standard_normal((T, d)))
    f = O.forward(x, logits, w1, w2, k)
    args = (f["x_perm"], w1, w2, f["H"], f["Y"], dout, f["topk_w"], f["counts"], f["offsets"],
            f["row_of"], f["src_of"], k)
    return f, O.mlp_backward(*args), O.mlp_backward_mx(*args), args


def test_mx_wgrad_equals_block_scaled_gemm_definition():
    f, b, m, _ = _run(seed=1)
    off = f["offsets"]
    for e in range(len(f["counts"])):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        ref2 = O.mx_gemm_rows(m["awt_q"][:, r0:r1], m["awt_s"][:, r0 // 32:r1 // 32],
                              m["dyt_q"][:, r0:r1], m["dyt_s"][:, r0 // 32:r1 // 32])
        ref1 = O.mx_gemm_rows(m["xt_q"][:, r0:r1], m["xt_s"][:, r0 // 32:r1 // 32],
                              m["dht_q"][:, r0:r1], m["dht_s"][:, r0 // 32:r1 // 32])
        np.testing.assert_allclose(m["dW2"][e], ref2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(m["dW1"][e], ref1, rtol=1e-12, atol=1e-12)


def test_mx_backward_within_tolerance_of_bf16():
    _, b, m, _ = _run(T=96, E=4, k=2, d=128, n=64, seed=2)
    for key in ("dx_perm", "dx", "dW1", "dW2"):
        err = O.max_abs_normalised_error(m[key], b[key])
        assert 0 < err <= TOL_MX, (key, err)
    for key in ("dH", "a_w", "dS"):        # the bf16 FC2 dgrad is shared
        assert np.array_equal(m[key], b[key])


def test_mx_exact_data_reduces_to_bf16_path():
    """Integer data in [-4, 4]: the block scale keeps every value an exact E4M3
    code, so each MX product equals the plain product."""
    rng = np.random.default_rng(3)
    M, K, N = 64, 96, 32
    a = rng.integers(-4, 5, (M, K)).astype(np.float64)
    bt = rng.integers(-4, 5, (N, K)).astype(np.float64)
    qa, sa, qat, sat = O.quant_mxfp8(a, True, True)
    qb, sb, qbt, sbt = O.quant_mxfp8(bt, True, True)
    assert np.array_equal(O.mx_dequant(qa, sa), a) and np.array_equal(O.mx_dequant(qat, sat), a.T)
    np.testing.assert_array_equal(O.mx_gemm_rows(qa, sa, qb, sb), a @ bt.T)
    # the wgrad form: K runs down the rows of two column-wise copies
    c = rng.integers(-4, 5, (M, N)).astype(np.float64)
    _, _, qct, sct = O.quant_mxfp8(c, False, True)
    np.testing.assert_array_equal(O.mx_dequant(qat, sat) @ O.mx_dequant(qct, sct).T, a.T @ c)


def test_mx_backward_zero_upstream_gradient():
    f, _, _, args = _run(seed=4)
    args = list(args)
    args[5] = np.zeros_like(args[5])
    m = O.mlp_backward_mx(*args)
    for key in ("dx", "dW1", "dW2", "dH"):
        assert np.all(m[key] == 0), key


def _exact_case(seed=5, T=80, E=3, k=2, d=64, n=64):
    """Small-integer data: every MXFP8 copy is exact, so every MX product equals
    the plain product of the same values."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, (T, d)).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = rng.integers(-2, 3, (E, d, 2 * n)).astype(np.float64) / 64.0
    w2 = rng.integers(-2, 3, (E, n, d)).astype(np.float64) / 64.0
    dout = rng.integers(-3, 4, (T, d)).astype(np.float64)
    return x, logits, w1, w2, dout


def test_mx_fc1_exact_data_equals_bf16_forward():
    x, logits, w1, w2, _ = _exact_case()
    f = O.forward(x, logits, w1, w2, 2)
    m = O.mlp_forward_mx(f["x_perm"], w1, w2, f["counts"], f["offsets"])
    end = int(f["offsets"][-1])
    assert np.array_equal(O.mx_dequant(m["x_q"], m["x_s"]), f["x_perm"][:end])
    np.testing.assert_array_equal(m["H"], f["H"])
    np.testing.assert_array_equal(m["A"], f["A"])


def test_mx_forward_within_tolerance_of_bf16():
    rng = np.random.default_rng(6)
    T, E, k, d, n = 96, 4, 2, 128, 64
    x = O.round_bf16(rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = O.round_bf16(0.2 * rng.standard_normal((E, d, 2 * n)))
    w2 = O.round_bf16(0.2 * rng.standard_normal((E, n, d)))
    f = O.forward(x, logits, w1, w2, k)
    for fc1_mx in (True, False):
        m = O.mlp_forward_mx(f["x_perm"], w1, w2, f["counts"], f["offsets"], fc1_mx=fc1_mx)
        for key in ("H", "A", "Y"):
            err = O.max_abs_normalised_error(m[key], f[key])
            assert err <= (TOL_MX_CHAIN if key == "Y" and fc1_mx else TOL_MX), (fc1_mx, key, err)
            if key in ("H", "A"):
                assert (err > 0) == fc1_mx, (fc1_mx, key, err)


def test_mx_fc1_equals_block_scaled_definition_per_expert():
    """mx_fc1 = the block-scaled sum written out per block, then the GLU."""
    f, _, _, args = _run(seed=7)
    w1 = args[1]
    m = O.mlp_forward_mx(f["x_perm"], w1, args[2], f["counts"], f["offsets"])
    xv = O.mx_dequant(m["x_q"], m["x_s"])
    for e, r0, r1 in O.expert_segments(f["counts"], f["offsets"]):
        if r1 == r0:
            continue
        wv = O.mx_dequant(m["w1t_q"][e], m["w1t_s"][e])            # [2n, d]
        h = xv[r0:r1] @ wv.T
        np.testing.assert_array_equal(m["H"][r0:r1], O.round_bf16(h))
        hg, hu = O.deinterleave(h)
        np.testing.assert_array_equal(m["A"][r0:r1], O.round_bf16(O.silu(hg) * hu))


def test_mx_dgrad2_exact_data_equals_bf16_backward():
    x, logits, w1, w2, dout = _exact_case(seed=8)
    f = O.forward(x, logits, w1, w2, 2)
    args = (f["x_perm"], w1, w2, f["H"], f["Y"], dout, f["topk_w"], f["counts"], f["offsets"],
            f["row_of"], f["src_of"], 2)
    b = O.mlp_backward(*args)
    m = O.mlp_backward_mx(*args, dgrad2_mx=True)
    for key in ("dH", "a_w"):
        np.testing.assert_array_equal(m[key], b[key])
    # dS on the rewritten side equals the plain side up to the bf16 rounding of Y
    assert O.max_abs_normalised_error(m["dS"], b["dS"]) <= 1e-2


def test_mx_dgrad2_within_tolerance_and_rewritten_ds():
    f, b, _, args = _run(T=96, E=4, k=2, d=128, n=64, seed=9)
    m = O.mlp_backward_mx(*args, dgrad2_mx=True)
    assert np.array_equal(m["a_w"], b["a_w"])   # A' = w a does not depend on dA'
    for key in ("dH", "dS", "dx", "dW1", "dW2"):
        err = O.max_abs_normalised_error(m[key], b[key])
        assert 0 < err <= TOL_MX, (key, err)
    # dS = <dA'_mx, a> per row, the dA' from the block-scaled product of the copies
    dyv = O.mx_dequant(m["dy_q"], m["dy_s"])
    end = int(f["offsets"][-1])
    rows = np.asarray(f["row_of"], dtype=np.int64)
    H = f["H"]
    dsr = np.zeros(H.shape[0])
    for e, r0, r1 in O.expert_segments(f["counts"], f["offsets"]):
        if r1 > r0:
            dap = dyv[r0:r1] @ O.mx_dequant(m["w2q"][e], m["w2s"][e]).T
            hg, hu = O.deinterleave(H[r0:r1])
            dsr[r0:r1] = (dap * O.silu(hg) * hu).sum(axis=1)
    np.testing.assert_allclose(m["dS"].reshape(-1), dsr[rows], rtol=1e-10, atol=1e-12)
    assert end > 0
