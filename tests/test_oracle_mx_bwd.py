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
