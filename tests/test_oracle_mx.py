"""Pins for the oracle's MXFP8 codec, block quantization and MX GEMM (CPU only).

The E4M3 encoder is checked exhaustively against a nearest-value search over
the code table decoded from the bit-field definition (OCP 8-bit floating
point, E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, S.1111.111
is NaN, no infinities). Block scales are E8M0 powers of two chosen as the
smallest 2^e with amax <= 448 * 2^e, so no element saturates.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W


def _table():
    """(values, codes) of all finite E4M3 codes, from the bit fields."""
    vals, codes = [], []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ef, m = (c >> 3) & 15, c & 7
        if ef == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if ef == 0 else (1 + m / 8.0) * 2.0 ** (ef - 7)
        vals.append(s * v)
        codes.append(c)
    return np.array(vals), np.array(codes)


def _nearest_code(y):
    """Brute-force nearest E4M3 code; ties to the even mantissa; saturating."""
    vals, codes = _table()
    y = np.asarray(y, dtype=np.float64)
    yc = np.clip(y, -448.0, 448.0)
    dist = np.abs(yc[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among equidistant codes prefer an even mantissa (code LSB 0)
    even = (codes & 1) == 0
    pick_even = cand & even[None, :]
    use = np.where(pick_even.any(axis=1, keepdims=True), pick_even, cand)
    # zero: keep the sign of the input (+0 -> 0x00, -0 -> 0x80)
    first = np.argmax(use, axis=1)
    out = codes[first].astype(np.int64)
    zero = vals[first] == 0.0
    out = np.where(zero, np.where(np.signbit(y), 0x80, 0x00), out)
    return out.astype(np.uint8)


def test_e4m3_decode_table():
    vals, codes = _table()
    assert len(codes) == 254
    assert np.array_equal(O.e4m3_decode(codes), vals)
    assert O.e4m3_decode(0x7E) == 448.0 and O.e4m3_decode(0x01) == 2.0 ** -9
    assert np.isnan(O.e4m3_decode(0x7F)) and np.isnan(O.e4m3_decode(0xFF))


def test_e4m3_encode_exhaustive_over_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f32 = (bits << np.uint32(16)).view(np.float32)
    f = f32[np.isfinite(f32)].astype(np.float64)
    got = O.e4m3_encode(f)
    for s in range(0, f.size, 8192):
        assert np.array_equal(got[s:s + 8192], _nearest_code(f[s:s + 8192])), s


@pytest.mark.parametrize("e", [-127, -64, -9, -8, 0, 3, 119, 127])
def test_e4m3_encode_scaled_bf16(e):
    bits = np.arange(1 << 16, dtype=np.uint32)
    f32 = (bits << np.uint32(16)).view(np.float32)
    f = f32[np.isfinite(f32)].astype(np.float64)
    y = np.ldexp(f, -e)
    y = y[np.isfinite(y)]
    assert np.array_equal(O.e4m3_encode(y), _nearest_code(y))


def test_mx_hand_vectors():
    one = np.ones((1, 32))
    q, s, _, _ = O.quant_mxfp8(one, colwise=False)
    assert s[0, 0] == 0x77 and np.all(q == 0x78)
    v = np.zeros((1, 32))
    v[0, 0] = 448.0
    q, s, _, _ = O.quant_mxfp8(v, colwise=False)
    assert s[0, 0] == 0x7F and q[0, 0] == 0x7E and np.all(q[0, 1:] == 0)
    v[0, 0] = 480.0                                       # > 448: next scale, no clipping
    q, s, _, _ = O.quant_mxfp8(v, colwise=False)
    assert s[0, 0] == 0x80 and q[0, 0] == 0x77            # 480 / 2 = 240 = 1.875 * 2^7
    v = np.zeros((1, 32))
    v[0, 0], v[0, 1] = 1.0, 2.0 ** -17
    q, s, _, _ = O.quant_mxfp8(v, colwise=False)
    assert s[0, 0] == 0x77 and q[0, 1] == 0x01           # min subnormal
    q, s, _, _ = O.quant_mxfp8(np.zeros((1, 32)), colwise=False)
    assert s[0, 0] == 0x00 and np.all(q == 0)
    v = -np.ones((1, 32))
    q, s, _, _ = O.quant_mxfp8(v, colwise=False)
    assert s[0, 0] == 0x77 and np.all(q == 0xF8)


def test_mx_quant_error_bound_and_transposed_layout():
    wl = W.small("mx", T=256, k=1, E=1, d=256, n=32, seed=77)
    xb = W.make_inputs(dataclass_replace(wl, outlier_p=0.01, outlier_scale=50.0), ("x",))["x"]
    v = O.from_bf16(xb)
    q_r, s_r, q_c, s_c = O.quant_mxfp8(v)
    assert q_r.shape == (256, 256) and s_r.shape == (256, 8)
    assert q_c.shape == (256, 256) and s_c.shape == (256, 8)
    for q, s, ref in ((q_r, s_r, v), (q_c, s_c, v.T)):
        deq = O.mx_dequant(q, s)
        e = (s.astype(np.int64) - 127)
        blk_e = np.repeat(e, 32, axis=1)
        bound = np.maximum(2.0 ** -4 * np.abs(ref), np.ldexp(1.0, blk_e - 10))
        scaled = np.abs(ref) * np.ldexp(1.0, -blk_e)
        # the block maximum scales into (224, 448]: nothing saturates
        assert np.all(scaled <= 448.0)
        amax = np.abs(ref).reshape(ref.shape[0], -1, 32).max(2)
        nz = amax > 0
        assert np.all(amax[nz] * np.ldexp(1.0, -e[nz]) > 224.0)
        assert np.all(np.abs(deq - ref) <= bound)
    # and the relative error is within the MXFP8 tolerance everywhere
    assert O.max_abs_normalised_error(O.mx_dequant(q_r, s_r), v) <= 2.0 ** -4
    # colwise = rowwise of the transpose
    q_t, s_t, _, _ = O.quant_mxfp8(v.T.copy(), colwise=False)
    assert np.array_equal(q_t, q_c) and np.array_equal(s_t, s_c)


def dataclass_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)


def test_block_exponent_is_minimal_and_sufficient():
    """Brute force over every positive finite bf16 amax: the chosen e is the
    smallest integer in [-127, 127] with amax <= 448 * 2^e."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    e = O.mx_block_exponent(amax)
    fits = amax <= 448.0 * np.ldexp(1.0, e)
    tighter = amax <= 448.0 * np.ldexp(1.0, e - 1)
    assert np.all(fits | (e == 127))
    assert np.all(~tighter | (e == -127))
    assert O.mx_block_exponent(0.0) == -127


def test_mx_gemm_integer_exact():
    """Integer-valued codes with unit scales give an exact integer product."""
    rng = np.random.default_rng(2)
    R, N, K = 16, 12, 96
    ints = np.arange(-8, 9)
    a = rng.choice(ints, (R, K)).astype(np.float64)
    b = rng.choice(ints, (N, K)).astype(np.float64)
    aq, bq = O.e4m3_encode(a), O.e4m3_encode(b)
    s1 = np.full((R, K // 32), 127, np.uint8)
    s2 = np.full((N, K // 32), 127, np.uint8)
    got = O.mx_gemm_rows(aq, s1, bq, s2)
    assert np.array_equal(got, (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64))


def test_mx_gemm_equals_dequantized_matmul():
    rng = np.random.default_rng(3)
    R, N, K = 8, 10, 128
    a = O.round_bf16(rng.standard_normal((R, K)) * np.exp(rng.standard_normal((R, K))))
    b = O.round_bf16(rng.standard_normal((N, K)))
    aq, as_, _, _ = O.quant_mxfp8(a, colwise=False)
    bq, bs, _, _ = O.quant_mxfp8(b, colwise=False)
    got = O.mx_gemm_rows(aq, as_, bq, bs)
    ref = O.mx_dequant(aq, as_) @ O.mx_dequant(bq, bs).T
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # and it approximates the bf16 product within the MX tolerance
    assert O.max_abs_normalised_error(got, a @ b.T) < 6e-2


def test_mx_fc2_rounds_y_to_bf16():
    """The grouped MX FC2 stores Y in bf16: small-integer codes with unit scales
    make the exact dot products 257 and 259 (9 significant bits), which bf16
    (8 bits) rounds to 256 (a tie, to the even significand) and 260. Without
    the storage rounding Y would hold 257 and 259. Also checks that expert e's
    rows meet W2_e (a second expert whose weights are 2x the first's)."""
    E, n, d = 2, 32, 2
    M_cap = 2 * 128
    counts = np.array([1, 1])
    offsets = np.array([0, 128, 256])
    a = np.zeros((M_cap, n))
    a[0] = 8.0
    a[0, 0] = 9.0                     # 9 + 31 * 8 = 257 against a column of ones
    a[128] = 8.0
    a[128, :3] = 9.0                  # 3 * 9 + 29 * 8 = 259
    a_q = O.e4m3_encode(a)
    a_s = np.full((M_cap, n // 32), 127, np.uint8)
    w = np.zeros((E, d, n))           # W2_e stored transposed [d, n]
    w[0, 0] = 1.0
    w[0, 1] = 0.5
    w[1, 0] = 2.0
    w[1, 1] = 1.0
    w_q = O.e4m3_encode(w)
    w_s = np.full((E, d, n // 32), 127, np.uint8)
    Y = O.mx_fc2(a_q, a_s, w_q, w_s, counts, offsets)
    assert Y[0, 0] == 256.0 and Y[0, 1] == 128.0      # 257 -> 256, 128.5 -> 128
    assert Y[128, 0] == 520.0 and Y[128, 1] == 260.0  # 518 -> 520, 259 -> 260
    Yx = O.mx_fc2(a_q, a_s, w_q, w_s, counts, offsets, rounding=False)
    assert Yx[0, 0] == 257.0 and Yx[128, 1] == 259.0
    assert not Y[1:128].any() and not Y[129:].any()   # padding rows stay zero
