"""GPU parity of the MXFP8 backward: the dGLU epilogue's fused quantization,
the MX-scaled FC1 dgrad and the two MX-scaled ragged wgrads.

* DGRAD2 stays bf16: dH, A' and dS within 2e-2 of the oracle (as the bf16 path).
* Its fused MXFP8 copies equal, bit for bit, the oracle's quantization of the
  GPU's own bf16 dH and A' over the whole expert region (and, as an extra,
  the standalone quantization kernel's copies of them); the column-wise
  dY_u / X_perm copies and row-wise W1 copy equal the oracle's quantization
  of the (bit-exact) permuted inputs.
* The three MX GEMMs on the GPU's own codes: dW1 and dW2 within 1e-3 of the
  fp64 block-scaled product of those codes, dX_perm within 1e-2 (one bf16
  rounding). The scaled MFMA is not exact-products-plus-fp32-sum: on random
  codes it lands about 7e-5 (max-abs-normalised) from the fp64 product, far
  above fp32 summation error, so the bound leaves a 10x margin over that.
* End to end against the oracle's MXFP8 backward from the same seeded inputs:
  within 6e-2 (the codes on the two sides may differ where dH rounds
  differently in bf16). Empty experts: dW exactly 0.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

from ._util import bf16_bits, bf16_tensor, bf16_values, check_fused_copies_vs_oracle, f32_tensor, rel_err

pytestmark = pytest.mark.gpu

CASES = [
    W.small("mxb-small", T=600, k=2, E=4, d=256, n=256, seed=41, routing="zipf"),
    W.small("mxb-ragged", T=700, k=3, E=6, d=192, n=320, seed=21, routing="zipf"),
    W.small("mxb-empty", T=300, k=2, E=16, d=256, n=128, seed=22, routing="zipf"),
    W.small("mxb-wide", T=1200, k=2, E=4, d=640, n=384, seed=23),
    W.small("mxb-many", T=400, k=4, E=300, d=128, n=128, seed=26, routing="zipf"),
]


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _np(t):
    return t.cpu().numpy()


def _run_gpu(M, wl, inp, act, dgrad2_mx=False):
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=True)
    for name in ("dh", "a_w", "ds", "dx_perm", "dx", "dw1", "dw2"):
        getattr(buf, name).fill_(float("nan"))
    for name in M.MX_BWD_FIELDS:
        getattr(buf, name).fill_(0xAB)
    x, w1, w2 = bf16_tensor(inp["x"]), bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    logits, dout = f32_tensor(inp["logits"]), bf16_tensor(inp["dout"])
    buf.quantize_weights(w1, w2)
    M.forward(buf, x, logits, w1, w2, act=act)
    M.backward(buf, dout, w1, w2, act=act, mx=True, dgrad2_mx=dgrad2_mx)
    torch.cuda.synchronize()
    return buf


def _gpu_quant(M, t, mode):
    """Standalone quantization kernel on a bf16 device matrix [R, C]."""
    R, C = t.shape
    U8 = torch.uint8
    q_row = torch.empty(R, C, dtype=U8, device="cuda") if mode & 1 else None
    s_row = torch.empty(R, C // 32, dtype=U8, device="cuda") if mode & 1 else None
    q_col = torch.empty(C, R, dtype=U8, device="cuda") if mode & 2 else None
    s_col = torch.empty(C, R // 32, dtype=U8, device="cuda") if mode & 2 else None
    M.moe_quant_mxfp8(t.contiguous(), mode, q_row, s_row, q_col, s_col)
    torch.cuda.synchronize()
    return [None if v is None else _np(v) for v in (q_row, s_row, q_col, s_col)]


def _check(name, got, ref, tol):
    assert np.isfinite(got).all(), f"{name}: unwritten (NaN) or non-finite elements"
    err = rel_err(got, ref)
    print(f"  {name}: max-abs-normalised error {err:.3e}", flush=True)
    assert err <= tol, f"{name}: {err}"


# dgrad2_mx: the FC2 dgrad also on MXFP8 (dY_u row-wise x W2_e along d); d must be a
# multiple of 128 for it
def _random_cases(count, seed):
    """Seeded shapes for the all-MXFP8 backward: any token count (one token included),
    k up to min(E, 8), 1-40 experts, d and n multiples of 128 up to 640."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        E = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = 1 if i == 0 else int(rng.integers(2, 1200))
        d, n = 128 * int(rng.integers(1, 6)), 128 * int(rng.integers(1, 6))
        out.append(W.small(f"mxb-random{i}", T=T, k=k, E=E, d=d, n=n, seed=300 + i,
                           routing=("normal", "zipf")[i % 2]))
    return out


MX_DG2 = [(c, "swiglu", False) for c in CASES] + [(CASES[1], "geglu", False)] + [
    (CASES[0], "swiglu", True), (CASES[2], "swiglu", True), (CASES[3], "geglu", True)] + [
    (c, "swiglu", True) for c in _random_cases(4, 77)]


@pytest.mark.parametrize("wl,act,dgrad2_mx", MX_DG2,
                         ids=[f"{c.name}-{a}" + ("-dgrad2mx" if g else "") for c, a, g in MX_DG2])
def test_mx_backward_parity(M, wl, act, dgrad2_mx):
    print(f"mx backward case {wl} act={act} dgrad2_mx={dgrad2_mx}", flush=True)
    inp = W.make_inputs(wl)
    buf = _run_gpu(M, wl, inp, M.MOE_ACT_GEGLU if act == "geglu" else M.MOE_ACT_SWIGLU, dgrad2_mx)
    x, w1, w2 = O.from_bf16(inp["x"]), O.from_bf16(inp["w1"]), O.from_bf16(inp["w2"])
    f = O.forward(x, inp["logits"], w1, w2, wl.k, act=act)
    b = O.mlp_backward_mx(f["x_perm"], w1, w2, f["H"], f["Y"], O.from_bf16(inp["dout"]), f["topk_w"],
                          f["counts"], f["offsets"], f["row_of"], f["src_of"], wl.k, act=act,
                          dgrad2_mx=dgrad2_mx)
    offsets = f["offsets"]
    end = int(offsets[-1])
    assert np.array_equal(_np(buf.offsets), offsets)
    if dgrad2_mx:   # the FC2 dgrad operands: the oracle's quantization of the same bf16 values
        assert np.array_equal(_np(buf.dy_q)[:end], b["dy_q"]) and np.array_equal(
            _np(buf.dy_s)[:end], b["dy_s"]), "dY_u row copy"
        assert np.array_equal(_np(buf.w2_q), b["w2q"]) and np.array_equal(_np(buf.w2_s), b["w2s"]), "W2 copy"

    # DGRAD2 (bf16, or MX on codes identical to the oracle's) as in the bf16 path
    _check("dS", _np(buf.ds), b["dS"], 2e-2)
    _check("dH", bf16_values(buf.dh)[:end], b["dH"][:end], 2e-2)
    _check("A'", bf16_values(buf.a_w)[:end], b["a_w"][:end], 2e-2)

    # fused copies == the oracle's quantization of the GPU's own bf16 dH and A', bit for bit
    check_fused_copies_vs_oracle(buf.dh, end, buf.dh_q, buf.dh_s, buf.dht_q, buf.dht_s, "dH")
    check_fused_copies_vs_oracle(buf.a_w, end, None, None, buf.awt_q, buf.awt_s, "A'")
    # extra: == the standalone quantization kernel's copies of the same bf16 tensors
    g = _gpu_quant(M, buf.dh[:end], 3)
    assert np.array_equal(_np(buf.dh_q)[:end], g[0]), "dH row codes"
    assert np.array_equal(_np(buf.dh_s)[:end], g[1]), "dH row scales"
    assert np.array_equal(_np(buf.dht_q)[:, :end], g[2]), "dH column codes"
    assert np.array_equal(_np(buf.dht_s)[:, :end // 32], g[3]), "dH column scales"
    g = _gpu_quant(M, buf.a_w[:end], 2)
    assert np.array_equal(_np(buf.awt_q)[:, :end], g[2]), "A' column codes"
    assert np.array_equal(_np(buf.awt_s)[:, :end // 32], g[3]), "A' column scales"
    # quantized inputs == the oracle's quantization of the same bf16 values
    assert np.array_equal(_np(buf.dyt_q)[:, :end], b["dyt_q"]) and np.array_equal(
        _np(buf.dyt_s)[:, :end // 32], b["dyt_s"]), "dY_u column copy"
    assert np.array_equal(_np(buf.xt_q)[:, :end], b["xt_q"]) and np.array_equal(
        _np(buf.xt_s)[:, :end // 32], b["xt_s"]), "X_perm column copy"
    assert np.array_equal(_np(buf.w1_q), b["w1q"]) and np.array_equal(_np(buf.w1_s), b["w1s"]), "W1 copy"

    # the MX GEMMs on the GPU's own codes
    dht_d = O.mx_dequant(_np(buf.dht_q)[:, :end], _np(buf.dht_s)[:, :end // 32])
    awt_d = O.mx_dequant(_np(buf.awt_q)[:, :end], _np(buf.awt_s)[:, :end // 32])
    xt_d = O.mx_dequant(b["xt_q"], b["xt_s"])
    dyt_d = O.mx_dequant(b["dyt_q"], b["dyt_s"])
    dW1 = np.zeros(w1.shape)
    dW2 = np.zeros(w2.shape)
    dxp = np.zeros((end, wl.d))
    for e in range(wl.E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            dW1[e] = xt_d[:, r0:r1] @ dht_d[:, r0:r1].T
            dW2[e] = awt_d[:, r0:r1] @ dyt_d[:, r0:r1].T
            dxp[r0:r1] = O.mx_gemm_rows(_np(buf.dh_q)[r0:r1], _np(buf.dh_s)[r0:r1], b["w1q"][e], b["w1s"][e])
    _check("dW1 (own codes)", _np(buf.dw1), dW1, 1e-3)
    _check("dW2 (own codes)", _np(buf.dw2), dW2, 1e-3)
    _check("dX_perm (own codes)", bf16_values(buf.dx_perm)[:end], dxp, 1e-2)

    # end to end against the oracle's MXFP8 backward
    _check("dX_perm", bf16_values(buf.dx_perm)[:end], b["dx_perm"][:end], 6e-2)
    _check("dX", bf16_values(buf.dx), b["dx"], 6e-2)
    _check("dW1", _np(buf.dw1), b["dW1"], 6e-2)
    _check("dW2", _np(buf.dw2), b["dW2"], 6e-2)
    pad = f["src_of"][:end] < 0
    v = bf16_bits(buf.dx_perm)[:end][pad]
    assert np.all((v == 0) | (v == 0x8000)), "padding rows of dX_perm"
    for e in np.nonzero(f["counts"] == 0)[0]:
        assert torch.all(buf.dw1[e] == 0) and torch.all(buf.dw2[e] == 0)


@pytest.mark.parametrize("wl", [CASES[0], CASES[2]], ids=[CASES[0].name, CASES[2].name])
def test_groupgemm_quantize_dgrad1(M, wl):
    """GroupGemm + Quantize in the backward: the MX FC1 dgrad's epilogue writes the row-wise
    MXFP8 copy of dX_perm and its transposed column-wise copy, bit for bit the oracle's
    quantization of the GPU's own bf16 dX_perm, without changing dX_perm (and alone when
    dx_perm is NULL)."""
    inp = W.make_inputs(wl)
    buf = _run_gpu(M, wl, inp, M.MOE_ACT_SWIGLU)
    end = int(buf.offsets[-1].item())
    dx_ref = buf.dx_perm.clone()
    for t in (buf.dx_q, buf.dx_s, buf.dxt_q, buf.dxt_s):
        t.fill_(0xAB)
    w1, w2 = bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    args = (buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of, buf.row_of, buf.offsets,
            buf.dh, buf.a_w, buf.ds)
    mx = buf.mx_bwd(dgrad2=False, quant_dx=True, transposed_dx=True)
    M.moe_grouped_mlp_bwd(*args, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, M.MOE_STAGE_DGRAD1, mx=mx)
    torch.cuda.synchronize()
    assert torch.equal(buf.dx_perm[:end], dx_ref[:end])
    check_fused_copies_vs_oracle(buf.dx_perm, end, buf.dx_q, buf.dx_s, buf.dxt_q, buf.dxt_s, "dX_perm")
    q_ref, qt_ref = buf.dx_q[:end].clone(), buf.dxt_q[:, :end].clone()
    buf.dx_q.fill_(0xAB)
    buf.dxt_q.fill_(0xAB)
    M.moe_grouped_mlp_bwd(*args, None, buf.dw1, buf.dw2, buf.bwd_ws, M.MOE_STAGE_DGRAD1, mx=mx)
    torch.cuda.synchronize()
    assert torch.equal(buf.dx_q[:end], q_ref) and torch.equal(buf.dxt_q[:, :end], qt_ref)
    if end < buf.M_cap:
        assert torch.all(buf.dxt_q[:, end:] == 0xAB)


def test_mx_wgrad_all_tokens_to_one_expert(M):
    """One expert takes every row, the rest are empty: the longest ragged-K
    tiles and many zero-K tiles in one launch."""
    wl = W.small("mxb-one", T=520, k=1, E=8, d=128, n=128, seed=31)
    inp = W.make_inputs(wl)
    inp["logits"][:] = 0.0                     # ties everywhere -> expert 0
    buf = _run_gpu(M, wl, inp, M.MOE_ACT_SWIGLU)
    x, w1, w2 = O.from_bf16(inp["x"]), O.from_bf16(inp["w1"]), O.from_bf16(inp["w2"])
    f = O.forward(x, inp["logits"], w1, w2, wl.k)
    b = O.mlp_backward_mx(f["x_perm"], w1, w2, f["H"], f["Y"], O.from_bf16(inp["dout"]), f["topk_w"],
                          f["counts"], f["offsets"], f["row_of"], f["src_of"], wl.k)
    assert list(_np(buf.counts)) == [520, 0, 0, 0, 0, 0, 0, 0]
    _check("dX", bf16_values(buf.dx), b["dx"], 6e-2)
    _check("dW1", _np(buf.dw1), b["dW1"], 6e-2)
    _check("dW2", _np(buf.dw2), b["dW2"], 6e-2)
    assert torch.all(buf.dw1[1:] == 0) and torch.all(buf.dw2[1:] == 0)


@pytest.mark.parametrize("wl", [CASES[0], CASES[2]], ids=[CASES[0].name, CASES[2].name])
def test_mx_step_without_bf16_copies(M, wl):
    """The MXFP8 step as bench.py runs it: permute fused with the quantization
    of x, FC1 on MXFP8 operands keeping A only as its MXFP8 copy (a = NULL),
    the MX FC2, and a backward whose FC2 dgrad writes only the MXFP8 copies of
    dH and A' (dh = a_w = NULL). Every output, and every MXFP8 copy, equals
    bit for bit the same step with the bf16 A, dH and A' written."""
    print(f"mx step without bf16 copies: {wl}", flush=True)
    inp = W.make_inputs(wl)
    x, w1, w2 = bf16_tensor(inp["x"]), bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    logits, dout = f32_tensor(inp["logits"]), bf16_tensor(inp["dout"])
    outs = ("y", "out", "ds", "dx_perm", "dx", "dw1", "dw2", "dlogits", "h")
    codes = ("a_q", "a_s", "x_q", "x_s", "xt_q", "xt_s", "dy_q", "dy_s", "dyt_q", "dyt_s",
             "dh_q", "dh_s", "dht_q", "dht_s", "awt_q", "awt_s")

    def run(bf16_copies):
        buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=True)
        for name in outs + ("a", "dh", "a_w"):
            getattr(buf, name).fill_(float("nan"))
        for name in codes:
            getattr(buf, name).fill_(0xAB)
        buf.quantize_weights(w1, w2)
        mx = buf.mx_fwd()
        M.moe_route_counts(logits, wl.k, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets, buf.row_of,
                           buf.src_of, buf.M_cap, buf.err, buf.route_ws)
        M.moe_permute_quant_mxfp8(x, buf.src_of, wl.k, wl.E, M.MOE_QUANT_ROWWISE | M.MOE_QUANT_COLWISE,
                                  buf.x_q, buf.x_s, buf.xt_q, buf.xt_s)
        buf.xt_from_forward = True
        a = buf.a if bf16_copies else None
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, a, buf.y, M.MOE_STAGE_FC1, mx=mx)
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, a, buf.y, M.MOE_STAGE_FC2, mx=mx)
        M.moe_combine(buf.y, buf.row_of, buf.topk_w, wl.k, buf.out)
        M.backward(buf, dout, w1, w2, logits=logits, mx=True, mx_bf16_copies=bf16_copies)
        torch.cuda.synchronize()
        end = int(buf.offsets[-1].item())
        got = {}
        for name in outs + codes:
            t = getattr(buf, name)
            got[name] = t.contiguous().view(torch.uint8).cpu().numpy()
        return got, end, buf

    full, end, buf_full = run(True)
    lean, end2, buf_lean = run(False)
    assert end == end2
    for name in full:
        assert np.array_equal(full[name], lean[name]), f"{name} differs without the bf16 copies"
    # the lean run left its bf16 A, dH and A' untouched (still the NaN fill)
    for name in ("a", "dh", "a_w"):
        assert torch.isnan(getattr(buf_lean, name).float()).all(), f"{name} was written"
        assert not torch.isnan(getattr(buf_full, name)[:end].float()).all(), f"{name} was not written"
