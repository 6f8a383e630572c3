"""GPU parity of the MXFP8 path: block quantization, the fused quantization
epilogue of FC1 and the MX-scaled grouped FC2.

* Standalone quantization: codes and scales bit-exact against the oracle on
  seeded inputs (with outliers), on every finite bf16 pattern, and on edge
  cases (zero blocks, subnormals, saturation, partial tiles, batches).
* Fused epilogue: its codes and scales equal, bit for bit, the oracle's
  quantization of the GPU's own bf16 A over the whole expert region (the two
  A's may differ in the last bf16 bit, so codes are compared on the GPU's A);
  as an extra, they equal the standalone kernel's codes of the same A, and
  they dequantize to within 6e-2 of the oracle's A.
* MX FC2: within 6e-2 of the oracle's MX forward from the same seeded inputs;
  on identical codes (verified bit-exact) within 1e-2.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

from ._util import bf16_tensor, bf16_values, check_fused_copies_vs_oracle, f32_tensor, rel_err

pytestmark = pytest.mark.gpu
U8 = torch.uint8


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _scales(shape, offset):
    """0xAB-filled uint8 scale array of `shape` starting `offset` bytes into its allocation
    (offset 1: no longer word-aligned, so the kernel must fall back to byte stores)."""
    n = int(np.prod(shape))
    return torch.full((n + offset,), 0xAB, dtype=U8, device="cuda")[offset:].view(shape)


def _gpu_quant(M, bits, mode=3, scale_offset=0):
    """bits: uint16 [batch, R, C] or [R, C] -> numpy codes/scales (None if not requested)."""
    x = bf16_tensor(bits)
    shp = bits.shape if bits.ndim == 3 else (1,) + bits.shape
    B, R, C = shp
    q_row = torch.full((B, R, C), 0xAB, dtype=U8, device="cuda") if mode & 1 else None
    s_row = _scales((B, R, C // 32), scale_offset) if mode & 1 else None
    q_col = torch.full((B, C, R), 0xAB, dtype=U8, device="cuda") if mode & 2 else None
    s_col = _scales((B, C, R // 32), scale_offset) if mode & 2 else None
    M.moe_quant_mxfp8(x.view(B, R, C), mode, q_row, s_row, q_col, s_col)
    torch.cuda.synchronize()
    f = (lambda t: None if t is None else t.cpu().numpy())
    return f(q_row), f(s_row), f(q_col), f(s_col)


def _check_quant(M, bits, mode=3, scale_offset=0):
    g = _gpu_quant(M, bits, mode, scale_offset)
    b3 = bits if bits.ndim == 3 else bits[None]
    for b in range(b3.shape[0]):
        q_r, s_r, q_c, s_c = O.quant_mxfp8(O.from_bf16(b3[b]), rowwise=bool(mode & 1),
                                           colwise=bool(mode & 2))
        if mode & 1:
            assert np.array_equal(g[0][b], q_r), "row codes"
            assert np.array_equal(g[1][b], s_r), "row scales"
        if mode & 2:
            assert np.array_equal(g[2][b], q_c), "col codes"
            assert np.array_equal(g[3][b], s_c), "col scales"


@pytest.mark.parametrize("R,C,mode", [(256, 256, 3), (96, 160, 3), (4096, 2048, 3), (160, 64, 1),
                                      (64, 96, 2), (1000, 32, 1), (2560, 384, 3), (4608, 256, 2),
                                      (1152, 416, 3)])
def test_quant_bit_exact_seeded(M, R, C, mode):
    print(f"quant case R={R} C={C} mode={mode}", flush=True)
    rng = np.random.default_rng(R * 31 + C)
    v = rng.standard_normal((R, C)).astype(np.float32)
    v[rng.random((R, C)) < 0.01] *= 50.0
    _check_quant(M, W.f32_to_bf16_bits(v), mode)


def test_quant_unaligned_scale_arrays(M):
    """Scale arrays that start off a word boundary take the byte-store paths
    (row scales per byte, column scales per byte) with the same results."""
    rng = np.random.default_rng(17)
    v = rng.standard_normal((2560, 384)).astype(np.float32)
    v[rng.random(v.shape) < 0.01] *= 50.0
    _check_quant(M, W.f32_to_bf16_bits(v), 3, scale_offset=1)


def test_quant_every_bf16_pattern(M):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.from_bf16(bits)
    bits = np.where(np.isfinite(f), bits, 0).astype(np.uint16)
    # 2048 x 32: every row-block holds 32 consecutive patterns; also a shuffled copy
    _check_quant(M, bits.reshape(2048, 32), 3)
    rng = np.random.default_rng(5)
    _check_quant(M, rng.permutation(bits).reshape(1024, 64), 3)


def test_quant_edge_cases(M):
    R, C = 64, 128
    v = np.zeros((R, C), np.float32)
    v[0, :32] = 1.0                         # scale 0x77, codes 0x78
    v[1, 0] = 448.0                         # amax 448 -> scale 0x7F
    v[2, 0] = 480.0                         # above 448: the next scale
    v[3, 0], v[3, 1] = 1.0, 2.0 ** -17      # min subnormal code
    v[4, :32] = -1.0
    v[5, :32] = 2.0 ** -130                 # subnormal bf16 block
    v[6, :32] = np.float32(3.0e38)          # near the top of the bf16 range
    v[7, :32] = 1.9375                      # significand above 1.75: scale rounds up
    v[8, 0], v[8, 1] = 1.0, 3 * 2.0 ** -18  # ties at subnormal spacing
    v[9, :] = -0.0
    _check_quant(M, W.f32_to_bf16_bits(v), 3)


def test_quant_batched(M):
    rng = np.random.default_rng(9)
    v = rng.standard_normal((3, 128, 96)).astype(np.float32) * np.exp(rng.standard_normal((3, 128, 96))).astype(np.float32)
    _check_quant(M, W.f32_to_bf16_bits(v), 3)
    # whole strips of 1024 rows in every matrix of the batch (the 16-byte column-scale runs)
    v = rng.standard_normal((2, 1536, 256)).astype(np.float32)
    _check_quant(M, W.f32_to_bf16_bits(v), 3)


def _mx_buffers(M, wl):
    return M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=True)


def _run_mx_forward(M, wl, inp, act=0, gather=False):
    buf = _mx_buffers(M, wl)
    for t in (buf.a_q, buf.a_s, buf.at_q, buf.at_s):
        t.fill_(0xAB)
    x, w1, w2 = bf16_tensor(inp["x"]), bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    logits = f32_tensor(inp["logits"])
    # W2_e quantized along n (column-wise blocks of [n, d]) and stored transposed [d, n]
    M.moe_quant_mxfp8(w2, M.MOE_QUANT_COLWISE, None, None, buf.w2t_q, buf.w2t_s)
    mx = dict(a_q=buf.a_q, a_s=buf.a_s, at_q=buf.at_q, at_s=buf.at_s, w2t_q=buf.w2t_q, w2t_s=buf.w2t_s)
    M.moe_route_counts(logits, wl.k, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets, buf.row_of,
                       buf.src_of, buf.M_cap, buf.err, buf.route_ws)
    if gather:
        M.moe_grouped_mlp_fwd(x, w1, w2, buf.offsets, buf.h, buf.a, buf.y,
                              M.MOE_STAGES_FWD | M.MOE_GATHER_ROWS, mx=mx, act=act, src_of=buf.src_of,
                              k=wl.k)
    else:
        M.moe_permute(x, buf.row_of, buf.src_of, buf.offsets, wl.k, wl.E, buf.x_perm)
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, buf.a, buf.y, M.MOE_STAGES_FWD,
                              mx=mx, act=act)
    M.moe_combine(buf.y, buf.row_of, buf.topk_w, wl.k, buf.out)
    torch.cuda.synchronize()
    return buf


MX_CASES = [
    W.small("mx-small", T=600, k=2, E=4, d=256, n=256, seed=41, routing="zipf"),
    W.small("mx-ragged", T=777, k=3, E=6, d=384, n=384, seed=42, routing="normal"),
]


@pytest.mark.parametrize("wl,act,gather",
                         [(c, "swiglu", False) for c in MX_CASES] + [(MX_CASES[1], "geglu", False),
                                                                      (MX_CASES[1], "swiglu", True)],
                         ids=[c.name for c in MX_CASES] + [MX_CASES[1].name + "-geglu",
                                                           MX_CASES[1].name + "-gather"])
def test_fused_quant_epilogue(M, wl, act, gather):
    print(f"fused mx case {wl} act={act} gather={gather}", flush=True)
    inp = W.make_inputs(wl)
    buf = _run_mx_forward(M, wl, inp, act=M.MOE_ACT_GEGLU if act == "geglu" else M.MOE_ACT_SWIGLU,
                          gather=gather)
    end = int(buf.offsets[-1].item())
    # against the oracle: its quantization of the GPU's own bf16 A, bit for bit
    check_fused_copies_vs_oracle(buf.a, end, buf.a_q, buf.a_s, buf.at_q, buf.at_s)
    # GPU-internal extra: the fused codes equal the standalone quantization of the same A
    a_bits = buf.a.view(torch.int16).cpu().numpy().view(np.uint16)
    g = _gpu_quant(M, a_bits[:end], 3)
    assert np.array_equal(buf.a_q.cpu().numpy()[:end], g[0][0])
    assert np.array_equal(buf.a_s.cpu().numpy()[:end], g[1][0])
    assert np.array_equal(buf.at_q.cpu().numpy()[:, :end], g[2][0])
    assert np.array_equal(buf.at_s.cpu().numpy()[:, :end // 32], g[3][0])
    # against the oracle: dequantized codes approximate the oracle's A
    f = O.forward(O.from_bf16(inp["x"]), inp["logits"], O.from_bf16(inp["w1"]),
                  O.from_bf16(inp["w2"]), wl.k, act=act)
    deq = O.mx_dequant(buf.a_q.cpu().numpy()[:end], buf.a_s.cpu().numpy()[:end])
    err = rel_err(deq, f["A"][:end])
    print(f"  dequantized A vs oracle A: {err:.3e}", flush=True)
    assert err <= 6e-2


@pytest.mark.parametrize("wl", MX_CASES, ids=[c.name for c in MX_CASES])
def test_mx_forward_parity(M, wl):
    print(f"mx forward case {wl}", flush=True)
    inp = W.make_inputs(wl)
    buf = _run_mx_forward(M, wl, inp)
    x, w1, w2 = O.from_bf16(inp["x"]), O.from_bf16(inp["w1"]), O.from_bf16(inp["w2"])
    f = O.forward(x, inp["logits"], w1, w2, wl.k)
    end = int(f["offsets"][-1])
    a_q, a_s, _, _ = O.quant_mxfp8(f["A"], rowwise=True, colwise=False)
    w2t_q = np.stack([O.quant_mxfp8(w2[e], rowwise=False, colwise=True)[2] for e in range(wl.E)])
    w2t_s = np.stack([O.quant_mxfp8(w2[e], rowwise=False, colwise=True)[3] for e in range(wl.E)])
    assert np.array_equal(buf.w2t_q.cpu().numpy(), w2t_q)
    assert np.array_equal(buf.w2t_s.cpu().numpy(), w2t_s)
    Y = O.mx_fc2(a_q, a_s, w2t_q, w2t_s, f["counts"], f["offsets"])
    out = O.combine(Y, f["row_of"], wl.k, f["topk_w"])
    e1 = rel_err(bf16_values(buf.y)[:end], Y[:end])
    e2 = rel_err(bf16_values(buf.out), out)
    e3 = rel_err(bf16_values(buf.out), f["out"])
    print(f"  Y {e1:.3e}  out {e2:.3e}  out vs bf16 path {e3:.3e}", flush=True)
    assert e1 <= 6e-2 and e2 <= 6e-2 and e3 <= 6e-2


def test_mx_fc2_on_identical_codes(M):
    """FC2 stage alone: the codes of both operands are the same on both sides
    (the quantization is bit-exact), so only the summation order differs."""
    wl = W.small("mx-fc2", T=512, k=2, E=4, d=512, n=256, seed=43, routing="zipf")
    inp = W.make_inputs(wl)
    idx, w = O.route(inp["logits"], wl.k)
    M_cap = O.capacity_rows(wl.T, wl.k, wl.E)
    counts, offsets, row_of, src_of = O.layout(idx, wl.E, M_cap)
    rng = np.random.default_rng(7)
    a = rng.standard_normal((M_cap, wl.n)).astype(np.float32)
    a[src_of < 0] = 0.0
    a_bits = W.f32_to_bf16_bits(a)
    buf = _mx_buffers(M, wl)
    g = _gpu_quant(M, a_bits, 1)
    buf.a_q.copy_(torch.from_numpy(g[0][0]))
    buf.a_s.copy_(torch.from_numpy(g[1][0]))
    M.moe_quant_mxfp8(bf16_tensor(inp["w2"]), M.MOE_QUANT_COLWISE, None, None, buf.w2t_q, buf.w2t_s)
    buf.offsets.copy_(torch.from_numpy(offsets))
    mx = dict(a_q=buf.a_q, a_s=buf.a_s, w2t_q=buf.w2t_q, w2t_s=buf.w2t_s)
    M.moe_grouped_mlp_fwd(None, bf16_tensor(inp["w1"]), None, buf.offsets, None, buf.a, buf.y,
                          M.MOE_STAGE_FC2, mx=mx)
    torch.cuda.synchronize()
    a_q, a_s, _, _ = O.quant_mxfp8(O.from_bf16(a_bits), rowwise=True, colwise=False)
    assert np.array_equal(g[0][0], a_q) and np.array_equal(g[1][0], a_s)
    w2 = O.from_bf16(inp["w2"])
    w2t_q = np.stack([O.quant_mxfp8(w2[e], rowwise=False, colwise=True)[2] for e in range(wl.E)])
    w2t_s = np.stack([O.quant_mxfp8(w2[e], rowwise=False, colwise=True)[3] for e in range(wl.E)])
    Y = O.mx_fc2(a_q, a_s, w2t_q, w2t_s, counts, offsets)
    end = int(offsets[-1])
    err = rel_err(bf16_values(buf.y)[:end], Y[:end])
    print(f"  MX FC2 on identical codes: {err:.3e}", flush=True)
    assert err <= 1e-2


FC1_MX_CASES = [
    W.small("mx1-small", T=600, k=2, E=4, d=256, n=256, seed=41, routing="zipf"),
    W.small("mx1-empty", T=300, k=2, E=16, d=384, n=128, seed=22, routing="zipf"),
]


@pytest.mark.parametrize("wl,act", [(c, "swiglu") for c in FC1_MX_CASES] + [(FC1_MX_CASES[0], "geglu")],
                         ids=[c.name for c in FC1_MX_CASES] + [FC1_MX_CASES[0].name + "-geglu"])
def test_mx_fc1_forward_parity(M, wl, act):
    """FC1 on MXFP8 too: X_perm and W1 copies bit-exact against the oracle's
    quantization, H and A from identical codes within 2e-2 (one bf16 rounding;
    the scaled MFMA's own deviation is ~1e-4), Y and out within 6e-2 of the
    oracle's MXFP8 forward (a few A codes may round differently)."""
    print(f"mx fc1 case {wl} act={act}", flush=True)
    inp = W.make_inputs(wl)
    buf = _mx_buffers(M, wl)
    for name in ("h", "a", "y", "out"):
        getattr(buf, name).fill_(float("nan"))
    x, w1, w2 = bf16_tensor(inp["x"]), bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    buf.quantize_weights(w1, w2)
    gact = M.MOE_ACT_GEGLU if act == "geglu" else M.MOE_ACT_SWIGLU
    M.forward(buf, x, f32_tensor(inp["logits"]), w1, w2, act=gact, mx=True)
    torch.cuda.synchronize()
    xo, w1o, w2o = O.from_bf16(inp["x"]), O.from_bf16(inp["w1"]), O.from_bf16(inp["w2"])
    f = O.forward(xo, inp["logits"], w1o, w2o, wl.k, act=act)
    m = O.mlp_forward_mx(f["x_perm"], w1o, w2o, f["counts"], f["offsets"], act=act)
    end = int(f["offsets"][-1])
    assert np.array_equal(buf.x_q.cpu().numpy()[:end], m["x_q"])
    assert np.array_equal(buf.x_s.cpu().numpy()[:end], m["x_s"])
    assert np.array_equal(buf.w1t_q.cpu().numpy(), m["w1t_q"])
    assert np.array_equal(buf.w1t_s.cpu().numpy(), m["w1t_s"])
    # the column-wise X copy made in the same pass (the FC1 wgrad operand)
    _, _, xt_q, xt_s = O.quant_mxfp8(f["x_perm"][:end], rowwise=False, colwise=True)
    assert np.array_equal(buf.xt_q.cpu().numpy()[:, :end], xt_q)
    assert np.array_equal(buf.xt_s.cpu().numpy()[:, :end // 32], xt_s)
    for name, got, ref, tol in (("H", bf16_values(buf.h)[:end], m["H"][:end], 2e-2),
                                ("A", bf16_values(buf.a)[:end], m["A"][:end], 2e-2),
                                ("Y", bf16_values(buf.y)[:end], m["Y"][:end], 6e-2)):
        assert np.isfinite(got).all(), name
        err = rel_err(got, ref)
        print(f"  {name}: {err:.3e}", flush=True)
        assert err <= tol, (name, err)
    out = O.combine(m["Y"], f["row_of"], wl.k, f["topk_w"])
    err = rel_err(bf16_values(buf.out), out)
    print(f"  out: {err:.3e}", flush=True)
    assert err <= 6e-2
    # the fused A copy equals the oracle's quantization of the GPU's bf16 A, bit for bit
    check_fused_copies_vs_oracle(buf.a, end, buf.a_q, buf.a_s, None, None)
    # extra: and the standalone quantization kernel's copy of the same A
    a_bits = buf.a.view(torch.int16).cpu().numpy().view(np.uint16)
    g = _gpu_quant(M, a_bits[:end], 1)
    assert np.array_equal(buf.a_q.cpu().numpy()[:end], g[0][0])


PQ_CASES = [
    W.small("pq-k1", T=700, k=1, E=4, d=256, n=64, seed=51, routing="zipf"),
    W.small("pq-k3", T=333, k=3, E=6, d=96, n=64, seed=52, routing="normal"),
    W.small("pq-empty", T=200, k=2, E=16, d=160, n=64, seed=53, routing="zipf"),
    W.small("pq-strips", T=1536, k=1, E=4, d=256, n=64, seed=54, routing="zipf"),  # M_cap = 2048
]


@pytest.mark.parametrize("wl", PQ_CASES, ids=[c.name for c in PQ_CASES])
def test_permute_quant_bit_exact(M, wl):
    """The fused permute + quantization equals the oracle's quantization of the
    oracle's permutation, bit for bit, on every row of [0, M_cap) (rows past
    the last region are zero codes), for k = 1 and k > 1 and partial column
    tiles."""
    print(f"permute-quant case {wl}", flush=True)
    inp = W.make_inputs(wl)
    M_cap = M.moe_capacity_rows(wl.T, wl.k, wl.E)
    idx, w = O.route(inp["logits"], wl.k)
    counts, offsets, row_of, src_of = O.layout(idx, wl.E, M_cap)
    x = bf16_tensor(inp["x"])
    so = torch.from_numpy(src_of).cuda()
    d = wl.d
    bufs = [torch.full(shape, 0xAB, dtype=U8, device="cuda")
            for shape in ((M_cap, d), (M_cap, d // 32), (d, M_cap), (d, M_cap // 32))]
    M.moe_permute_quant_mxfp8(x, so, wl.k, wl.E, 3, *bufs)
    torch.cuda.synchronize()
    xp = O.permute(O.from_bf16(inp["x"]), row_of, wl.k, M_cap)     # zero rows where src_of < 0
    ref = O.quant_mxfp8(xp, rowwise=True, colwise=True)
    for name, got, want in zip(("row codes", "row scales", "col codes", "col scales"), bufs, ref):
        assert np.array_equal(got.cpu().numpy(), want), name
    # row-wise only and column-wise only give the same bytes
    for mode in (1, 2):
        part = [torch.full_like(b_, 0xAB) for b_ in bufs]
        M.moe_permute_quant_mxfp8(x, so, wl.k, wl.E, mode, *(part if mode == 3 else
                                  (part[0], part[1], None, None) if mode == 1 else (None, None, part[2], part[3])))
        torch.cuda.synchronize()
        sel = (0, 1) if mode == 1 else (2, 3)
        for i in sel:
            assert np.array_equal(part[i].cpu().numpy(), ref[i]), (mode, i)



GQ_CASES = [MX_CASES[0], MX_CASES[1], FC1_MX_CASES[1]]


@pytest.mark.parametrize("wl", GQ_CASES, ids=[c.name for c in GQ_CASES])
def test_groupgemm_quantize_fc2(M, wl):
    """GroupGemm + Quantize: the FC2 epilogue's row-wise MXFP8 copy of Y and its
    transposed column-wise copy equal, bit for bit, the oracle's quantization of the
    GPU's own bf16 Y, on the bf16 FC2 (plain FC1, mx given only for the copies) and on
    the MXFP8 FC2; the bf16 Y beside them is unchanged, and with y = NULL the copies
    alone are written (the same bytes)."""
    print(f"groupgemm+quantize case {wl}", flush=True)
    inp = W.make_inputs(wl)
    x, w1, w2 = bf16_tensor(inp["x"]), bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    logits = f32_tensor(inp["logits"])
    buf = _mx_buffers(M, wl)
    M.moe_route_counts(logits, wl.k, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets, buf.row_of,
                       buf.src_of, buf.M_cap, buf.err, buf.route_ws)
    M.moe_permute(x, buf.row_of, buf.src_of, buf.offsets, wl.k, wl.E, buf.x_perm)
    M.moe_quant_mxfp8(w2, M.MOE_QUANT_COLWISE, None, None, buf.w2t_q, buf.w2t_s)
    end = int(buf.offsets[-1].item())
    for fc2_mx in (False, True):
        # reference: the same FC2 without the quantized copy
        mx0 = dict(a_q=buf.a_q, a_s=buf.a_s, w2t_q=buf.w2t_q, w2t_s=buf.w2t_s) if fc2_mx else None
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, buf.a, buf.y, M.MOE_STAGES_FWD,
                              mx=mx0)
        y_ref = buf.y.clone()
        for t in (buf.y_q, buf.y_s, buf.yt_q, buf.yt_s):
            t.fill_(0xAB)
        buf.y.fill_(float("nan"))
        mx1 = dict(mx0 or {}, y_q=buf.y_q, y_s=buf.y_s, yt_q=buf.yt_q, yt_s=buf.yt_s)
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, buf.a, buf.y, M.MOE_STAGES_FWD,
                              mx=mx1)
        torch.cuda.synchronize()
        assert torch.equal(buf.y[:end], y_ref[:end]), "bf16 Y changed"
        check_fused_copies_vs_oracle(buf.y, end, buf.y_q, buf.y_s, buf.yt_q, buf.yt_s, "Y")
        q_ref, s_ref = buf.y_q[:end].clone(), buf.y_s[:end].clone()
        qt_ref, st_ref = buf.yt_q[:, :end].clone(), buf.yt_s[:, :end // 32].clone()
        # quantized copies only (no bf16 Y)
        buf.y_q.fill_(0xAB)
        buf.yt_q.fill_(0xAB)
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, None, buf.a, None, M.MOE_STAGE_FC2, mx=mx1)
        torch.cuda.synchronize()
        assert torch.equal(buf.y_q[:end], q_ref) and torch.equal(buf.y_s[:end], s_ref)
        assert torch.equal(buf.yt_q[:, :end], qt_ref) and torch.equal(buf.yt_s[:, :end // 32], st_ref)
        # rows past the last region are never written
        if end < buf.M_cap:
            assert torch.all(buf.y_q[end:] == 0xAB)
            assert torch.all(buf.yt_q[:, end:] == 0xAB)
