"""Parity at the full workload sizes, in the launch configuration bench.py times.

The GPU runs the whole forward + backward at full size. The oracle then runs
on what it can finish in seconds and that still determines individual outputs
exactly:
  * routing and layout of ALL tokens (bit-exact);
  * the whole path for a sample of tokens: every per-row result of a token
    (H, A, Y rows of its pairs, out, dS, dH, A', dX_perm rows, dX) depends only
    on that token, so the oracle run on the sampled tokens alone gives the
    reference values;
  * weight gradients of one 32-column activation block of the busiest expert:
    SwiGLU is column-wise, so the MLP restricted to that block over all of the
    expert's rows gives dW1[:, block] and dW2[block, :] exactly;
  * properties at any size: padding rows zero, empty experts' dW exactly 0.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

from ._util import bf16_tensor, bf16_values, check_fused_copies_vs_oracle, f32_tensor, rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _gpu(M, wl, inp, mx=False, gather=False):
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=mx)
    x, w1, w2, dout = (bf16_tensor(inp[key]) for key in ("x", "w1", "w2", "dout"))
    logits = f32_tensor(inp["logits"])
    if mx:
        M.moe_quant_mxfp8(w2, M.MOE_QUANT_COLWISE, None, None, buf.w2t_q, buf.w2t_s)
        mxd = dict(a_q=buf.a_q, a_s=buf.a_s, at_q=buf.at_q, at_s=buf.at_s, w2t_q=buf.w2t_q,
                   w2t_s=buf.w2t_s)
        M.moe_route_counts(logits, wl.k, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets,
                           buf.row_of, buf.src_of, buf.M_cap, buf.err, buf.route_ws)
        M.moe_permute(x, buf.row_of, buf.src_of, buf.offsets, wl.k, wl.E, buf.x_perm)
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, buf.a, buf.y,
                              M.MOE_STAGES_FWD, mx=mxd)
        M.moe_combine(buf.y, buf.row_of, buf.topk_w, wl.k, buf.out)
    else:
        M.forward(buf, x, logits, w1, w2, gather=gather)
        M.backward(buf, dout, w1, w2, x=x if gather else None)
    torch.cuda.synchronize()
    return buf


def _oracle_tokens(wl, inp, ts, mx=False):
    """The oracle's forward/backward on the tokens ts (experts compacted)."""
    idx, w = O.route(inp["logits"][ts], wl.k)
    used = np.unique(idx)
    remap = np.full(wl.E, -1, np.int64)
    remap[used] = np.arange(used.size)
    idx_c = remap[idx]
    w1 = O.from_bf16(inp["w1"][used])
    w2 = O.from_bf16(inp["w2"][used])
    M_cap = O.capacity_rows(len(ts), wl.k, used.size)
    counts, offsets, row_of, src_of = O.layout(idx_c, used.size, M_cap)
    x_perm = O.permute(O.from_bf16(inp["x"][ts]), row_of, wl.k, M_cap)
    H, A, Y = O.mlp_forward(x_perm, w1, w2, counts, offsets)
    r = dict(idx=idx, w=w, row_of=row_of, H=H, A=A, Y=Y, used=used)
    if mx:
        a_q, a_s, _, _ = O.quant_mxfp8(A, rowwise=True, colwise=False)
        cols = [O.quant_mxfp8(w2[e], rowwise=False, colwise=True) for e in range(used.size)]
        r["w2t_q"] = np.stack([c[2] for c in cols])
        r["w2t_s"] = np.stack([c[3] for c in cols])
        Y = O.mx_fc2(a_q, a_s, r["w2t_q"], r["w2t_s"], counts, offsets)
        r["Y"] = Y
    r["out"] = O.combine(Y, row_of, wl.k, w)
    if not mx:
        b = O.mlp_backward(x_perm, w1, w2, H, Y, O.from_bf16(inp["dout"][ts]), w, counts, offsets,
                           row_of, src_of, wl.k)
        r.update(b)
    return r


def _oracle_block_wgrad(wl, inp, idx, w, e, blk):
    """dW1[e][:, gate/up of block blk] and dW2[e][blk rows, :] over all rows of e."""
    pairs = np.nonzero(idx.reshape(-1) == e)[0]        # ascending pair order = row order
    toks = pairs // wl.k
    c = pairs.size
    g = O.GLU_INTERLEAVE
    w1 = O.from_bf16(inp["w1"][e][:, 2 * g * blk:2 * g * (blk + 1)])[None]
    w2 = O.from_bf16(inp["w2"][e][g * blk:g * (blk + 1), :])[None]
    x_perm = O.from_bf16(inp["x"][toks])
    counts = np.array([c]); offsets = np.array([0, c])
    H, A, Y = O.mlp_forward(x_perm, w1, w2, counts, offsets)
    b = O.mlp_backward(x_perm, w1, w2, H, Y, O.from_bf16(inp["dout"][toks]),
                       w.reshape(-1)[pairs][:, None], counts, offsets, np.arange(c), np.arange(c), 1)
    return b["dW1"][0], b["dW2"][0]


def _sample_tokens(wl, idx, counts, rng, n=12):
    """Tokens spread over experts, including one routed to the busiest expert's last rows."""
    ts = set(rng.choice(wl.T, size=n - 2, replace=False).tolist())
    flat = idx.reshape(-1)
    e_big = int(np.argmax(counts))
    pairs = np.nonzero(flat == e_big)[0]
    ts.add(int(pairs[-1] // wl.k))                    # last real row of the busiest expert
    ts.add(int(pairs[len(pairs) // 2] // wl.k))
    return np.array(sorted(ts))


@pytest.mark.parametrize("name,gather", [("balanced", False), ("skewed", False), ("train", False),
                                         ("skewed", True), ("skewed-large", False)],
                         ids=["balanced", "skewed", "train", "skewed-gather", "skewed-large"])
def test_fullsize_forward_backward(M, name, gather):
    wl = W.WORKLOADS[name]
    print(f"full-size case {wl} gather={gather}", flush=True)
    inp = W.make_inputs(wl)
    buf = _gpu(M, wl, inp, gather=gather)
    # routing and layout of every token
    idx, w = O.route(inp["logits"], wl.k)
    M_cap = O.capacity_rows(wl.T, wl.k, wl.E)
    counts, offsets, row_of, src_of = O.layout(idx, wl.E, M_cap)
    assert np.array_equal(buf.topk_idx.cpu().numpy(), idx)
    assert np.array_equal(buf.counts.cpu().numpy(), counts)
    assert np.array_equal(buf.offsets.cpu().numpy(), offsets)
    assert np.array_equal(buf.row_of.cpu().numpy(), row_of)
    assert np.array_equal(buf.src_of.cpu().numpy(), src_of)
    assert int(buf.err.item()) == 0
    if name.startswith("skewed"):
        assert (counts == 0).sum() >= 3
    if name == "skewed-large":   # permuted tensors past 2^31 bytes
        assert buf.M_cap * wl.d * 2 >= 2 ** 31
    # per-token results on a sample
    rng = np.random.default_rng(wl.seed)
    ts = _sample_tokens(wl, idx, counts, rng)
    r = _oracle_tokens(wl, inp, ts)
    g_rows = row_of.reshape(wl.T, wl.k)[ts].reshape(-1)       # full-size rows of the sampled pairs
    o_rows = r["row_of"]
    for key, gt, ref in (("H", buf.h, r["H"]), ("A", buf.a, r["A"]), ("Y", buf.y, r["Y"]),
                         ("dH", buf.dh, r["dH"]), ("A'", buf.a_w, r["a_w"]),
                         ("dX_perm", buf.dx_perm, r["dx_perm"])):
        got = bf16_values(gt[torch.from_numpy(g_rows).long().cuda()])
        err = rel_err(got, ref[o_rows])
        print(f"  {key}: {err:.3e}", flush=True)
        assert err <= TOL, key
    tsel = torch.from_numpy(ts).long().cuda()
    for key, got, ref in (("out", bf16_values(buf.out[tsel]), r["out"]),
                          ("dX", bf16_values(buf.dx[tsel]), r["dx"]),
                          ("dS", buf.ds[tsel].cpu().numpy(), r["dS"])):
        err = rel_err(got, ref)
        print(f"  {key}: {err:.3e}", flush=True)
        assert err <= TOL, key
    # weight gradients: one column block of the busiest expert
    e_big = int(np.argmax(counts))
    blk = int(rng.integers(wl.n // O.GLU_INTERLEAVE))
    dW1_b, dW2_b = _oracle_block_wgrad(wl, inp, idx, w, e_big, blk)
    g = O.GLU_INTERLEAVE
    got1 = buf.dw1[e_big][:, 2 * g * blk:2 * g * (blk + 1)].cpu().numpy()
    got2 = buf.dw2[e_big][g * blk:g * (blk + 1), :].cpu().numpy()
    e1, e2 = rel_err(got1, dW1_b), rel_err(got2, dW2_b)
    print(f"  dW1 block: {e1:.3e}  dW2 block: {e2:.3e}", flush=True)
    assert e1 <= TOL and e2 <= TOL
    # properties at full size
    pad = src_of[:int(offsets[-1])] < 0
    if pad.any():
        prow = torch.from_numpy(np.nonzero(pad)[0][:512]).long().cuda()
        for t in (buf.h, buf.a, buf.y, buf.dh, buf.a_w, buf.dx_perm) + (() if gather else (buf.x_perm,)):
            assert torch.all(t[prow].float() == 0)
    for e in np.nonzero(counts == 0)[0]:
        assert torch.all(buf.dw1[e] == 0) and torch.all(buf.dw2[e] == 0)


def _oracle_tokens_mx(wl, inp, ts):
    """The oracle's MXFP8 forward and backward (every GEMM on MXFP8) on the tokens ts.
    Row-wise copies are per row, so these rows equal the full-size ones; the
    column-wise copies (wgrads) mix rows and are checked separately."""
    idx, w = O.route(inp["logits"][ts], wl.k)
    used = np.unique(idx)
    remap = np.full(wl.E, -1, np.int64)
    remap[used] = np.arange(used.size)
    w1 = O.from_bf16(inp["w1"][used])
    w2 = O.from_bf16(inp["w2"][used])
    M_cap = O.capacity_rows(len(ts), wl.k, used.size)
    counts, offsets, row_of, src_of = O.layout(remap[idx], used.size, M_cap)
    x_perm = O.permute(O.from_bf16(inp["x"][ts]), row_of, wl.k, M_cap)
    f = O.mlp_forward_mx(x_perm, w1, w2, counts, offsets)
    r = dict(idx=idx, w=w, row_of=row_of, used=used, **f)
    r["out"] = O.combine(f["Y"], row_of, wl.k, w)
    b = O.mlp_backward_mx(x_perm, w1, w2, f["H"], f["Y"], O.from_bf16(inp["dout"][ts]), w, counts,
                          offsets, row_of, src_of, wl.k, dgrad2_mx=True)
    for key in ("dS", "dH", "a_w", "dx_perm", "dx"):
        r[key] = b[key]
    return r


def test_fullsize_mxfp8_step(M):
    """The mxfp8 workload as bench.py runs it: fused permute + quantization,
    MX FC1 + SwiGLU + MXFP8 A, MX FC2, combine, then the MX FC2 dgrad + dGLU
    with MXFP8 dH / A', MX wgrads and MX FC1 dgrad, and the router backward."""
    wl = W.WORKLOADS["mxfp8"]
    print(f"full-size case {wl} (every GEMM on MXFP8)", flush=True)
    inp = W.make_inputs(wl)
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=True)
    x, w1, w2, dout = (bf16_tensor(inp[key]) for key in ("x", "w1", "w2", "dout"))
    logits = f32_tensor(inp["logits"])
    buf.quantize_weights(w1, w2)
    M.forward(buf, x, logits, w1, w2, mx=True)
    M.backward(buf, dout, w1, w2, logits=logits, mx=True)
    torch.cuda.synchronize()
    idx, w = O.route(inp["logits"], wl.k)
    M_cap = O.capacity_rows(wl.T, wl.k, wl.E)
    counts, offsets, row_of, src_of = O.layout(idx, wl.E, M_cap)
    assert np.array_equal(buf.offsets.cpu().numpy(), offsets)
    assert np.array_equal(buf.row_of.cpu().numpy(), row_of)
    rng = np.random.default_rng(wl.seed)
    # tokens of two experts keep the oracle's weight quantization small
    ts = np.concatenate([rng.choice(np.arange(0, 4096), 5, replace=False),
                         rng.choice(np.arange(28672, 32768), 5, replace=False)])
    ts.sort()
    r = _oracle_tokens_mx(wl, inp, ts)
    for i, e in enumerate(r["used"]):   # weight copies of the sampled experts
        assert np.array_equal(buf.w1t_q[e].cpu().numpy(), r["w1t_q"][i])
        assert np.array_equal(buf.w2t_q[e].cpu().numpy(), r["w2t_q"][i])
    g_rows = row_of.reshape(wl.T, wl.k)[ts].reshape(-1)
    gsel = torch.from_numpy(g_rows).long().cuda()
    o_rows = r["row_of"]
    assert np.array_equal(buf.x_q[gsel].cpu().numpy(), r["x_q"][o_rows])   # row-wise X copy
    for key, gt, ref, tol in (("H", buf.h, r["H"], 2e-2), ("A", buf.a, r["A"], 2e-2),
                              ("Y", buf.y, r["Y"], 6e-2), ("dH", buf.dh, r["dH"], 2e-2),
                              ("A'", buf.a_w, r["a_w"], 2e-2), ("dX_perm", buf.dx_perm, r["dx_perm"], 6e-2)):
        err = rel_err(bf16_values(gt[gsel]), ref[o_rows])
        print(f"  {key}: {err:.3e}", flush=True)
        assert err <= tol, key
    tsel = torch.from_numpy(ts).long().cuda()
    for key, got, ref, tol in (("out", bf16_values(buf.out[tsel]), r["out"], 6e-2),
                               ("dX", bf16_values(buf.dx[tsel]), r["dx"], 6e-2),
                               ("dS", buf.ds[tsel].cpu().numpy(), r["dS"], 2e-2)):
        err = rel_err(got, ref)
        print(f"  {key}: {err:.3e}", flush=True)
        assert err <= tol, key
    # every fused MXFP8 copy over the whole region of expert 0 (rows 0..4095):
    # the oracle's quantization of the GPU's own bf16 A, dH and A', bit for bit
    check_fused_copies_vs_oracle(buf.a[:4096], 4096, buf.a_q, buf.a_s, None, None, "A (expert 0)")
    check_fused_copies_vs_oracle(buf.dh[:4096], 4096, buf.dh_q, buf.dh_s, buf.dht_q, buf.dht_s,
                                 "dH (expert 0)")
    check_fused_copies_vs_oracle(buf.a_w[:4096], 4096, None, None, buf.awt_q, buf.awt_s, "A' (expert 0)")
    # column-wise copies of two 32-row blocks of expert 0: X from the oracle's
    # permutation, dH and A' from the GPU's own bf16 values (bit-exact)
    xp = O.from_bf16(inp["x"][:4096])          # expert 0 holds tokens 0..4095 in order
    for blk in (0, 77):
        r0 = 32 * blk
        rows = slice(r0, r0 + 32)
        _, _, q, sc = O.quant_mxfp8(xp[rows], rowwise=False, colwise=True)
        assert np.array_equal(buf.xt_q[:, rows].cpu().numpy(), q)
        assert np.array_equal(buf.xt_s[:, blk].cpu().numpy(), sc[:, 0])
        _, _, q, sc = O.quant_mxfp8(bf16_values(buf.dh[rows]), rowwise=False, colwise=True)
        assert np.array_equal(buf.dht_q[:, rows].cpu().numpy(), q)
        _, _, q, sc = O.quant_mxfp8(bf16_values(buf.a_w[rows]), rowwise=False, colwise=True)
        assert np.array_equal(buf.awt_q[:, rows].cpu().numpy(), q)
    # MX wgrads of one 64-column block of expert 0, on the GPU's own codes
    e, R = 0, slice(0, 4096)
    cb = slice(64 * 5, 64 * 6)
    xt = O.mx_dequant(buf.xt_q[:, R].cpu().numpy(), buf.xt_s[:, :128].cpu().numpy())
    dht = O.mx_dequant(buf.dht_q[cb, R].cpu().numpy(), buf.dht_s[cb, :128].cpu().numpy())
    e1 = rel_err(buf.dw1[e][:, cb].cpu().numpy(), xt @ dht.T)
    awt = O.mx_dequant(buf.awt_q[32 * 5:32 * 6, R].cpu().numpy(), buf.awt_s[32 * 5:32 * 6, :128].cpu().numpy())
    dyt = O.mx_dequant(buf.dyt_q[:, R].cpu().numpy(), buf.dyt_s[:, :128].cpu().numpy())
    e2 = rel_err(buf.dw2[e][32 * 5:32 * 6, :].cpu().numpy(), awt @ dyt.T)
    print(f"  MX dW1 block (own codes): {e1:.3e}  MX dW2 block: {e2:.3e}", flush=True)
    assert e1 <= 1e-3 and e2 <= 1e-3
