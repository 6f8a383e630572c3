"""GPU parity of routing, ragged layout, permute and combine against the oracle.

Integer outputs (top-k indices, counts, offsets, row maps) and permuted rows
must match bit for bit; routing weights and combine outputs within 2e-2 of
the max-abs-normalised error (in practice ~1e-7 and one bf16 rounding).
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

from ._util import bf16_bits, bf16_tensor, bf16_values, f32_tensor, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _route(M, logits_np, k, renorm=False):
    T, E = logits_np.shape
    cap = M.moe_capacity_rows(T, k, E)
    dev = "cuda"
    out = dict(
        topk_idx=torch.empty(T, k, dtype=torch.int32, device=dev),
        topk_w=torch.empty(T, k, dtype=torch.float32, device=dev),
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        row_of=torch.empty(T * k, dtype=torch.int32, device=dev),
        src_of=torch.full((cap,), 12345, dtype=torch.int32, device=dev),
        err=torch.zeros(1, dtype=torch.int32, device=dev),
        ws=torch.empty(max(16, M.moe_route_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev),
    )
    M.moe_route_counts(f32_tensor(logits_np), k, out["topk_idx"], out["topk_w"], out["counts"],
                       out["offsets"], out["row_of"], out["src_of"], cap, out["err"], out["ws"], renorm)
    torch.cuda.synchronize()
    return cap, {key: v.cpu().numpy() for key, v in out.items()}


ROUTE_CASES = [
    # (T, E, k, kind)
    (256, 8, 2, "normal"),
    (1000, 32, 8, "zipf"),
    (333, 5, 3, "normal"),
    (64, 64, 4, "ties"),
    (130, 1, 1, "normal"),
    (2048, 128, 2, "normal"),
    (77, 1024, 6, "normal"),
    (4096, 16, 1, "constant"),
    (5000, 24, 4, "normal"),
    (300, 64, 12, "normal"),     # k > 8: the renormalised weights of slots 8.. are recomputed
    (200, 40, 16, "ties"),
    # the fused two-kernel layout at one GPU's skewed share (512 chunks of 32
    # tokens) and with 2 token passes per chunk (511 chunks of 64 tokens, a
    # partial last one); the general four-kernel layout where the fused pair
    # would need more passes or histogram entries (128 and 1024 experts)
    (16384, 32, 8, "zipf"),
    (32700, 32, 8, "zipf"),
    (20000, 128, 4, "zipf"),
    (9000, 1024, 4, "normal"),
    (500, 256, 8, "ties"),       # 4 logits per lane
    (150, 600, 5, "normal"),     # 16 logits per lane
]


def _logits(T, E, kind, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "zipf":
        lg += (-3.0 * 1.2 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    elif kind == "ties":
        lg = np.round(lg * 2).astype(np.float32)          # many exact ties
    elif kind == "constant":
        lg[:] = 0.5
    return lg


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_and_layout_bit_exact(M, T, E, k, kind):
    print(f"route case T={T} E={E} k={k} {kind}", flush=True)
    lg = _logits(T, E, kind, T * 7 + E)
    for renorm in (False, True):
        cap, g = _route(M, lg, k, renorm)
        idx, w = O.route(lg, k, renorm)
        counts, offsets, row_of, src_of = O.layout(idx, E, cap)
        assert np.array_equal(g["topk_idx"], idx)
        np.testing.assert_allclose(g["topk_w"], w, rtol=2e-6, atol=1e-7)
        assert np.array_equal(g["counts"], counts)
        assert np.array_equal(g["offsets"], offsets)
        assert np.array_equal(g["row_of"], row_of)
        assert np.array_equal(g["src_of"], src_of)      # -1 everywhere else, up to M_cap
        assert g["err"][0] == 0


def test_route_flags_nonfinite_logits(M):
    lg = _logits(64, 8, "normal", 3)
    lg[5, 2] = np.nan
    lg[9, 0] = np.inf
    cap, g = _route(M, lg, 2)
    assert g["err"][0] & M.MOE_ERRBIT_NONFINITE_LOGIT
    assert ((g["topk_idx"] >= 0) & (g["topk_idx"] < 8)).all()
    assert g["offsets"][-1] <= cap
    assert (np.sort(g["row_of"]) == np.unique(g["row_of"])).all()


@pytest.mark.parametrize("E", [64, 32, 16])
@pytest.mark.parametrize("k", [2, 12])
def test_route_nonfinite_logits_renorm(M, k, E):
    """With renormalisation (and k > 8, where slots 8.. take another code path
    with 64 experts; 32 and 16 experts take the ranked top-k) a non-finite logit
    is never preferred and weighs 0, so every weight stays finite in [0, 1] and
    each affected token's weights still sum to 1; rows with only finite logits
    match the oracle exactly as before."""
    T = 96
    lg = _logits(T, E, "normal", 11)
    bad_rows = [3, 17, 40, 50]
    lg[3, 5] = np.nan
    lg[17, :20] = np.inf          # more non-finite logits than k - 8 ...
    lg[40, ::2] = -np.inf         # ... and half of the row
    lg[50, 6:] = np.nan           # fewer finite logits than k: slots 6.. pick non-finite ones
    cap, g = _route(M, lg, k, renorm=True)
    assert g["err"][0] & M.MOE_ERRBIT_NONFINITE_LOGIT
    w = g["topk_w"]
    assert np.isfinite(w).all() and (w >= 0).all() and (w <= 1).all()
    # a row with some finite logit renormalises to 1; a row with none (row 17 at
    # 16 experts) gets weight 0 everywhere
    want = np.isfinite(lg[bad_rows]).any(axis=1).astype(np.float64)
    np.testing.assert_allclose(w[bad_rows].sum(axis=1), want, rtol=1e-5)
    idx = g["topk_idx"]
    assert ((idx >= 0) & (idx < E)).all()
    for t in bad_rows:            # a chosen non-finite logit weighs exactly 0
        chosen = lg[t, idx[t]]
        assert (w[t][~np.isfinite(chosen)] == 0).all()
    good = np.setdiff1d(np.arange(T), bad_rows)
    o_idx, o_w = O.route(lg[good], k, renorm=True)
    assert np.array_equal(idx[good], o_idx)
    np.testing.assert_allclose(w[good], o_w, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("T,E,k,d", [(256, 8, 2, 128), (999, 13, 3, 200), (64, 4, 4, 8),
                                     (4096, 32, 8, 1024)])
def test_permute_and_combine(M, T, E, k, d):
    print(f"permute case T={T} E={E} k={k} d={d}", flush=True)
    rng = np.random.default_rng(T + d)
    lg = _logits(T, E, "zipf", T)
    cap, g = _route(M, lg, k)
    xb = W.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    x = bf16_tensor(xb)
    src_of = torch.from_numpy(g["src_of"]).cuda()
    offsets = torch.from_numpy(g["offsets"]).cuda()
    row_of = torch.from_numpy(g["row_of"]).cuda()
    x_perm = torch.full((cap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_permute(x, row_of, src_of, offsets, k, E, x_perm)
    torch.cuda.synchronize()
    # the oracle derives its own routing and layout from the same logits
    o_idx, o_w = O.route(lg, k)
    _, o_off, o_row_of, _ = O.layout(o_idx, E, cap)
    assert np.array_equal(o_off, g["offsets"])
    ref = O.permute(O.from_bf16(xb), o_row_of, k, cap)
    end = int(g["offsets"][-1])
    got = bf16_bits(x_perm)[:end]
    assert np.array_equal(got, O.bf16_bits(ref[:end]))   # pad rows are exactly +0
    # rows past offsets[E] are untouched (still NaN)
    if end < cap:
        assert torch.isnan(x_perm[end:].float()).all()
    # combine with the routing weights and with unit weights
    w = torch.from_numpy(g["topk_w"]).cuda()
    out = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    for ww, wn in ((w, o_w), (None, None)):
        M.moe_combine(x_perm, row_of, ww, k, out)
        torch.cuda.synchronize()
        ref_o = O.combine(ref, o_row_of, k, wn)
        assert rel_err(bf16_values(out), ref_o) < 2e-2
        # fp32 in-order sum then one rounding: at most 1 bf16 ulp from the fp64 value
        diff = np.abs(bf16_values(out) - ref_o)
        assert np.all(diff <= 2.0 ** -7 * np.abs(ref_o) + 1e-6 * np.abs(ref_o).max())
