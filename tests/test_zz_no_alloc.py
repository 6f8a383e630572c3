"""The allocation-free routing entry point (moe_route_counts_noalloc) against
moe_route_counts with a caller workspace: the same kernels on the library's
static scratch, so every output must match bit for bit. Two calls in a row,
the second with a smaller input (the scratch keeps the first call's contents,
which must not leak into the second), and both against the oracle's routing
and layout as well."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

from ._util import f32_tensor

pytestmark = pytest.mark.gpu

KEYS = ("topk_idx", "topk_w", "counts", "offsets", "row_of", "src_of", "err")


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _bufs(M, T, E, k):
    cap = M.moe_capacity_rows(T, k, E)
    dev = "cuda"
    return cap, dict(
        topk_idx=torch.full((T, k), -7, dtype=torch.int32, device=dev),
        topk_w=torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
        counts=torch.full((E,), -7, dtype=torch.int32, device=dev),
        offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
        row_of=torch.full((T * k,), -7, dtype=torch.int32, device=dev),
        src_of=torch.full((cap,), 12345, dtype=torch.int32, device=dev),
        err=torch.zeros(1, dtype=torch.int32, device=dev),
    )


def _run(M, lg, k, noalloc, renorm=False):
    T, E = lg.shape
    cap, b = _bufs(M, T, E, k)
    args = (f32_tensor(lg), k, b["topk_idx"], b["topk_w"], b["counts"], b["offsets"], b["row_of"],
            b["src_of"], cap, b["err"])
    if noalloc:
        M.moe_route_counts_noalloc(*args, renorm=renorm)
    else:
        ws = torch.empty(max(16, M.moe_route_workspace_bytes(T, k, E)), dtype=torch.uint8, device="cuda")
        M.moe_route_counts(*args, ws, renorm)
    torch.cuda.synchronize()
    return cap, {key: v.cpu().numpy() for key, v in b.items()}


def _logits(T, E, seed, zipf):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if zipf:
        lg += (-3.0 * 1.2 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    return lg


@pytest.mark.parametrize("renorm", [False, True])
def test_noalloc_route_matches_workspace_route(M, renorm):
    # a routing on the general layout path (1024 experts), then the skewed shape
    # (131072 pairs over 32 experts, fused path), then a smaller one, all on the
    # same scratch
    for (T, E, k, seed, zipf) in ((9000, 1024, 4, 11, False), (16384, 32, 8, 1003, True),
                                  (1000, 12, 3, 7, False)):
        print(f"noalloc route case T={T} E={E} k={k} renorm={renorm}", flush=True)
        lg = _logits(T, E, seed, zipf)
        cap, ref = _run(M, lg, k, noalloc=False, renorm=renorm)
        _, got = _run(M, lg, k, noalloc=True, renorm=renorm)
        for key in KEYS:
            assert np.array_equal(got[key], ref[key]), key      # bitwise, weights included
        idx, w = O.route(lg, k, renorm)
        counts, offsets, row_of, src_of = O.layout(idx, E, cap)
        assert np.array_equal(got["topk_idx"], idx)
        np.testing.assert_allclose(got["topk_w"], w, rtol=2e-6, atol=1e-7)
        for key, want in (("counts", counts), ("offsets", offsets), ("row_of", row_of), ("src_of", src_of)):
            assert np.array_equal(got[key], want), key
        assert got["err"][0] == 0

