"""GPU parity of the router backward (moe_route_bwd) against the oracle.

The chosen experts come from the oracle's routing of the same seeded logits
(the GPU routing equals it bit for bit, tested elsewhere); dS is seeded.
fp32 on the GPU vs fp64 in the oracle: max-abs-normalised error <= 1e-5.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

from ._util import f32_tensor, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


@pytest.mark.parametrize("T,E,k,renorm", [(257, 8, 2, False), (1000, 32, 8, False), (64, 1024, 4, False),
                                          (333, 6, 3, True), (99, 128, 2, True), (16, 64, 64, False)])
def test_route_bwd_parity(M, T, E, k, renorm):
    print(f"route bwd case T={T} E={E} k={k} renorm={renorm}", flush=True)
    rng = np.random.default_rng(T + E + k)
    logits = (2 * rng.standard_normal((T, E))).astype(np.float32)
    ds = rng.standard_normal((T, k)).astype(np.float32)
    idx, _ = O.route(logits, k, renorm)
    ref = O.route_backward(logits, idx, ds, renorm)
    dl = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_route_bwd(f32_tensor(logits), torch.from_numpy(idx).cuda(), f32_tensor(ds), dl, renorm)
    got = dl.cpu().numpy()
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    print(f"  max-abs-normalised error {err:.3e}", flush=True)
    assert err <= 1e-5
    assert np.abs(got.sum(axis=1)).max() <= 1e-5 * max(1.0, np.abs(ref).max())
    if renorm:   # experts not chosen get exactly zero
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert np.all(got[mask] == 0)


def test_route_bwd_single_renormalised_slot_is_zero(M):
    # k = 1 with renormalisation: w = 1 for every logit vector, so dlogits = 0
    T, E = 50, 16
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ds = rng.standard_normal((T, 1)).astype(np.float32)
    idx, _ = O.route(logits, 1, True)
    assert np.all(O.route_backward(logits, idx, ds, True) == 0)
    dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    M.moe_route_bwd(f32_tensor(logits), torch.from_numpy(idx).cuda(), f32_tensor(ds), dl, True)
    assert np.abs(dl.cpu().numpy()).max() <= 1e-6 * np.abs(ds).max()


def test_route_bwd_nonfinite_logits(M):
    T, E, k = 40, 8, 2
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[3, 5] = np.nan
    logits[7, :] = -np.inf
    logits[9, 1] = np.inf
    ds = rng.standard_normal((T, k)).astype(np.float32)
    idx, _ = O.route(np.where(np.isfinite(logits), logits, -np.inf).astype(np.float32), k)
    dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    M.moe_route_bwd(f32_tensor(logits), torch.from_numpy(idx).cuda(), f32_tensor(ds), dl)
    got = dl.cpu().numpy()
    assert np.isfinite(got).all()
    # a non-finite logit has probability 0 and gradient 0; an all -inf row is all zero
    assert got[3, 5] == 0 and got[9, 1] == 0 and np.all(got[7] == 0)
    ok = np.ones(T, bool)
    ok[[3, 7, 9]] = False
    ref = O.route_backward(logits[ok], idx[ok], ds[ok])
    assert rel_err(got[ok], ref) <= 1e-5
