"""Pins for the oracle's routing, layout, permute and combine (CPU only).

Each check ties the oracle to something other than itself: brute-force loops
on tiny inputs, a library softmax, the pages' worked examples, invariants
and closed forms.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_routing_examples.json")


def _idx_from_counts(counts, k=1, seed=0):
    """A top-1 assignment realising the given per-expert counts, shuffled."""
    rng = np.random.default_rng(seed)
    pairs = np.concatenate([np.full(c, e) for e, c in enumerate(counts)]).astype(np.int32)
    rng.shuffle(pairs)
    return pairs.reshape(-1, k)


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("T,E,k", [(37, 8, 2), (64, 5, 3), (16, 32, 8), (9, 4, 4)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[::3, 1] = logits[::3, 2]          # plant exact ties
    idx, w = O.route(logits, k)
    for t in range(T):
        ranked = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        assert list(idx[t]) == ranked[:k]
        mx = max(float(v) for v in logits[t])
        z = [math.exp(float(v) - mx) for v in logits[t]]
        s = math.fsum(z)
        for j in range(k):
            assert abs(w[t, j] - z[ranked[j]] / s) < 1e-15


def test_route_weights_match_library_softmax():
    rng = np.random.default_rng(7)
    logits = (3 * rng.standard_normal((50, 16))).astype(np.float32)
    idx, w = O.route(logits, 4)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=1e-13)
    _, wr = O.route(logits, 4, renorm=True)
    np.testing.assert_allclose(wr.sum(1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)   # slots in descending weight


def test_route_constant_logits_ties_to_lower_index():
    logits = np.zeros((10, 8), dtype=np.float32)
    idx, w = O.route(logits, 3)
    assert (idx == np.array([0, 1, 2])).all()
    assert np.all(w == 1.0 / 8)
    _, wr = O.route(logits, 3, renorm=True)
    np.testing.assert_allclose(wr, 1.0 / 3, rtol=1e-15)


def test_route_balanced_workload_weights_are_one():
    w = W.small("bal", T=256, k=1, E=8, d=32, n=32, seed=5, routing="balanced")
    logits = W.make_inputs(w, ("logits",))["logits"]
    idx, wt = O.route(logits, 1)
    assert (idx[:, 0] == np.arange(256) // 32).all()
    assert np.all(wt.astype(np.float32) == 1.0)


def test_route_zipf_workload_leaves_experts_empty():
    """Skewed workload: several experts receive no tokens at all."""
    w = W.WORKLOADS["skewed"]
    logits = W.make_inputs(w, ("logits",))["logits"]
    idx, _ = O.route(logits, w.k)
    counts = np.bincount(idx.reshape(-1), minlength=w.E)
    assert counts.sum() == w.T * w.k
    assert (counts == 0).sum() >= 3
    assert counts.max() == w.T                 # some experts see every token


def test_route_uniform_routing_is_balanced_in_distribution():
    """iid logits: every k-subset equally likely, so counts ~ T*k/E each."""
    w = W.WORKLOADS["train"]
    logits = W.make_inputs(w, ("logits",))["logits"]
    idx, _ = O.route(logits, w.k)
    counts = np.bincount(idx.reshape(-1), minlength=w.E)
    expect = w.T * w.k / w.E
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 80.0                           # 31 dof; p ~ 1e-5 threshold


# ---------------------------------------------------------------- layout
@pytest.mark.parametrize("T,E,k", [(40, 6, 2), (300, 8, 2), (129, 3, 3), (5, 16, 1)])
def test_layout_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = O.route(logits, k)
    M_cap = O.capacity_rows(T, k, E)
    counts, offsets, row_of, src_of = O.layout(idx, E, M_cap)
    seen = [0] * E
    off = [0]
    cnt = [0] * E
    for p in range(T * k):
        cnt[int(idx.reshape(-1)[p])] += 1
    for e in range(E):
        off.append(off[-1] + 128 * ((cnt[e] + 127) // 128))
    assert list(counts) == cnt and list(offsets) == off
    for p in range(T * k):
        e = int(idx.reshape(-1)[p])
        assert row_of[p] == off[e] + seen[e]
        seen[e] += 1
    assert src_of.size == M_cap
    for r in range(M_cap):
        expect = -1
        for p in range(T * k):
            if row_of[p] == r:
                expect = p
        assert src_of[r] == expect
    assert off[-1] <= M_cap


def test_layout_capacity_is_worst_case():
    T, k, E = 1000, 4, 16
    for seed in range(5):
        rng = np.random.default_rng(seed)
        # adversarial: every expert gets count = 1 mod 128 when possible
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx, _ = O.route(logits, k)
        _, offsets, _, _ = O.layout(idx, E)
        assert offsets[-1] <= O.capacity_rows(T, k, E)
    # the bound is reached when every count is 1 mod 128 past a multiple
    counts = [129] * 8
    idx = _idx_from_counts(counts)
    _, offsets, _, _ = O.layout(idx, 8)
    assert offsets[-1] == 8 * 256
    assert O.capacity_rows(idx.size, 1, 8) >= 8 * 256


# ---------------------------------------------------------------- page examples
def test_page_ragged_grid_layout():
    g = json.load(open(GOLDEN))
    counts = g["ragged_grid"]["counts"]
    idx = _idx_from_counts(counts)
    c, off1, row_of, src_of = O.layout(idx, len(counts), align=1)
    assert list(c) == counts
    assert list(np.diff(off1)) == counts            # ragged rows, no gaps
    c, off, _, _ = O.layout(idx, len(counts), align=g["alignment"]["align"])
    assert all(o % 128 == 0 for o in off)
    assert list(np.diff(off)) == [128] * 4          # each group fits one 128-row block


def test_page_dropless_contiguous_buffer():
    g = json.load(open(GOLDEN))["dropless_vs_capacity"]
    counts = g["counts"]
    idx = _idx_from_counts(counts, seed=3)
    c, off, row_of, src_of = O.layout(idx, 3, align=1)
    # dropless: all 23 tokens land in one buffer with no gaps and no drops
    assert off[-1] == sum(counts) == 23
    assert sorted(row_of.tolist()) == list(range(23))
    assert (src_of >= 0).all()
    # the capacity-10 layout of the same page would waste and drop
    cap = g["capacity"]
    assert [max(cap - x, 0) for x in counts] == g["capacity_wasted_slots"]
    assert [max(x - cap, 0) for x in counts] == g["capacity_dropped_tokens"]


def test_page_empty_group_passes_through():
    g = json.load(open(GOLDEN))["empty_group"]
    local = g["gpu1_local_counts"]
    # local experts (E2, E3) of GPU 1 as experts 0 and 1 of a 2-expert layout
    idx = _idx_from_counts(local)
    c, off, row_of, src_of = O.layout(idx, 2)
    assert list(c) == local
    assert off[2] == off[1]                          # empty expert: zero rows
    assert off[1] == 128


# ---------------------------------------------------------------- permute/combine
def test_permute_unpermute_identity():
    rng = np.random.default_rng(11)
    T, E, k, d = 77, 6, 3, 24
    x = O.round_bf16(rng.standard_normal((T, d)))
    idx, _ = O.route(rng.standard_normal((T, E)).astype(np.float32), k)
    M_cap = O.capacity_rows(T, k, E)
    counts, offsets, row_of, src_of = O.layout(idx, E, M_cap)
    xp = O.permute(x, row_of, k, M_cap)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xp[row_of[t * k + j]], x[t])
    pad = src_of < 0
    assert np.all(xp[pad] == 0.0)
    # unit weights, k a power of two: combine(permute(x)) = k*x exactly
    k2 = 2
    idx2, _ = O.route(rng.standard_normal((T, E)).astype(np.float32), k2)
    c2, o2, r2, s2 = O.layout(idx2, E)
    xp2 = O.permute(x, r2, k2, int(o2[-1]))
    assert np.array_equal(O.combine(xp2, r2, k2, None), 2 * x)


def test_combine_weights_in_slot_order():
    T, k, d = 4, 3, 5
    y = np.arange(T * k * d, dtype=np.float64).reshape(T * k, d)
    row_of = np.arange(T * k)[::-1].copy()
    w = np.array([[1.0, 2.0, 4.0]] * T)
    out = O.combine(y, row_of, k, w, rounding=False)
    for t in range(T):
        ref = sum(w[t, j] * y[row_of[t * k + j]] for j in range(k))
        assert np.array_equal(out[t], ref)


# ---------------------------------------------------------------- bf16 codec
def test_bf16_rounding_against_float32_bit_rounding():
    """fp64 -> bf16 (direct) agrees with fp32 -> bf16 whenever the fp64 value
    is already an fp32 value; checked over every fp32 exponent."""
    rng = np.random.default_rng(0)
    mant = rng.integers(0, 1 << 23, 4096, dtype=np.uint32)
    exps = rng.integers(1, 254, 4096, dtype=np.uint32)
    bits = (exps << np.uint32(23)) | mant
    bits[:64] = (np.uint32(120) << np.uint32(23)) | (np.arange(64, dtype=np.uint32) << np.uint32(15)) | np.uint32(0x4000)
    f = bits.view(np.float32)
    assert np.array_equal(O.bf16_bits(f.astype(np.float64)), W.f32_to_bf16_bits(f))
    assert np.array_equal(O.from_bf16(O.bf16_bits(f)), O.round_bf16(f))
    # ties to even at the 1.0 binade
    assert O.round_bf16(1 + 2 ** -8) == 1.0
    assert O.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
