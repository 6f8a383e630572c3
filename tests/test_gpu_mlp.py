"""GPU parity of the whole hot path (forward and backward) against the oracle.

Sizes run through several 256 x 256 tiles, ragged expert segments, empty
experts, partial N tiles and the all-tokens-to-one-expert case. Every output
buffer is poisoned with NaN first, so every defined element must be written.
Tolerance: max-abs-normalised error <= 2e-2 per floating tensor; integer and
copied tensors bit-exact; padding rows exactly zero; dW of empty experts 0.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

from ._util import bf16_bits, bf16_tensor, bf16_values, f32_tensor, rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-2

CASES = [
    W.WORKLOADS["tiny"],
    W.small("ragged", T=700, k=3, E=6, d=192, n=320, seed=21, routing="zipf"),
    W.small("empty", T=300, k=2, E=16, d=256, n=128, seed=22, routing="zipf"),
    W.small("wide", T=1200, k=2, E=4, d=512, n=384, seed=23),
    W.small("balanced", T=1024, k=1, E=4, d=256, n=256, seed=24, routing="balanced"),
    # many experts, most of them empty or with equal counts: the ragged-K schedule's
    # sort of experts by rows (300 keys padded to 512), ties and zero-row experts
    W.small("many-experts", T=512, k=4, E=300, d=128, n=64, seed=25, routing="normal"),
]


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _poison(buf):
    for name in ("x_perm", "h", "a", "y", "out", "dy_u", "dh", "a_w", "ds", "dx_perm", "dx",
                 "dw1", "dw2"):
        getattr(buf, name).fill_(float("nan"))


def _run_gpu(M, wl, inp, act=0, gather=False):
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n)
    _poison(buf)
    x = bf16_tensor(inp["x"])
    logits = f32_tensor(inp["logits"])
    w1 = bf16_tensor(inp["w1"])
    w2 = bf16_tensor(inp["w2"])
    dout = bf16_tensor(inp["dout"])
    M.forward(buf, x, logits, w1, w2, act=act, gather=gather)
    M.backward(buf, dout, w1, w2, act=act, x=x if gather else None)
    torch.cuda.synchronize()
    return buf


def _oracle(wl, inp, act="swiglu"):
    x = O.from_bf16(inp["x"])
    w1 = O.from_bf16(inp["w1"])
    w2 = O.from_bf16(inp["w2"])
    f = O.forward(x, inp["logits"], w1, w2, wl.k, act=act)
    b = O.mlp_backward(f["x_perm"], w1, w2, f["H"], f["Y"], O.from_bf16(inp["dout"]), f["topk_w"],
                       f["counts"], f["offsets"], f["row_of"], f["src_of"], wl.k, act=act)
    return f, b


def _check(name, got, ref, rows=None, tol=TOL):
    if rows is not None:
        got, ref = got[:rows], ref[:rows]
    assert np.isfinite(got).all(), f"{name}: unwritten (NaN) or non-finite elements"
    err = rel_err(got, ref)
    print(f"  {name}: max-abs-normalised error {err:.3e}", flush=True)
    assert err <= tol, f"{name}: {err}"


def _random_cases(count, seed):
    """Shapes drawn from a seeded generator: any token count (one token included),
    k up to min(E, 8), 1-48 experts, d and n any multiple of 64 up to 640, each with
    its own routing recipe; they land on partial tiles in M, N and K."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        E = int(rng.integers(1, 49))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = 1 if i == 0 else int(rng.integers(2, 1500))
        d, n = 64 * int(rng.integers(1, 11)), 64 * int(rng.integers(1, 11))
        routing = ("normal", "zipf", "balanced")[int(rng.integers(0, 3))] if T % E == 0 else (
            "normal", "zipf")[int(rng.integers(0, 2))]
        out.append(W.small(f"random{i}", T=T, k=k, E=E, d=d, n=n, seed=100 + i, routing=routing))
    return out


RANDOM_CASES = _random_cases(8, 2024)
GEGLU_CASES = [CASES[1], CASES[2], CASES[4]]
# gathered rows (MOE_GATHER_ROWS): no permuted copies of x and dO
GATHER_CASES = [CASES[0], CASES[1], CASES[2], CASES[3]]


@pytest.mark.parametrize(
    "wl,act,gather",
    [(c, "swiglu", False) for c in CASES] + [(c, "geglu", False) for c in GEGLU_CASES]
    + [(c, "swiglu", True) for c in GATHER_CASES] + [(CASES[1], "geglu", True)]
    + [(c, "swiglu", False) for c in RANDOM_CASES],
    ids=[c.name for c in CASES] + [c.name + "-geglu" for c in GEGLU_CASES]
    + [c.name + "-gather" for c in GATHER_CASES] + [CASES[1].name + "-geglu-gather"]
    + [c.name for c in RANDOM_CASES])
def test_forward_backward_parity(M, wl, act, gather):
    print(f"mlp case {wl} act={act} gather={gather}", flush=True)
    inp = W.make_inputs(wl)
    buf = _run_gpu(M, wl, inp, act=M.MOE_ACT_GEGLU if act == "geglu" else M.MOE_ACT_SWIGLU,
                   gather=gather)
    f, b = _oracle(wl, inp, act)
    end = int(f["offsets"][-1])

    assert np.array_equal(buf.topk_idx.cpu().numpy(), f["topk_idx"])
    assert np.array_equal(buf.counts.cpu().numpy(), f["counts"])
    assert np.array_equal(buf.offsets.cpu().numpy(), f["offsets"])
    assert np.array_equal(buf.row_of.cpu().numpy(), f["row_of"])
    assert np.array_equal(buf.src_of.cpu().numpy(), f["src_of"])
    if not gather:
        assert np.array_equal(bf16_bits(buf.x_perm)[:end], O.bf16_bits(f["x_perm"][:end]))
        assert np.array_equal(bf16_bits(buf.dy_u)[:end], O.bf16_bits(b["dy_u"][:end]))

    _check("H", bf16_values(buf.h), f["H"], end)
    _check("A", bf16_values(buf.a), f["A"], end)
    _check("Y", bf16_values(buf.y), f["Y"], end)
    _check("out", bf16_values(buf.out), f["out"])
    _check("dS", buf.ds.cpu().numpy(), b["dS"])
    _check("dH", bf16_values(buf.dh), b["dH"], end)
    _check("A'", bf16_values(buf.a_w), b["a_w"], end)
    _check("dX_perm", bf16_values(buf.dx_perm), b["dx_perm"], end)
    _check("dX", bf16_values(buf.dx), b["dx"])
    _check("dW1", buf.dw1.cpu().numpy(), b["dW1"])
    _check("dW2", buf.dw2.cpu().numpy(), b["dW2"])

    # padding rows of every permuted tensor are exactly zero
    pad = f["src_of"][:end] < 0
    for name in ("h", "a", "y", "dh", "a_w", "dx_perm") + (() if gather else ("x_perm", "dy_u")):
        v = bf16_bits(getattr(buf, name))[:end][pad]
        assert np.all((v == 0) | (v == 0x8000)), name
    # empty experts: exactly zero weight gradients
    for e in np.nonzero(f["counts"] == 0)[0]:
        assert torch.all(buf.dw1[e] == 0) and torch.all(buf.dw2[e] == 0)


# non-gated squared ReLU: W1_e [d, n] (the first n columns of the generated W1)
SRELU_CASES = [CASES[0], CASES[1], CASES[2], CASES[4]]


@pytest.mark.parametrize("wl,gather", [(c, False) for c in SRELU_CASES] + [(CASES[1], True)],
                         ids=[c.name for c in SRELU_CASES] + [CASES[1].name + "-gather"])
def test_srelu_forward_backward_parity(M, wl, gather):
    print(f"mlp case {wl} act=srelu gather={gather}", flush=True)
    inp = dict(W.make_inputs(wl))
    inp["w1"] = np.ascontiguousarray(inp["w1"][:, :, :wl.n])
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, gated=False)
    _poison(buf)
    x, w1, w2 = bf16_tensor(inp["x"]), bf16_tensor(inp["w1"]), bf16_tensor(inp["w2"])
    dout = bf16_tensor(inp["dout"])
    M.forward(buf, x, f32_tensor(inp["logits"]), w1, w2, act=M.MOE_ACT_SRELU, gather=gather)
    M.backward(buf, dout, w1, w2, act=M.MOE_ACT_SRELU, x=x if gather else None)
    torch.cuda.synchronize()
    f, b = _oracle(wl, inp, "srelu")
    end = int(f["offsets"][-1])
    assert buf.h.shape[1] == wl.n
    _check("H", bf16_values(buf.h), f["H"], end)
    _check("A", bf16_values(buf.a), f["A"], end)
    _check("Y", bf16_values(buf.y), f["Y"], end)
    _check("out", bf16_values(buf.out), f["out"])
    _check("dS", buf.ds.cpu().numpy(), b["dS"])
    _check("dH", bf16_values(buf.dh), b["dH"], end)
    _check("A'", bf16_values(buf.a_w), b["a_w"], end)
    _check("dX_perm", bf16_values(buf.dx_perm), b["dx_perm"], end)
    _check("dX", bf16_values(buf.dx), b["dx"])
    _check("dW1", buf.dw1.cpu().numpy(), b["dW1"])
    _check("dW2", buf.dw2.cpu().numpy(), b["dW2"])
    pad = f["src_of"][:end] < 0
    for name in ("h", "a", "y", "dh", "a_w", "dx_perm"):
        v = bf16_bits(getattr(buf, name))[:end][pad]
        assert np.all((v == 0) | (v == 0x8000)), name
    for e in np.nonzero(f["counts"] == 0)[0]:
        assert torch.all(buf.dw1[e] == 0) and torch.all(buf.dw2[e] == 0)


def test_all_tokens_to_one_expert(M):
    wl = W.small("one", T=520, k=1, E=8, d=128, n=128, seed=31)
    inp = W.make_inputs(wl)
    inp["logits"][:] = 0.0                     # ties everywhere -> expert 0
    buf = _run_gpu(M, wl, inp)
    f, b = _oracle(wl, inp)
    assert list(buf.counts.cpu().numpy()) == [520, 0, 0, 0, 0, 0, 0, 0]
    _check("out", bf16_values(buf.out), f["out"])
    _check("dX", bf16_values(buf.dx), b["dx"])
    _check("dW1", buf.dw1.cpu().numpy(), b["dW1"])
    assert torch.all(buf.dw1[1:] == 0) and torch.all(buf.dw2[1:] == 0)


def test_max_experts(M):
    """E = 1024 (the library maximum): most experts get a few rows, many none."""
    wl = W.small("e1024", T=600, k=4, E=1024, d=128, n=64, seed=33, routing="normal")
    print(f"mlp case {wl}", flush=True)
    inp = W.make_inputs(wl)
    buf = _run_gpu(M, wl, inp)
    f, b = _oracle(wl, inp)
    assert np.array_equal(buf.offsets.cpu().numpy(), f["offsets"])
    assert (f["counts"] == 0).sum() > 0
    end = int(f["offsets"][-1])
    _check("Y", bf16_values(buf.y), f["Y"], end)
    _check("out", bf16_values(buf.out), f["out"])
    _check("dS", buf.ds.cpu().numpy(), b["dS"])
    _check("dX", bf16_values(buf.dx), b["dx"])
    _check("dW1", buf.dw1.cpu().numpy(), b["dW1"])
    _check("dW2", buf.dw2.cpu().numpy(), b["dW2"])
    for e in np.nonzero(f["counts"] == 0)[0][:64]:
        assert torch.all(buf.dw1[e] == 0) and torch.all(buf.dw2[e] == 0)


def test_determinism(M):
    wl = CASES[1]
    inp = W.make_inputs(wl)
    a = _run_gpu(M, wl, inp)
    b = _run_gpu(M, wl, inp)
    end = int(a.offsets[-1])
    for name in ("topk_w", "out", "ds", "dx", "dw1", "dw2"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    for name in ("h", "a", "y", "dh", "a_w", "dx_perm"):
        assert torch.equal(getattr(a, name)[:end], getattr(b, name)[:end]), name
