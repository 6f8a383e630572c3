"""The whole forward + backward captures in ONE hipGraph and replays correctly
when the routing changes between replays.

Nothing in the path reads shapes back to the host, so the graph recorded once
re-derives counts, offsets and tiles on the device at every replay. The inputs
(logits, x, dO) are overwritten in place before each replay; every replay is
checked against the oracle, with eager work and synchronisations in between.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from ragged_grouped_gemm_device_amd import workloads as W

from ._util import bf16_tensor, bf16_values, f32_tensor, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from ragged_grouped_gemm_device_amd import moe
    moe.load()
    return moe


def _oracle(wl, inp, logits):
    x, w1, w2 = O.from_bf16(inp["x"]), O.from_bf16(inp["w1"]), O.from_bf16(inp["w2"])
    f = O.forward(x, logits, w1, w2, wl.k)
    b = O.mlp_backward(f["x_perm"], w1, w2, f["H"], f["Y"], O.from_bf16(inp["dout"]), f["topk_w"],
                       f["counts"], f["offsets"], f["row_of"], f["src_of"], wl.k)
    return f, b


def test_forward_backward_single_graph_rerouted(M):
    wl = W.small("graph", T=900, k=2, E=8, d=256, n=256, seed=61)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(62)
    routings = {
        "normal": rng.standard_normal((wl.T, wl.E)).astype(np.float32),
        "zipf": (rng.standard_normal((wl.T, wl.E)) - 3.6 * np.log(rng.permutation(wl.E) + 1.0)).astype(np.float32),
        "constant": np.zeros((wl.T, wl.E), np.float32),  # ties: experts 0 and 1 take every token
        "reseeded": np.random.default_rng(63).standard_normal((wl.T, wl.E)).astype(np.float32),
    }
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n)
    x, w1, w2, dout = (bf16_tensor(inp[key]) for key in ("x", "w1", "w2", "dout"))
    logits = f32_tensor(routings["normal"])

    def step():
        M.forward(buf, x, logits, w1, w2)
        M.backward(buf, dout, w1, w2, logits=logits)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for name, lg in routings.items():
            print(f"graph replay {rep} routing {name}", flush=True)
            logits.copy_(torch.from_numpy(lg))
            buf.dx.fill_(float("nan"))          # eager work between replays
            buf.out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            f, b = _oracle(wl, inp, lg)
            assert np.array_equal(buf.counts.cpu().numpy(), f["counts"]), name
            assert np.array_equal(buf.offsets.cpu().numpy(), f["offsets"]), name
            assert np.array_equal(buf.row_of.cpu().numpy(), f["row_of"]), name
            dl_ref = O.route_backward(lg, f["topk_idx"], b["dS"])
            for key, got, ref in (("dlogits", buf.dlogits.cpu().numpy(), dl_ref),
                                  ("out", bf16_values(buf.out), f["out"]),
                                  ("dx", bf16_values(buf.dx), b["dx"]),
                                  ("dS", buf.ds.cpu().numpy(), b["dS"]),
                                  ("dW1", buf.dw1.cpu().numpy(), b["dW1"]),
                                  ("dW2", buf.dw2.cpu().numpy(), b["dW2"])):
                err = rel_err(got, ref)
                assert err <= 2e-2, (name, key, err)
            if name == "constant":
                assert list(buf.counts.cpu().numpy()) == [wl.T, wl.T] + [0] * (wl.E - 2)
                assert torch.all(buf.dw1[2:] == 0) and torch.all(buf.dw2[2:] == 0)


def test_graph_matches_eager_bitwise(M):
    """Replaying the graph gives exactly the eager results (same kernels, same order)."""
    wl = W.small("graph2", T=512, k=4, E=16, d=128, n=128, seed=64, routing="zipf")
    inp = W.make_inputs(wl)
    x, w1, w2, dout = (bf16_tensor(inp[key]) for key in ("x", "w1", "w2", "dout"))
    logits = f32_tensor(inp["logits"])
    eager = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n)
    M.forward(eager, x, logits, w1, w2)
    M.backward(eager, dout, w1, w2)
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.forward(buf, x, logits, w1, w2)
        M.backward(buf, dout, w1, w2)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.forward(buf, x, logits, w1, w2)
        M.backward(buf, dout, w1, w2)
    for _ in range(3):
        buf.out.zero_()
        buf.dw1.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name in ("out", "dx", "ds", "dw1", "dw2", "topk_w"):
            assert torch.equal(getattr(buf, name), getattr(eager, name)), name


def test_mxfp8_step_single_graph_rerouted(M):
    """The MXFP8 step (fused permute + quantization, every GEMM on MXFP8, router
    backward) captures in one graph; every replay under a new routing equals
    the eager MXFP8 step bit for bit and stays within the MXFP8 tolerance of the
    oracle's MXFP8 forward and backward."""
    wl = W.small("graph-mx", T=700, k=2, E=8, d=256, n=256, seed=65)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(66)
    routings = {
        "normal": rng.standard_normal((wl.T, wl.E)).astype(np.float32),
        "zipf": (rng.standard_normal((wl.T, wl.E)) - 3.6 * np.log(rng.permutation(wl.E) + 1.0)).astype(np.float32),
        "constant": np.zeros((wl.T, wl.E), np.float32),
    }
    x, w1, w2, dout = (bf16_tensor(inp[key]) for key in ("x", "w1", "w2", "dout"))
    logits = f32_tensor(routings["normal"])
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=True)
    eager = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=True)
    buf.quantize_weights(w1, w2)
    eager.quantize_weights(w1, w2)

    def step(b):
        M.forward(b, x, logits, w1, w2, mx=True)
        M.backward(b, dout, w1, w2, logits=logits, mx=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(buf)
    torch.cuda.synchronize()
    xo, w1o, w2o = O.from_bf16(inp["x"]), O.from_bf16(inp["w1"]), O.from_bf16(inp["w2"])
    for rep in range(2):
        for name, lg in routings.items():
            print(f"mx graph replay {rep} routing {name}", flush=True)
            logits.copy_(torch.from_numpy(lg))
            buf.dx.fill_(float("nan"))
            buf.out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            step(eager)
            torch.cuda.synchronize()
            for key in ("out", "dx", "ds", "dw1", "dw2", "dlogits"):
                assert torch.equal(getattr(buf, key), getattr(eager, key)), (name, key)
            f = O.forward(xo, lg, w1o, w2o, wl.k)
            m = O.mlp_forward_mx(f["x_perm"], w1o, w2o, f["counts"], f["offsets"])
            out = O.combine(m["Y"], f["row_of"], wl.k, f["topk_w"])
            b = O.mlp_backward_mx(f["x_perm"], w1o, w2o, m["H"], m["Y"], O.from_bf16(inp["dout"]),
                                  f["topk_w"], f["counts"], f["offsets"], f["row_of"], f["src_of"],
                                  wl.k, dgrad2_mx=True)
            for key, got, ref in (("out", bf16_values(buf.out), out), ("dx", bf16_values(buf.dx), b["dx"]),
                                  ("dS", buf.ds.cpu().numpy(), b["dS"]), ("dW1", buf.dw1.cpu().numpy(), b["dW1"]),
                                  ("dW2", buf.dw2.cpu().numpy(), b["dW2"])):
                err = rel_err(got, ref)
                assert err <= 6e-2, (name, key, err)
