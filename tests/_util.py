"""Helpers shared by the tests: moving seeded inputs between numpy and torch."""
import numpy as np
import torch

from oracle import moe_oracle as O


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f32_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def check_fused_copies_vs_oracle(t_bf16, end, q_row, s_row, q_col, s_col, what="A"):
    """The MXFP8 copies a GEMM epilogue wrote of the bf16 tensor t_bf16 [M_cap, C] equal,
    bit for bit over the rows [0, end) of the expert regions, the oracle's quantization
    of that same bf16 tensor: row-wise codes [end, C] and scales [end, C/32] (when q_row
    is given), and the transposed column-wise codes [C, end] and scales [C, end/32] (when
    q_col is given)."""
    v = bf16_values(t_bf16[:end])
    rq, rs, cq, cs = O.quant_mxfp8(v, rowwise=q_row is not None, colwise=q_col is not None)
    if q_row is not None:
        assert np.array_equal(q_row[:end].cpu().numpy(), rq), f"{what} row codes vs oracle"
        assert np.array_equal(s_row[:end].cpu().numpy(), rs), f"{what} row scales vs oracle"
    if q_col is not None:
        assert np.array_equal(q_col[:, :end].cpu().numpy(), cq), f"{what} column codes vs oracle"
        assert np.array_equal(s_col[:, :end // 32].cpu().numpy(), cs), f"{what} column scales vs oracle"
