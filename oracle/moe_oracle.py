"""CPU oracle for the dropless MoE expert MLP -- TEST INFRASTRUCTURE ONLY.

This module is a plain, slow, fp64 restatement of what the hot path computes.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the GPU product path never calls it and shares no code with it
(it has its own bf16 and E4M3 codecs and its own routing/layout code).

Sources (web pages; cited by title and section):
  [P1] "NVIDIA CuTe DSL 융합 커널은 MoE 학습의 CPU·메모리 병목을 지운다"
       (summary of NVIDIA's "Boosting MoE Training Throughput with Advanced
       Fusion Kernels"): GLU epilogue over gate/up-interleaved weights,
       device-side per-expert counts, MXFP8 output plus transposed output.
  [P2] "SonicMoE로 보는 GPU 커널 최적화": the six sub-kernels of an MoE layer,
       the router-gradient rewrite dS = <dO, Y> = <dO W2^T, A>.
  [P3] "Dropless MoE 학습과 NVIDIA Transformer Engine 소개": ragged tensors,
       dropless contiguous buffers, 128-token expert alignment, prefused
       FC1 weights of shape (experts, embed_dim, 2*mlp_dim), expert-major
       buffer with one slot per (token, expert) pair, empty expert groups.

Readings where the pages are silent (each listed in the design notes):
  * routing: softmax over all E experts in fp64, top-k by raw logit
    (descending, ties to the lower expert index), weights = softmax
    probabilities of the chosen experts, optional renormalisation;
  * layout: rows of expert e are its pairs in ascending pair index t*k+j,
    each expert segment padded to a multiple of 128 rows, empty experts
    take zero rows;
  * interleave granularity g = 32 columns, gate block first;
  * Swish with beta = 1 (SiLU); GeGLU's GELU in its exact (erf) form,
    gelu(x) = x * Phi(x) with Phi the standard normal CDF;
  * storage points that the path keeps in bf16 (X_perm, H, A, Y, O, dY_u,
    dH, A', dX_perm, dX) are rounded to the nearest bf16 (ties to even);
    every other value is fp64;
  * A' = w * A (routing-weighted activation) and dW in fp64/fp32;
  * MXFP8 blocks of 32 elements (OCP MX v1.0 element and scale formats) with
    the shared exponent rounded up so that no element saturates: the smallest
    e with amax <= 448 * 2^e; E4M3 codes rounded to nearest-even, zero block
    -> scale 0. The pages name MXFP8 but give no scale rule. The floor rule
    (floor(log2 amax) - 8) would clip a block maximum whose significand is
    above 1.75 to 448 * 2^e, an error of up to 12.5% of that element, beyond
    the 6e-2 tolerance the MXFP8 path is held to; the rounded-up exponent
    never clips, at the cost of one binade of resolution for such blocks.

Parity pins live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

ALIGN = 128
GLU_INTERLEAVE = 32
MX_BLOCK = 32

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# --------------------------------------------------------------------------
# bf16 storage rounding (fp64 -> nearest bf16, ties to even), own codec
# --------------------------------------------------------------------------
def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each fp64 element (ties to even), as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range; below 2**-126 the
    spacing is fixed at 2**-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    _, q = np.frexp(x)                      # x = m * 2**q, 0.5 <= |m| < 1
    ulp_exp = np.maximum(q - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -ulp_exp)), ulp_exp)
    return np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)


def bf16_bits(x) -> np.ndarray:
    """Bit pattern (uint16) of round_bf16(x)."""
    r = round_bf16(x).astype(np.float32)     # exact: bf16 values are fp32 values
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_bf16(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _maybe_round(x, rounding: bool):
    return round_bf16(x) if rounding else np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# O1: routing  [P3, ragged-tensor section: a learned router picks the top-K
# experts per token; BASELINE workload: softmax top-k]
# --------------------------------------------------------------------------
def route(logits, k: int, renorm: bool = False):
    """Softmax top-k routing.

    logits: float32 [T, E]. Returns (topk_idx int32 [T, k], topk_w fp64 [T, k]).
    Experts are ordered by raw logit, descending, ties broken towards the lower
    expert index; slot j holds the j-th best expert. Weights are the softmax
    probabilities (over all E experts) of the chosen experts, renormalised over
    the k chosen ones if ``renorm``.
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = lg.shape
    if not (0 < k <= E):
        raise ValueError("need 0 < k <= E")
    order = np.argsort(-lg, axis=1, kind="stable")   # stable: equal logits keep ascending index
    idx = order[:, :k].astype(np.int32)
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


def route_backward(logits, topk_idx, dS, renorm: bool = False):
    """Gradient of the loss w.r.t. the router logits, given dS = dL/dw.

    The routing weights depend on the logits through the softmax; the chosen
    experts are a fixed (piecewise constant) function of them. Without
    renormalisation w_j = p_{e_j}, p = softmax over all E, so
        dl_e = p_e * (g_e - sum_j p_{e_j} dS_j),  g_e = dS_j if e = e_j else 0.
    With renormalisation w is the softmax over the k chosen logits, so
        dl_{e_j} = w_j * (dS_j - sum_i w_i dS_i), and 0 for experts not chosen.
    [P2 backward-rewrite section: dS is the router-score gradient the MLP
    backward produces; it flows on through the router's softmax.]
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    dS = np.asarray(dS, dtype=np.float64)
    T, E = lg.shape
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    d = np.zeros((T, E))
    if not renorm:
        g = np.zeros((T, E))
        np.put_along_axis(g, idx, dS, axis=1)
        c = (np.take_along_axis(p, idx, axis=1) * dS).sum(axis=1, keepdims=True)
        d = p * (g - c)
    else:
        w = np.take_along_axis(p, idx, axis=1)
        w = w / w.sum(axis=1, keepdims=True)
        c = (w * dS).sum(axis=1, keepdims=True)
        np.put_along_axis(d, idx, w * (dS - c), axis=1)
    return d


# --------------------------------------------------------------------------
# O2: counts, aligned offsets, row maps  [P1 core-idea section: per-expert
# counts kept on the device; P3 dropless section: one contiguous buffer;
# P3 grouped-GEMM section: 128-token alignment; P3 dropless-boundary
# section: one slot per (token, local expert) pair, expert regions padded]
# --------------------------------------------------------------------------
def capacity_rows(T: int, k: int, E: int, align: int = ALIGN) -> int:
    """Worst-case rows of the expert-major buffer: align(T*k) + align*E."""
    return -(-T * k // align) * align + align * E


def layout(topk_idx, E: int, M_cap: int | None = None, align: int = ALIGN):
    """Expert-major ragged layout of the (token, expert) pairs.

    Pair p = t*k + j goes to expert topk_idx[t, j]. Expert e's pairs occupy
    rows [offsets[e], offsets[e] + counts[e]) in ascending p; rows up to
    offsets[e+1] = offsets[e] + align*ceil(counts[e]/align) are padding.
    Returns counts [E], offsets [E+1], row_of [T*k], src_of [M_cap] (-1 = pad
    or unused row).
    """
    pairs = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    P = pairs.size
    counts = np.bincount(pairs, minlength=E).astype(np.int64)
    if counts.size != E:
        raise ValueError("expert index out of range")
    padded = -(-counts // align) * align
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    order = np.argsort(pairs, kind="stable")     # grouped by expert, ascending pair index
    first = np.zeros(E, dtype=np.int64)
    first[1:] = np.cumsum(counts)[:-1]           # start of each expert in `order`
    rank = np.empty(P, dtype=np.int64)
    rank[order] = np.arange(P) - first[pairs[order]]
    row_of = offsets[pairs] + rank
    if M_cap is None:
        M_cap = int(offsets[-1])
    src_of = np.full(M_cap, -1, dtype=np.int64)
    src_of[row_of] = np.arange(P)
    return (counts.astype(np.int32), offsets.astype(np.int32), row_of.astype(np.int32),
            src_of.astype(np.int32))


# --------------------------------------------------------------------------
# O3: permute (gather) and O7: combine  [P2 SonicMoE section: gather, scatter
# and expert aggregation sub-kernels; P3 EP section: combine restores token
# order and accumulates per token]
# --------------------------------------------------------------------------
def permute(x, row_of, k: int, M_cap: int):
    """X_perm[row_of[t*k+j]] = x[t]; every other row is zero. x: fp64 [T, d]."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros((M_cap, x.shape[1]), dtype=np.float64)
    P = np.asarray(row_of).size
    out[np.asarray(row_of, dtype=np.int64)] = x[np.arange(P) // k]
    return out


def combine(y, row_of, k: int, w=None, rounding: bool = True):
    """O[t] = sum over j ascending of w[t,j] * y[row_of[t*k+j]] (w = 1 if None)."""
    y = np.asarray(y, dtype=np.float64)
    rows = np.asarray(row_of, dtype=np.int64).reshape(-1, k)
    T = rows.shape[0]
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        wj = 1.0 if w is None else np.asarray(w, dtype=np.float64)[:, j:j + 1]
        out += wj * y[rows[:, j]]
    return _maybe_round(out, rounding)


# --------------------------------------------------------------------------
# O4: gate/up interleave  [P1 core-idea section: weights repacked so that
# gate and input columns interleave and one tile sees both halves; P3
# grouped-GEMM section: prefused FC1 weight (experts, embed_dim, 2*mlp_dim)]
# --------------------------------------------------------------------------
def interleave(gate, up, g: int = GLU_INTERLEAVE):
    """Columns [2bg, 2bg+g) = gate[:, bg:bg+g], [2bg+g, 2bg+2g) = up[:, bg:bg+g]."""
    gate = np.asarray(gate)
    up = np.asarray(up)
    *lead, n = gate.shape
    if n % g:
        raise ValueError("n must be a multiple of the interleave granularity")
    nb = n // g
    out = np.stack([gate.reshape(*lead, nb, g), up.reshape(*lead, nb, g)], axis=-2)
    return out.reshape(*lead, 2 * n)


def deinterleave(h, g: int = GLU_INTERLEAVE):
    """Inverse of interleave: returns (gate, up), each [..., n]."""
    h = np.asarray(h)
    *lead, n2 = h.shape
    n = n2 // 2
    nb = n // g
    hb = h.reshape(*lead, nb, 2, g)
    return hb[..., 0, :].reshape(*lead, n), hb[..., 1, :].reshape(*lead, n)


def silu(v):
    return v / (1.0 + np.exp(-v))


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def gelu(v):
    """GELU, exact form: v * Phi(v), Phi(v) = (1 + erf(v / sqrt 2)) / 2."""
    v = np.asarray(v, dtype=np.float64)
    return v * 0.5 * (1.0 + _erf(v / np.sqrt(2.0)))


def gelu_grad(v):
    """d gelu / dv = Phi(v) + v * phi(v), phi the standard normal density."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * (1.0 + _erf(v / np.sqrt(2.0))) + v * np.exp(-0.5 * v * v) / np.sqrt(2.0 * np.pi)


# the gate activation of each GLU variant and its derivative  [P1 problem
# section: SwiGLU and GeGLU epilogues and their backward]
GLU_ACTS = {
    "swiglu": (silu, lambda v: sigmoid(v) * (1.0 + v * (1.0 - sigmoid(v)))),
    "geglu": (gelu, gelu_grad),
}


def srelu(v):
    """Squared ReLU, relu(v)^2 [P1 problem and published-evidence sections: the
    sReLU family of fused epilogues; the plain reading is the non-gated squared
    ReLU, so FC1 then has n output columns instead of 2n]."""
    r = np.maximum(v, 0.0)
    return r * r


def srelu_grad(v):
    return 2.0 * np.maximum(v, 0.0)


# non-gated activations: A = f(H) with H of width n
PLAIN_ACTS = {"srelu": (srelu, srelu_grad)}


def is_gated(act: str) -> bool:
    return act in GLU_ACTS


# --------------------------------------------------------------------------
# O5/O6: per-expert FC1 + SwiGLU and FC2  [P1 problem and core-idea sections:
# the GLU activation applied to the FC1 output inside the GEMM epilogue;
# P3 grouped-GEMM section: one GEMM per expert on its real rows]
# --------------------------------------------------------------------------
def expert_segments(counts, offsets):
    """[(e, row_start, row_end)] of the real rows of every expert."""
    return [(e, int(offsets[e]), int(offsets[e]) + int(counts[e])) for e in range(len(counts))]


def mlp_forward(x_perm, w1, w2, counts, offsets, g: int = GLU_INTERLEAVE, rounding: bool = True,
                act: str = "swiglu"):
    """Grouped FC1 -> GLU (SwiGLU or GeGLU) or sReLU -> FC2 over the ragged expert-major rows.

    x_perm fp64 [M_cap, d], w1 fp64 [E, d, 2n] (interleaved; [E, d, n] for the
    non-gated sReLU, A = relu(H)^2), w2 fp64 [E, n, d].
    Returns H [M_cap, 2n] (bf16-rounded when stored), A [M_cap, n], Y [M_cap, d];
    rows outside the real segments are zero.
    A is computed from the unrounded FC1 output: A = act(gate) * up, act = silu
    (SwiGLU) or gelu (GeGLU).
    """
    gated = is_gated(act)
    act_fn = (GLU_ACTS if gated else PLAIN_ACTS)[act][0]
    x_perm = np.asarray(x_perm, dtype=np.float64)
    M_cap, d = x_perm.shape
    E, _, n2 = w1.shape
    n = n2 // 2 if gated else n2
    H = np.zeros((M_cap, n2))
    A = np.zeros((M_cap, n))
    Y = np.zeros((M_cap, d))
    for e, r0, r1 in expert_segments(counts, offsets):
        if r1 == r0:
            continue
        h = x_perm[r0:r1] @ w1[e]
        if gated:
            hg, hu = deinterleave(h, g)
            a = _maybe_round(act_fn(hg) * hu, rounding)
        else:
            a = _maybe_round(act_fn(h), rounding)
        H[r0:r1] = _maybe_round(h, rounding)
        A[r0:r1] = a
        Y[r0:r1] = _maybe_round(a @ w2[e], rounding)
    return H, A, Y


def forward(x, logits, w1, w2, k: int, renorm: bool = False, rounding: bool = True,
            g: int = GLU_INTERLEAVE, act: str = "swiglu"):
    """Whole forward: route -> layout -> permute -> FC1+SwiGLU -> FC2 -> combine.

    x fp64 [T, d] (bf16 values), logits float32 [T, E]. Returns a dict with
    every intermediate the backward needs.
    """
    T, d = x.shape
    E = logits.shape[1]
    idx, w = route(logits, k, renorm)
    M_cap = capacity_rows(T, k, E)
    counts, offsets, row_of, src_of = layout(idx, E, M_cap)
    x_perm = permute(x, row_of, k, M_cap)
    H, A, Y = mlp_forward(x_perm, w1, w2, counts, offsets, g, rounding, act)
    out = combine(Y, row_of, k, w, rounding)
    return dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets, row_of=row_of,
                src_of=src_of, M_cap=M_cap, x_perm=x_perm, H=H, A=A, Y=Y, out=out)


# --------------------------------------------------------------------------
# O10: backward  [P2 backward-rewrite section: dS = <dO_t, Y_(e,t)>; GEMM
# overlapping section: the dH kernel stores dH, dS and A'; P1 published-
# evidence section: dSwiGLU fused into the dgrad GEMM]
# --------------------------------------------------------------------------
def mlp_backward(x_perm, w1, w2, H, Y, dout, topk_w, counts, offsets, row_of, src_of, k: int,
                 g: int = GLU_INTERLEAVE, rounding: bool = True, act: str = "swiglu", dap=None):
    """Manual backward of the MLP for fixed routing weights.

    The routing weights w are treated as inputs: dS[t,j] = dL/dw[t,j] is the
    router-weight gradient, computed on the plain side <dO_t, Y_row>. Gradients
    of x, W1 and W2 follow the chain rule with the gate/up activation taken
    from the stored H. Returns dict(dy_u, dS, dH, a_w, dx_perm, dx, dW1, dW2).

    dap [M_cap, n], when given, replaces the FC2 dgrad dY_u W2_e^T (the
    unweighted dA' of each row, e.g. from an MXFP8 GEMM); dS is then taken on
    the rewritten side, <dA'_row, a_row> [P2 backward-rewrite section], since
    that product is what such a dA' feeds.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    M_cap, d = x_perm.shape
    E, _, n2 = w1.shape
    gated = is_gated(act)
    n = n2 // 2 if gated else n2
    T = dout.shape[0]
    dout = np.asarray(dout, dtype=np.float64)
    rows = np.asarray(row_of, dtype=np.int64)
    src = np.asarray(src_of, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64).reshape(-1)

    dy_u = permute(dout, rows, k, M_cap)                 # unweighted gather of dO
    w_row = np.zeros(M_cap)
    valid = src >= 0
    w_row[valid] = w[src[valid]]

    dS = np.einsum("pd,pd->p", dout[np.arange(T * k) // k], Y[rows]).reshape(T, k)
    ds_row = np.zeros(M_cap)

    dH = np.zeros((M_cap, n2))
    a_w = np.zeros((M_cap, n))
    dx_perm = np.zeros((M_cap, d))
    dW1 = np.zeros((E, d, n2))
    dW2 = np.zeros((E, n, d))
    for e, r0, r1 in expert_segments(counts, offsets):
        if r1 == r0:
            continue
        da_u = dy_u[r0:r1] @ w2[e].T if dap is None else dap[r0:r1]   # dA' (unweighted)
        da = w_row[r0:r1, None] * da_u
        if gated:
            hg, hu = deinterleave(H[r0:r1], g)
            f, f_grad = GLU_ACTS[act]
            fg = f(hg)
            a = fg * hu
            dg = da * hu * f_grad(hg)
            du = da * fg
            dh = _maybe_round(interleave(dg, du, g), rounding)
        else:
            f, f_grad = PLAIN_ACTS[act]
            a = f(H[r0:r1])
            dh = _maybe_round(da * f_grad(H[r0:r1]), rounding)
        ds_row[r0:r1] = np.einsum("rc,rc->r", da_u, a)
        aw = _maybe_round(w_row[r0:r1, None] * a, rounding)
        dH[r0:r1] = dh
        a_w[r0:r1] = aw
        dW2[e] = aw.T @ dy_u[r0:r1]
        dx_perm[r0:r1] = _maybe_round(dh @ w1[e].T, rounding)
        dW1[e] = x_perm[r0:r1].T @ dh
    dx = combine(dx_perm, rows, k, None, rounding)
    if dap is not None:
        dS = ds_row[rows].reshape(T, k)
    return dict(dy_u=dy_u, dS=dS, dH=dH, a_w=a_w, dx_perm=dx_perm, dx=dx, dW1=dW1, dW2=dW2)


# --------------------------------------------------------------------------
# O8: MXFP8 quantization  [P1 problem and core-idea sections: BF16 activation
# to MXFP8 with a transposed copy; P3 three-components section: group-aware
# MXFP8 quantization; block format per OCP MX v1.0: 32-element blocks, E8M0
# shared scale, E4M3 elements]
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_encode(y) -> np.ndarray:
    """E4M3 (OCP, 1-4-3, bias 7, no infinities) code of each fp64 value.

    Round to nearest, ties to even; magnitudes above 448 saturate to 448;
    the sign bit is kept for zero results. Inputs must be finite.
    """
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.abs(y)
    _, q = np.frexp(a)
    ex = np.maximum(q - 1, -6)                 # exponent of the binade; subnormals share -6
    ulp_exp = ex - 3
    r = np.rint(np.ldexp(a, -ulp_exp))         # multiples of the local spacing
    val = np.minimum(np.ldexp(r, ulp_exp), E4M3_MAX)
    _, q2 = np.frexp(val)
    e2 = q2 - 1
    normal = (val >= 2.0 ** -6)
    exp_field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, np.ldexp(val, -e2) * 8.0 - 8.0, np.ldexp(val, 9))
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(val == 0.0, 0, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    v = np.where(ef == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, ef - 7))
    v = np.where((ef == 15) & ((c & 7) == 7), np.nan, v)
    return s * v


def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent of a block: the smallest integer e with amax <= 448 * 2^e
    (so no element of the block saturates), clamped to [-127, 127]; a zero
    block takes -127 (scale code 0).

    Equivalently floor(log2 amax) - 8, plus one when amax's significand
    exceeds 1.75 (448 = 1.75 * 2^8)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, q = np.frexp(amax)                  # amax = m * 2^q, 0.5 <= m < 1
    e = (q - 1 - 8) + (2.0 * m > 1.75)
    e = np.clip(e, -127, 127)
    return np.where(amax == 0.0, -127, e).astype(np.int64)


def _quant_rows(v):
    """Quantize each row of v [R, C] in blocks of 32 consecutive columns."""
    R, C = v.shape
    blocks = v.reshape(R, C // MX_BLOCK, MX_BLOCK)
    e = mx_block_exponent(np.abs(blocks).max(axis=2))
    q = e4m3_encode(np.ldexp(blocks, -e[..., None]))
    return q.reshape(R, C), (e + 127).astype(np.uint8)


def quant_mxfp8(src, rowwise: bool = True, colwise: bool = True):
    """MXFP8 quantization of a bf16-valued matrix src [R, C] (fp64 array).

    rowwise: blocks of 32 consecutive columns of a row -> q_row u8 [R, C],
             s_row u8 [R, C/32].
    colwise ("transposed"): blocks of 32 consecutive rows of a column, stored
             transposed -> q_col u8 [C, R], s_col u8 [C, R/32].
    Returns (q_row, s_row, q_col, s_col) with None for the mode not requested.
    """
    v = np.asarray(src, dtype=np.float64)
    q_row = s_row = q_col = s_col = None
    if rowwise:
        if v.shape[1] % MX_BLOCK:
            raise ValueError("C must be a multiple of 32")
        q_row, s_row = _quant_rows(v)
    if colwise:
        if v.shape[0] % MX_BLOCK:
            raise ValueError("R must be a multiple of 32")
        q_col, s_col = _quant_rows(v.T)
    return q_row, s_row, q_col, s_col


def mx_dequant(q, s):
    """Dequantize codes q [R, C] with block scales s [R, C/32] (fp64)."""
    R, C = q.shape
    vals = e4m3_decode(q).reshape(R, C // MX_BLOCK, MX_BLOCK)
    sc = np.ldexp(1.0, np.asarray(s, dtype=np.int64) - 127)
    return (vals * sc[..., None]).reshape(R, C)


# --------------------------------------------------------------------------
# O9: MXFP8 grouped FC2  [P3 three-components section: MXFP8 grouped GEMM]
# --------------------------------------------------------------------------
def mx_gemm_rows(a_q, a_s, bt_q, bt_s):
    """C[r, c] = sum_b 2^(sa[r,b]-127) 2^(sb[c,b]-127) sum_{i in b} a[r,i] b[c,i].

    a_q [R, K] codes with a_s [R, K/32]; bt_q [N, K] codes (the B operand
    stored K-contiguous, i.e. transposed) with bt_s [N, K/32]. fp64 result.
    """
    R, K = a_q.shape
    N = bt_q.shape[0]
    av = e4m3_decode(a_q).reshape(R, K // MX_BLOCK, MX_BLOCK)
    bv = e4m3_decode(bt_q).reshape(N, K // MX_BLOCK, MX_BLOCK)
    partial = np.einsum("rbi,cbi->rcb", av, bv)          # per-block dot products
    sa = np.ldexp(1.0, np.asarray(a_s, dtype=np.int64) - 127)
    sb = np.ldexp(1.0, np.asarray(bt_s, dtype=np.int64) - 127)
    return np.einsum("rcb,rb,cb->rc", partial, sa, sb)


def mx_fc1(x_q, x_s, w1t_q, w1t_s, counts, offsets, g: int = GLU_INTERLEAVE, rounding: bool = True,
           act: str = "swiglu"):
    """Grouped MXFP8 FC1 with the GLU epilogue: H[R_e] = MX(X_perm[R_e]) x MX(W1_e).

    x_q [M_cap, d], x_s [M_cap, d/32] (X_perm row-wise, blocks along d);
    w1t_q [E, 2n, d], w1t_s [E, 2n, d/32] (W1_e quantized in blocks of 32
    along d and stored transposed). As in mlp_forward, A = act(gate) * up is
    taken from the unrounded product and H is stored rounded. Returns H, A.
    """
    act_fn = GLU_ACTS[act][0]
    M_cap = x_q.shape[0]
    E, n2, _ = w1t_q.shape
    H = np.zeros((M_cap, n2))
    A = np.zeros((M_cap, n2 // 2))
    for e, r0, r1 in expert_segments(counts, offsets):
        if r1 > r0:
            h = mx_gemm_rows(x_q[r0:r1], x_s[r0:r1], w1t_q[e], w1t_s[e])
            hg, hu = deinterleave(h, g)
            A[r0:r1] = _maybe_round(act_fn(hg) * hu, rounding)
            H[r0:r1] = _maybe_round(h, rounding)
    return H, A


def mlp_forward_mx(x_perm, w1, w2, counts, offsets, g: int = GLU_INTERLEAVE, act: str = "swiglu",
                   fc1_mx: bool = True):
    """MXFP8 forward of the expert MLP [P1 core-idea section: MXFP8 output of the
    FC1 epilogue; P3 three-components section: MXFP8 grouped GEMM].

    With fc1_mx, FC1 runs on X_perm quantized row-wise (blocks along d) and W1_e
    quantized along d (mx_fc1); otherwise FC1 is the bf16 product of
    mlp_forward. The bf16 A is quantized row-wise and FC2 runs on it and on W2_e
    quantized along n (mx_fc2). Returns dict(H, A, Y) and the quantized copies.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    E = w1.shape[0]
    end = int(offsets[-1])
    out = {}
    if fc1_mx:
        x_q, x_s, _, _ = quant_mxfp8(x_perm[:end], rowwise=True, colwise=False)
        w1t = [quant_mxfp8(w1[e], rowwise=False, colwise=True)[2:] for e in range(E)]
        w1t_q, w1t_s = np.stack([q for q, _ in w1t]), np.stack([sc for _, sc in w1t])
        Hm, Am = mx_fc1(x_q, x_s, w1t_q, w1t_s, counts, offsets, g, True, act)   # rows [0, end)
        H = np.zeros((x_perm.shape[0], Hm.shape[1]))
        A = np.zeros((x_perm.shape[0], Am.shape[1]))
        H[:end], A[:end] = Hm, Am
        out.update(x_q=x_q, x_s=x_s, w1t_q=w1t_q, w1t_s=w1t_s)
    else:
        H, A, _ = mlp_forward(x_perm, w1, w2, counts, offsets, g, True, act)
    a_q, a_s, _, _ = quant_mxfp8(A[:end], rowwise=True, colwise=False)
    w2t = [quant_mxfp8(w2[e], rowwise=False, colwise=True)[2:] for e in range(E)]
    w2t_q, w2t_s = np.stack([q for q, _ in w2t]), np.stack([sc for _, sc in w2t])
    Y = np.zeros((x_perm.shape[0], w2.shape[2]))
    Y[:end] = mx_fc2(a_q, a_s, w2t_q, w2t_s, counts, offsets)
    out.update(H=H, A=A, Y=Y, a_q=a_q, a_s=a_s, w2t_q=w2t_q, w2t_s=w2t_s)
    return out


def mx_fc2(a_q, a_s, w2t_q, w2t_s, counts, offsets, rounding: bool = True):
    """Grouped MXFP8 FC2: Y[R_e] = MX(A[R_e]) x MX(W2_e) for each expert.

    a_q [M_cap, n], a_s [M_cap, n/32]; w2t_q [E, d, n], w2t_s [E, d, n/32]
    (W2_e quantized in blocks of 32 along n and stored transposed).
    """
    M_cap = a_q.shape[0]
    E, d, _ = w2t_q.shape
    Y = np.zeros((M_cap, d))
    for e, r0, r1 in expert_segments(counts, offsets):
        if r1 > r0:
            Y[r0:r1] = _maybe_round(mx_gemm_rows(a_q[r0:r1], a_s[r0:r1], w2t_q[e], w2t_s[e]),
                                    rounding)
    return Y


# --------------------------------------------------------------------------
# O11: tolerance metric
# --------------------------------------------------------------------------
def mlp_backward_mx(x_perm, w1, w2, H, Y, dout, topk_w, counts, offsets, row_of, src_of, k: int,
                    g: int = GLU_INTERLEAVE, act: str = "swiglu", dgrad2_mx: bool = False):
    """MXFP8 backward of the expert MLP  [P1 core-idea and published-evidence
    sections: GroupGemm + dActivation + Quantize/Transpose; P3 three-components
    section: MXFP8 grouped GEMM].

    FC2 dgrad with the dGLU epilogue is bf16 (dH, A', dS exactly as in
    mlp_backward), or with dgrad2_mx runs on dY_u quantized row-wise (blocks
    along d) and W2_e quantized along d, the dGLU epilogue then taking that
    product as dA' (and dS on the rewritten side). Its outputs are quantized
    to MXFP8: dH row-wise (32-column
    blocks: the K of the FC1 dgrad) and column-wise (32-row blocks: the K of
    the FC1 wgrad), A' column-wise (the K of the FC2 wgrad). dY_u and X_perm
    are quantized column-wise and W1_e row-wise along 2n. Then
      dX_perm[R_e] = bf16(MX-GEMM(dH_q, W1q_e)),
      dW2_e = deq(A'_col)[:, R_e] @ deq(dY_col)[:, R_e]^T,
      dW1_e = deq(X_col)[:, R_e] @ deq(dH_col)[:, R_e]^T,
    over each expert's 128-aligned row region R_e (padding rows are zero), and
    dx = the unweighted combine of dX_perm.
    """
    E = w1.shape[0]
    end = int(offsets[-1])
    extra = {}
    dap = None
    if dgrad2_mx:
        M_cap = np.asarray(x_perm).shape[0]
        dy_u = permute(np.asarray(dout, dtype=np.float64), np.asarray(row_of, dtype=np.int64), k, M_cap)
        dy_q, dy_s, _, _ = quant_mxfp8(dy_u[:end], rowwise=True, colwise=False)
        w2r = [quant_mxfp8(w2[e], rowwise=True, colwise=False)[:2] for e in range(E)]
        dap = np.zeros((M_cap, w2.shape[1]))
        for e, r0, r1 in expert_segments(counts, offsets):
            if r1 > r0:
                dap[r0:r1] = mx_gemm_rows(dy_q[r0:r1], dy_s[r0:r1], w2r[e][0], w2r[e][1])
        extra = dict(dy_q=dy_q, dy_s=dy_s, w2q=np.stack([q for q, _ in w2r]),
                     w2s=np.stack([sc for _, sc in w2r]))
    b = mlp_backward(x_perm, w1, w2, H, Y, dout, topk_w, counts, offsets, row_of, src_of, k, g,
                     True, act, dap)
    dh_q, dh_s, dht_q, dht_s = quant_mxfp8(b["dH"][:end], rowwise=True, colwise=True)
    _, _, awt_q, awt_s = quant_mxfp8(b["a_w"][:end], rowwise=False, colwise=True)
    _, _, dyt_q, dyt_s = quant_mxfp8(b["dy_u"][:end], rowwise=False, colwise=True)
    _, _, xt_q, xt_s = quant_mxfp8(np.asarray(x_perm)[:end], rowwise=False, colwise=True)
    aw_d, dy_d = mx_dequant(awt_q, awt_s), mx_dequant(dyt_q, dyt_s)
    x_d, dh_d = mx_dequant(xt_q, xt_s), mx_dequant(dht_q, dht_s)
    M_cap = np.asarray(x_perm).shape[0]
    dx_perm = np.zeros((M_cap, w1.shape[1]))
    dW1 = np.zeros(w1.shape)
    dW2 = np.zeros(w2.shape)
    w1q = []
    for e in range(E):
        q, sc, _, _ = quant_mxfp8(w1[e], rowwise=True, colwise=False)
        w1q.append((q, sc))
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        dx_perm[r0:r1] = round_bf16(mx_gemm_rows(dh_q[r0:r1], dh_s[r0:r1], q, sc))
        dW2[e] = aw_d[:, r0:r1] @ dy_d[:, r0:r1].T
        dW1[e] = x_d[:, r0:r1] @ dh_d[:, r0:r1].T
    dx = combine(dx_perm, np.asarray(row_of, dtype=np.int64), k, None, True)
    out = dict(b)
    out.update(dx_perm=dx_perm, dx=dx, dW1=dW1, dW2=dW2, dh_q=dh_q, dh_s=dh_s, dht_q=dht_q,
               dht_s=dht_s, awt_q=awt_q, awt_s=awt_s, dyt_q=dyt_q, dyt_s=dyt_s, xt_q=xt_q,
               xt_s=xt_s, w1q=np.stack([q for q, _ in w1q]), w1s=np.stack([s for _, s in w1q]))
    out.update(extra)
    return out


def max_abs_normalised_error(got, ref) -> float:
    """max|got - ref| / max|ref| (0 when both are all-zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
