"""ctypes binding of libmoe.so: the C ABI of include/moe.h with the same names.

Argument marshalling only: every step runs in the library's HIP kernels, on
torch's current HIP stream. torch tensors supply device memory; bf16 tensors
are passed by address (torch.bfloat16 or int16/uint16 bit patterns).
Failing to load the library raises immediately -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_LAUNCH = -4
MOE_ALIGN = 128
MOE_MX_BLOCK = 32
MOE_GLU_INTERLEAVE = 32
MOE_MAX_EXPERTS = 1024
MOE_ACT_SWIGLU = 0
MOE_ACT_GEGLU = 1
MOE_ACT_SRELU = 2   # non-gated relu(h)^2: FC1 width n
MOE_STAGE_FC1 = 0x01
MOE_STAGE_FC2 = 0x02
MOE_STAGE_DGRAD2 = 0x04
MOE_STAGE_WGRAD2 = 0x08
MOE_STAGE_DGRAD1 = 0x10
MOE_STAGE_WGRAD1 = 0x20
MOE_STAGES_FWD = MOE_STAGE_FC1 | MOE_STAGE_FC2
MOE_STAGES_BWD = MOE_STAGE_DGRAD2 | MOE_STAGE_WGRAD2 | MOE_STAGE_DGRAD1 | MOE_STAGE_WGRAD1
MOE_GATHER_ROWS = 0x100
MOE_ERRBIT_NONFINITE_LOGIT = 0x1
MOE_QUANT_ROWWISE = 0x1
MOE_QUANT_COLWISE = 0x2
MOE_ROUTE_STATIC_SCRATCH_BYTES = 8 << 20

# (name, restype, argtypes) of every exported symbol
_P = C.c_void_p
_I = C.c_int
_I64 = C.c_int64
_SZ = C.c_size_t
SIGNATURES = {
    "moe_status_str": (C.c_char_p, [_I]),
    "moe_capacity_rows": (_I64, [_I, _I, _I]),
    "moe_route_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_mlp_bwd_workspace_bytes": (_SZ, [_I, _I64]),
    "moe_route_counts": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "moe_route_counts_noalloc": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I64, _P, _P]),
    "moe_route_bwd": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_permute": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_grouped_mlp_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _I, C.c_uint, _P, _P, _P,
                                 _P, _P]),
    "moe_grouped_mlp_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _I,
                                 C.c_uint, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "moe_quant_mxfp8": (_I, [_P, _I, _I64, _I, _I, _P, _P, _P, _P, _P]),
    "moe_permute_quant_mxfp8": (_I, [_P, _P, _I, _I, _I, _I, _I64, _I, _P, _P, _P, _P, _P]),
}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_lib().moe_status_str(status).decode()} ({status})")
        self.status = status


MX_FWD_FIELDS = ("a_q", "a_s", "at_q", "at_s", "w2t_q", "w2t_s", "x_q", "x_s", "w1t_q", "w1t_s",
                 "y_q", "y_s", "yt_q", "yt_s")
MX_BWD_FIELDS = ("dh_q", "dh_s", "dht_q", "dht_s", "awt_q", "awt_s", "dyt_q", "dyt_s", "xt_q", "xt_s",
                 "w1_q", "w1_s", "dy_q", "dy_s", "w2_q", "w2_s", "dx_q", "dx_s",
                 "dxt_q", "dxt_s")


class moe_mx_fwd(C.Structure):
    _fields_ = [(name, _P) for name in MX_FWD_FIELDS]


class moe_mx_bwd(C.Structure):
    _fields_ = [(name, _P) for name in MX_BWD_FIELDS]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run ragged_grouped_gemm_device_amd.build")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def load():
    """Load libmoe.so (raises if it is missing) and return the CDLL."""
    return _lib()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoEError(fn, rc)


# ------------------------------------------------------------------ host-only
def moe_status_str(status: int) -> str:
    return _lib().moe_status_str(status).decode()


def moe_capacity_rows(T: int, k: int, E: int) -> int:
    return int(_lib().moe_capacity_rows(T, k, E))


def moe_route_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(_lib().moe_route_workspace_bytes(T, k, E))


def moe_mlp_bwd_workspace_bytes(n: int, M_cap: int) -> int:
    return int(_lib().moe_mlp_bwd_workspace_bytes(n, M_cap))


# ------------------------------------------------------------------ device calls
def moe_route_counts(logits, k, topk_idx, topk_w, counts, offsets, row_of, src_of, M_cap,
                     err_word, workspace, renorm=False):
    T, E = logits.shape
    rc = _lib().moe_route_counts(_ptr(logits), T, E, k, int(bool(renorm)), _ptr(topk_idx),
                                 _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(row_of),
                                 _ptr(src_of), M_cap, _ptr(err_word), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream())
    _check("moe_route_counts", rc)


def moe_route_counts_noalloc(logits, k, topk_idx, topk_w, counts, offsets, row_of, src_of, M_cap,
                             err_word, renorm=False):
    """moe_route_counts on the library's static scratch (no workspace argument)."""
    T, E = logits.shape
    rc = _lib().moe_route_counts_noalloc(_ptr(logits), T, E, k, int(bool(renorm)), _ptr(topk_idx),
                                         _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(row_of),
                                         _ptr(src_of), M_cap, _ptr(err_word), _stream())
    _check("moe_route_counts_noalloc", rc)


def moe_route_bwd(logits, topk_idx, ds, dlogits, renorm=False):
    T, E = logits.shape
    k = topk_idx.shape[1]
    rc = _lib().moe_route_bwd(_ptr(logits), _ptr(topk_idx), _ptr(ds), T, E, k, int(renorm),
                              _ptr(dlogits), _stream())
    _check("moe_route_bwd", rc)


def moe_permute(x, row_of, src_of, offsets, k, E, x_perm):
    T, d = x.shape
    rc = _lib().moe_permute(_ptr(x), _ptr(row_of), _ptr(src_of), _ptr(offsets), T, k, E, d,
                            x_perm.shape[0], _ptr(x_perm), _stream())
    _check("moe_permute", rc)


def moe_combine(y, row_of, w, k, out):
    T, d = out.shape
    rc = _lib().moe_combine(_ptr(y), _ptr(row_of), _ptr(w), T, k, d, _ptr(out), _stream())
    _check("moe_combine", rc)


def _fits(t, rows, cols, name):
    """The C ABI takes bare pointers: a tensor given for an operand of `cols` columns must be a
    dense [>= rows, cols] matrix (or [E, rows, cols] when rows is a tuple), else the kernels
    would address past it."""
    if t is None:
        return
    want = tuple(rows) + (cols,) if isinstance(rows, tuple) else None
    ok = t.is_contiguous() and (tuple(t.shape) == want if want else
                                t.dim() == 2 and t.shape[1] == cols and t.shape[0] >= rows)
    if not ok:
        raise ValueError(f"{name}: shape {tuple(t.shape)} does not fit "
                         f"{want if want else f'[>= {rows}, {cols}]'} (dense)")


def moe_grouped_mlp_fwd(x_perm, w1, w2, offsets, h, a, y, stages=MOE_STAGES_FWD, mx=None,
                        act=MOE_ACT_SWIGLU, src_of=None, k=0):
    """With MOE_GATHER_ROWS in stages, x_perm is the un-permuted x [T, d] and src_of, k are
    required."""
    E, d, n1 = w1.shape
    n = n1 if act == MOE_ACT_SRELU else n1 // 2
    M_cap = (a if a is not None else mx["a_q"]).shape[0]  # a may be None with mx
    T = x_perm.shape[0] if (stages & MOE_GATHER_ROWS) else 0
    if x_perm is not None:
        _fits(x_perm, T if (stages & MOE_GATHER_ROWS) else M_cap, d, "x_perm")
    _fits(w2, (E, n), d, "w2")
    _fits(h, M_cap, n1, "h")
    _fits(a, M_cap, n, "a")
    _fits(y, M_cap, d, "y")
    mxp = None
    if mx is not None:
        mxs = moe_mx_fwd(*[_ptr(mx.get(key)) for key in MX_FWD_FIELDS])
        mxp = C.byref(mxs)
    rc = _lib().moe_grouped_mlp_fwd(_ptr(x_perm), _ptr(w1), _ptr(w2), _ptr(offsets), _ptr(src_of), T,
                                    k, E, d, n, M_cap, act, stages, _ptr(h), _ptr(a), _ptr(y),
                                    mxp, _stream())
    _check("moe_grouped_mlp_fwd", rc)


def moe_grouped_mlp_bwd(x_perm, w1, w2, h, dy_u, topk_w, src_of, row_of, offsets, dh, a_w, ds,
                        dx_perm, dw1, dw2, workspace, stages=MOE_STAGES_BWD, act=MOE_ACT_SWIGLU,
                        mx=None, shape=None):
    """mx: dict of the moe_mx_bwd fields (missing ones pass NULL). shape = (E, d, n) when w1
    is not given (an MX call that reads only the quantized copies)."""
    if w1 is not None:
        E, d, n1 = w1.shape
        n = n1 if act == MOE_ACT_SRELU else n1 // 2
    else:
        E, d, n = shape
    mxp = None
    if mx is not None:
        mxp = C.byref(moe_mx_bwd(*[_ptr(mx.get(key)) for key in MX_BWD_FIELDS]))
    T, k = topk_w.shape
    M_cap = src_of.shape[0]
    n1 = n if act == MOE_ACT_SRELU else 2 * n
    rows_in = T if (stages & MOE_GATHER_ROWS) else M_cap
    _fits(x_perm, rows_in, d, "x_perm")
    _fits(dy_u, rows_in, d, "dy_u")
    _fits(w2, (E, n), d, "w2")
    _fits(h, M_cap, n1, "h")
    _fits(dh, M_cap, n1, "dh")
    _fits(a_w, M_cap, n, "a_w")
    _fits(dx_perm, M_cap, d, "dx_perm")
    _fits(dw1, (E, d), n1, "dw1")
    _fits(dw2, (E, n), d, "dw2")
    rc = _lib().moe_grouped_mlp_bwd(_ptr(x_perm), _ptr(w1), _ptr(w2), _ptr(h), _ptr(dy_u),
                                    _ptr(topk_w), _ptr(src_of), _ptr(row_of), _ptr(offsets), T, k,
                                    E, d, n, M_cap, act, stages, _ptr(dh), _ptr(a_w), _ptr(ds),
                                    _ptr(dx_perm), _ptr(dw1), _ptr(dw2), _ptr(workspace),
                                    0 if workspace is None else workspace.numel() * workspace.element_size(),
                                    mxp, _stream())
    _check("moe_grouped_mlp_bwd", rc)


def moe_quant_mxfp8(src, mode, q_row=None, s_row=None, q_col=None, s_col=None):
    if src.dim() == 2:
        batch, (R, Cc) = 1, src.shape
    else:
        batch, R, Cc = src.shape
    rc = _lib().moe_quant_mxfp8(_ptr(src), batch, R, Cc, mode, _ptr(q_row), _ptr(s_row),
                                _ptr(q_col), _ptr(s_col), _stream())
    _check("moe_quant_mxfp8", rc)


def moe_permute_quant_mxfp8(x, src_of, k, E, mode, q_row=None, s_row=None, q_col=None, s_col=None):
    T, d = x.shape
    rc = _lib().moe_permute_quant_mxfp8(_ptr(x), _ptr(src_of), T, k, E, d, src_of.shape[0], mode,
                                        _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _stream())
    _check("moe_permute_quant_mxfp8", rc)


# ------------------------------------------------------------------ buffers
class Buffers:
    """Device buffers of one forward + backward pass (plain torch allocations)."""

    def __init__(self, T: int, k: int, E: int, d: int, n: int, device="cuda", mx: bool = False,
                 gated: bool = True):
        dev = torch.device(device)
        bf, i32, f32, u8 = torch.bfloat16, torch.int32, torch.float32, torch.uint8
        self.T, self.k, self.E, self.d, self.n = T, k, E, d, n
        self.M_cap = M = moe_capacity_rows(T, k, E)
        self.topk_idx = torch.empty(T, k, dtype=i32, device=dev)
        self.topk_w = torch.empty(T, k, dtype=f32, device=dev)
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.row_of = torch.empty(T * k, dtype=i32, device=dev)
        self.src_of = torch.empty(M, dtype=i32, device=dev)
        self.err = torch.zeros(1, dtype=i32, device=dev)
        self.route_ws = torch.empty(max(16, moe_route_workspace_bytes(T, k, E)), dtype=u8, device=dev)
        self.x_perm = torch.empty(M, d, dtype=bf, device=dev)
        n1 = 2 * n if gated else n   # FC1 width (non-gated sReLU: n)
        self.h = torch.empty(M, n1, dtype=bf, device=dev)
        self.a = torch.empty(M, n, dtype=bf, device=dev)
        self.y = torch.empty(M, d, dtype=bf, device=dev)
        self.out = torch.empty(T, d, dtype=bf, device=dev)
        self.dy_u = torch.empty(M, d, dtype=bf, device=dev)
        self.dh = torch.empty(M, n1, dtype=bf, device=dev)
        self.a_w = torch.empty(M, n, dtype=bf, device=dev)
        self.ds = torch.empty(T, k, dtype=f32, device=dev)
        self.dx_perm = torch.empty(M, d, dtype=bf, device=dev)
        self.dx = torch.empty(T, d, dtype=bf, device=dev)
        self.dw1 = torch.empty(E, d, n1, dtype=f32, device=dev)
        self.dw2 = torch.empty(E, n, d, dtype=f32, device=dev)
        self.dlogits = torch.empty(T, E, dtype=f32, device=dev)
        self.bwd_ws = torch.empty(max(16, moe_mlp_bwd_workspace_bytes(n, M)), dtype=u8, device=dev)
        if mx:
            self.a_q = torch.empty(M, n, dtype=u8, device=dev)
            self.a_s = torch.empty(M, n // 32, dtype=u8, device=dev)
            self.at_q = torch.empty(n, M, dtype=u8, device=dev)
            self.at_s = torch.empty(n, M // 32, dtype=u8, device=dev)
            self.w2t_q = torch.empty(E, d, n, dtype=u8, device=dev)
            self.w2t_s = torch.empty(E, d, n // 32, dtype=u8, device=dev)
            self.dh_q = torch.empty(M, 2 * n, dtype=u8, device=dev)
            self.dh_s = torch.empty(M, 2 * n // 32, dtype=u8, device=dev)
            self.dht_q = torch.empty(2 * n, M, dtype=u8, device=dev)
            self.dht_s = torch.empty(2 * n, M // 32, dtype=u8, device=dev)
            self.awt_q = torch.empty(n, M, dtype=u8, device=dev)
            self.awt_s = torch.empty(n, M // 32, dtype=u8, device=dev)
            self.dyt_q = torch.empty(d, M, dtype=u8, device=dev)
            self.dyt_s = torch.empty(d, M // 32, dtype=u8, device=dev)
            self.xt_q = torch.empty(d, M, dtype=u8, device=dev)
            self.xt_s = torch.empty(d, M // 32, dtype=u8, device=dev)
            self.w1_q = torch.empty(E, d, 2 * n, dtype=u8, device=dev)
            self.w1_s = torch.empty(E, d, 2 * n // 32, dtype=u8, device=dev)
            self.x_q = torch.empty(M, d, dtype=u8, device=dev)
            self.x_s = torch.empty(M, d // 32, dtype=u8, device=dev)
            self.w1t_q = torch.empty(E, 2 * n, d, dtype=u8, device=dev)
            self.w1t_s = torch.empty(E, 2 * n, d // 32, dtype=u8, device=dev)
            self.dy_q = torch.empty(M, d, dtype=u8, device=dev)
            self.dy_s = torch.empty(M, d // 32, dtype=u8, device=dev)
            self.w2_q = torch.empty(E, n, d, dtype=u8, device=dev)
            self.w2_s = torch.empty(E, n, d // 32, dtype=u8, device=dev)
            # row-wise MXFP8 copies of the FC2 output and of the FC1 dgrad output
            # (GroupGemm + Quantize), written only when asked
            self.y_q = torch.empty(M, d, dtype=u8, device=dev)
            self.y_s = torch.empty(M, d // 32, dtype=u8, device=dev)
            self.dx_q = torch.empty(M, d, dtype=u8, device=dev)
            self.dx_s = torch.empty(M, d // 32, dtype=u8, device=dev)
            # and their column-wise copies, transposed
            self.yt_q = torch.empty(d, M, dtype=u8, device=dev)
            self.yt_s = torch.empty(d, M // 32, dtype=u8, device=dev)
            self.dxt_q = torch.empty(d, M, dtype=u8, device=dev)
            self.dxt_s = torch.empty(d, M // 32, dtype=u8, device=dev)
        self.xt_from_forward = False

    def quantize_weights(self, w1, w2):
        """MXFP8 weight copies: W1_e along 2n [E, d, 2n] (FC1 dgrad) and along d, transposed
        [E, 2n, d] (FC1); W2_e along d [E, n, d] (FC2 dgrad) and along n, transposed [E, d, n]
        (FC2)."""
        moe_quant_mxfp8(w1, MOE_QUANT_ROWWISE | MOE_QUANT_COLWISE, self.w1_q, self.w1_s, self.w1t_q,
                        self.w1t_s)
        moe_quant_mxfp8(w2, MOE_QUANT_ROWWISE | MOE_QUANT_COLWISE, self.w2_q, self.w2_s, self.w2t_q,
                        self.w2t_s)

    def mx_fwd(self, fc1=True, transposed_a=False, quant_y=False, transposed_y=False):
        """The moe_mx_fwd fields: FC1 on MXFP8 operands when fc1; the transposed copy of A
        only when asked (the training step's FC2 wgrad reads A' = w A, quantized by the FC2
        dgrad, not A); the row-wise MXFP8 copy of Y (FC2 epilogue) when quant_y, with its
        transposed column-wise copy when transposed_y."""
        keys = MX_FWD_FIELDS[:10] if fc1 else MX_FWD_FIELDS[:6]
        d = {key: getattr(self, key) for key in keys}
        if not transposed_a:
            d["at_q"] = d["at_s"] = None
        if quant_y:
            d["y_q"], d["y_s"] = self.y_q, self.y_s
            if transposed_y:
                d["yt_q"], d["yt_s"] = self.yt_q, self.yt_s
        return d

    def mx_bwd(self, dgrad2=True, quant_dx=False, transposed_dx=False):
        keys = MX_BWD_FIELDS[:16] if dgrad2 else MX_BWD_FIELDS[:12]
        d = {key: getattr(self, key) for key in keys}
        if quant_dx:
            d["dx_q"], d["dx_s"] = self.dx_q, self.dx_s
            if transposed_dx:
                d["dxt_q"], d["dxt_s"] = self.dxt_q, self.dxt_s
        return d


def forward(buf: Buffers, x, logits, w1, w2, renorm=False, fwd_stages=MOE_STAGES_FWD, store_h=True,
            act=MOE_ACT_SWIGLU, gather=False, mx=False):
    """route -> permute -> FC1+GLU -> FC2 -> combine (all enqueued, no sync). With gather, FC1
    reads the rows of x through src_of and no permuted copy is made. With mx (buffers made with
    mx=True, quantize_weights done), X_perm is quantized row-wise (FC1 operand) and column-wise
    (FC1 wgrad operand) in one pass and both GEMMs run on MXFP8."""
    moe_route_counts(logits, buf.k, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets, buf.row_of,
                     buf.src_of, buf.M_cap, buf.err, buf.route_ws, renorm)
    buf.xt_from_forward = bool(mx)
    if mx:
        if gather:
            raise ValueError("the MXFP8 FC1 reads the quantized permuted copy: no row gather")
        # X_perm only as its MXFP8 copies: row-wise (FC1) and column-wise (FC1 wgrad)
        moe_permute_quant_mxfp8(x, buf.src_of, buf.k, buf.E, MOE_QUANT_ROWWISE | MOE_QUANT_COLWISE,
                                buf.x_q, buf.x_s, buf.xt_q, buf.xt_s)
        moe_grouped_mlp_fwd(None, w1, w2, buf.offsets, buf.h if store_h else None, buf.a,
                            buf.y, fwd_stages, mx=buf.mx_fwd(), act=act)
    elif gather:
        moe_grouped_mlp_fwd(x, w1, w2, buf.offsets, buf.h if store_h else None, buf.a, buf.y,
                            fwd_stages | MOE_GATHER_ROWS, act=act, src_of=buf.src_of, k=buf.k)
    else:
        moe_permute(x, buf.row_of, buf.src_of, buf.offsets, buf.k, buf.E, buf.x_perm)
        moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h if store_h else None, buf.a,
                            buf.y, fwd_stages, act=act)
    moe_combine(buf.y, buf.row_of, buf.topk_w, buf.k, buf.out)


def backward(buf: Buffers, dout, w1, w2, stages=MOE_STAGES_BWD, act=MOE_ACT_SWIGLU, logits=None,
             renorm=False, x=None, mx=False, dgrad2_mx=True, mx_bf16_copies=True):
    """gather dO -> dgrad2+dGLU (+dS) -> wgrad2 -> dgrad1 -> unpermute-sum -> wgrad1, and with
    the forward's logits also the router backward dS -> dlogits. With x given (the un-permuted
    input), the GEMMs read x and dO through src_of instead of permuted copies. With mx (buffers
    made with mx=True and quantize_weights done), dY_u is quantized (row-wise for the FC2 dgrad
    when dgrad2_mx, column-wise for the FC2 wgrad), X_perm column-wise unless the MXFP8 forward
    already did, and the GEMMs run on MXFP8 (the FC2 dgrad only with dgrad2_mx). With mx and
    mx_bf16_copies=False the FC2 dgrad writes only the MXFP8 copies of dH and A' (buf.dh and
    buf.a_w are left untouched), which is all the later MXFP8 stages read. The FC1 wgrad runs
    last, after the unpermute-sum has read dX_perm."""
    early, late = stages & ~MOE_STAGE_WGRAD1, stages & MOE_STAGE_WGRAD1
    if mx:
        if x is not None:
            raise ValueError("the MXFP8 backward quantizes the permuted copies: no row gather")
        if dgrad2_mx:   # dY_u only as its MXFP8 copies
            moe_permute_quant_mxfp8(dout, buf.src_of, buf.k, buf.E, MOE_QUANT_ROWWISE | MOE_QUANT_COLWISE,
                                    buf.dy_q, buf.dy_s, buf.dyt_q, buf.dyt_s)
        else:
            moe_permute(dout, buf.row_of, buf.src_of, buf.offsets, buf.k, buf.E, buf.dy_u)
            moe_quant_mxfp8(buf.dy_u, MOE_QUANT_COLWISE, None, None, buf.dyt_q, buf.dyt_s)
        if not buf.xt_from_forward:
            moe_quant_mxfp8(buf.x_perm, MOE_QUANT_COLWISE, None, None, buf.xt_q, buf.xt_s)
        dh, a_w = (buf.dh, buf.a_w) if mx_bf16_copies else (None, None)
        bwd = lambda st: moe_grouped_mlp_bwd(buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of,
                                             buf.row_of, buf.offsets, dh, a_w, buf.ds, buf.dx_perm, buf.dw1,
                                             buf.dw2, buf.bwd_ws, st, act=act, mx=buf.mx_bwd(dgrad2_mx))
    elif x is not None:
        bwd = lambda st: moe_grouped_mlp_bwd(x, w1, w2, buf.h, dout, buf.topk_w, buf.src_of, buf.row_of,
                                             buf.offsets, buf.dh, buf.a_w, buf.ds, buf.dx_perm, buf.dw1,
                                             buf.dw2, buf.bwd_ws, st | MOE_GATHER_ROWS, act=act)
    else:
        moe_permute(dout, buf.row_of, buf.src_of, buf.offsets, buf.k, buf.E, buf.dy_u)
        bwd = lambda st: moe_grouped_mlp_bwd(buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of,
                                             buf.row_of, buf.offsets, buf.dh, buf.a_w, buf.ds, buf.dx_perm,
                                             buf.dw1, buf.dw2, buf.bwd_ws, st, act=act)
    if early:
        bwd(early)
    moe_combine(buf.dx_perm, buf.row_of, None, buf.k, buf.dx)
    if late:
        bwd(late)
    if logits is not None:
        moe_route_bwd(logits, buf.topk_idx, buf.ds, buf.dlogits, renorm)
