"""The C ABI library loads, exports every symbol include/moe.h declares, and
rejects invalid arguments on the host before launching anything (CPU only)."""
import ctypes as C
import os
import re

import pytest

from ragged_grouped_gemm_device_amd import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="libmoe.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = M.load()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
        assert n in M.SIGNATURES, n


def test_constants_match_header():
    src = open(HEADER).read()
    for name in ("MOE_ALIGN", "MOE_MX_BLOCK", "MOE_GLU_INTERLEAVE", "MOE_MAX_EXPERTS",
                 "MOE_STAGE_FC1", "MOE_STAGE_FC2", "MOE_STAGE_DGRAD2", "MOE_STAGE_WGRAD2",
                 "MOE_STAGE_DGRAD1", "MOE_STAGE_WGRAD1", "MOE_QUANT_ROWWISE", "MOE_QUANT_COLWISE",
                 "MOE_ERRBIT_NONFINITE_LOGIT", "MOE_ACT_SWIGLU", "MOE_ACT_GEGLU"):
        m = re.search(r"#define\s+%s\s+(\(?-?[0-9a-fx]+\)?)" % name, src)
        assert m, name
        assert int(m.group(1).strip("()"), 0) == getattr(M, name), name
    for name in ("MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
                 "MOE_ERR_LAUNCH"):
        m = re.search(r"#define\s+%s\s+\(?(-?\d+)\)?" % name, src)
        assert int(m.group(1)) == getattr(M, name)


def test_static_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define\s+MOE_ROUTE_STATIC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == M.MOE_ROUTE_STATIC_SCRATCH_BYTES
    launch = open(os.path.join(ROOT, "ragged_grouped_gemm_device_amd", "csrc", "launch.hpp")).read()
    m = re.search(r"kRouteStaticScratch\s*=\s*\(size_t\)(\d+)\s*<<\s*(\d+)", launch)
    assert m and int(m.group(1)) << int(m.group(2)) == M.MOE_ROUTE_STATIC_SCRATCH_BYTES


def test_status_strings_and_capacity():
    assert M.moe_status_str(0) == "MOE_OK"
    assert M.moe_status_str(-3) == "MOE_ERR_WORKSPACE"
    assert M.moe_status_str(12345) == "MOE_ERR_UNKNOWN"
    assert M.moe_capacity_rows(256, 2, 8) == 512 + 1024
    assert M.moe_capacity_rows(16384, 8, 32) == 131072 + 4096
    assert M.moe_capacity_rows(8192, 4, 32) == 32768 + 4096
    assert M.moe_capacity_rows(1, 1, 1) == 256
    assert M.moe_capacity_rows(10, 3, 2) == -1          # k > E
    assert M.moe_capacity_rows(10, 1, 2000) == -1       # E > MOE_MAX_EXPERTS
    assert M.moe_route_workspace_bytes(0, 1, 1) == 0
    # the layout's scratch: one histogram row of E counters per chunk on the
    # fused path (1024 threads route 1024 / G tokens per pass), two per 1024-pair
    # chunk on the general path
    assert M.moe_route_workspace_bytes(32768, 1, 8) == 256 * 8 * 4       # 128 tokens per chunk
    assert M.moe_route_workspace_bytes(16384, 8, 32) == 512 * 32 * 4     # 32 tokens per chunk
    assert M.moe_route_workspace_bytes(32700, 8, 32) == 511 * 32 * 4     # 2 passes of 32 tokens
    assert M.moe_route_workspace_bytes(20000, 4, 128) == 2 * 79 * 128 * 4
    assert M.moe_route_workspace_bytes(9000, 4, 1024) == 2 * 36 * 1024 * 4
    assert M.moe_mlp_bwd_workspace_bytes(2048, 1024) == 1024 * 32 * 4


def _fake(addr=0x1000):
    return C.c_void_p(addr)


def test_host_validation_returns_before_launch():
    lib = M.load()
    f = _fake()
    # NULL logits
    rc = lib.moe_route_counts(None, 8, 4, 2, 0, f, f, f, f, f, f, 1024, None, f, 1 << 20, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    # k > E
    rc = lib.moe_route_counts(f, 8, 4, 5, 0, f, f, f, f, f, f, 1024, None, f, 1 << 20, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    # capacity too small
    rc = lib.moe_route_counts(f, 8, 4, 2, 0, f, f, f, f, f, f, 100, None, f, 1 << 20, None)
    assert rc == M.MOE_ERR_WORKSPACE
    # workspace too small
    rc = lib.moe_route_counts(f, 8, 4, 2, 0, f, f, f, f, f, f, 1024, None, f, 0, None)
    assert rc == M.MOE_ERR_WORKSPACE
    # misaligned workspace
    rc = lib.moe_route_counts(f, 8, 4, 2, 0, f, f, f, f, f, f, 1024, None, _fake(0x1004), 1 << 20, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    # allocation-free routing: host checks as above, and a layout whose scratch would
    # exceed the static array (2^24 pairs x 1024 experts: 128 MiB) is refused
    rc = lib.moe_route_counts_noalloc(None, 8, 4, 2, 0, f, f, f, f, f, f, 1024, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    rc = lib.moe_route_counts_noalloc(f, 8, 4, 2, 0, f, f, f, f, f, f, 100, None, None)
    assert rc == M.MOE_ERR_WORKSPACE
    big_T, big_E = 1 << 21, 1024
    assert M.moe_route_workspace_bytes(big_T, 8, big_E) > M.MOE_ROUTE_STATIC_SCRATCH_BYTES
    rc = lib.moe_route_counts_noalloc(f, big_T, big_E, 8, 0, f, f, f, f, f, f,
                                      M.moe_capacity_rows(big_T, 8, big_E), None, None)
    assert rc == M.MOE_ERR_WORKSPACE
    # permute: d not a multiple of 8
    rc = lib.moe_permute(f, f, f, f, 8, 2, 4, 12, 1024, f, None)
    assert rc == M.MOE_ERR_UNSUPPORTED
    rc = lib.moe_permute(_fake(0x1002), f, f, f, 8, 2, 4, 16, 1024, f, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    rc = lib.moe_permute(f, None, f, f, 8, 2, 4, 16, 1024, f, None)  # NULL row_of
    assert rc == M.MOE_ERR_INVALID_ARG
    # router backward: k > E, NULL output
    rc = lib.moe_route_bwd(f, f, f, 8, 4, 5, 0, f, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    rc = lib.moe_route_bwd(f, f, f, 8, 4, 2, 0, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    # combine: NULL output
    rc = lib.moe_combine(f, f, None, 8, 2, 16, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    # mlp fwd: unsupported activation / shapes / stage bits
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 64, 1024, 7, 3, None, f, f, None, None)
    assert rc == M.MOE_ERR_UNSUPPORTED
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 96, 64, 1024, 0, 3, None, f, f, None, None)
    assert rc == M.MOE_ERR_UNSUPPORTED
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 64, 1000, 0, 3, None, f, f, None, None)
    assert rc == M.MOE_ERR_UNSUPPORTED
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 64, 1024, 0, 0x40, None, f, f, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 64, 1024, 0, 3, None, f, None, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG              # FC2 without y
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 64, 1024, 0, 3, None, None, f, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG              # a may be NULL only with mx
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 64, 1024, 0, 1, None, _fake(0x1004), f, None,
                                 None)
    assert rc == M.MOE_ERR_INVALID_ARG              # misaligned a
    # gathered rows need src_of, and a valid routing shape
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 8, 2, 4, 128, 64, 1024, 0, 0x101, None, f, f, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    rc = lib.moe_grouped_mlp_fwd(f, f, f, f, f, 8, 5, 4, 128, 64, 1024, 0, 0x101, None, f, f, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG              # k > E
    # mlp bwd: workspace too small for the dS partials
    rc = lib.moe_grouped_mlp_bwd(f, f, f, f, f, f, f, f, f, 8, 2, 4, 128, 64, 1024, 0, 0x04,
                                 f, f, f, f, f, f, f, 0, None, None)
    assert rc == M.MOE_ERR_WORKSPACE
    rc = lib.moe_grouped_mlp_bwd(f, f, f, f, f, f, f, f, f, 8, 2, 4, 128, 64, 256, 0, 0x04,
                                 f, f, f, f, f, f, f, 1 << 20, None, None)
    assert rc == M.MOE_ERR_WORKSPACE               # M_cap below capacity
    # dh and a_w may be NULL only with mx (their MXFP8 copies are then what the later stages read)
    for dh, a_w in ((None, f), (f, None)):
        rc = lib.moe_grouped_mlp_bwd(f, f, f, f, f, f, f, f, f, 8, 2, 4, 128, 64, 1024, 0, 0x04,
                                     dh, a_w, f, f, f, f, f, 1 << 20, None, None)
        assert rc == M.MOE_ERR_INVALID_ARG
    # MXFP8 backward: every copy a requested stage reads or writes must be given
    full = {key: f for key in M.MX_BWD_FIELDS}
    for stage, needed in ((0x04, ("dh_q", "dht_s", "awt_q")), (0x08, ("awt_s", "dyt_q")),
                          (0x10, ("dh_s", "w1_q")), (0x20, ("xt_q", "dht_q"))):
        for key in needed:
            mx = M.moe_mx_bwd(*[None if k2 == key else full[k2] for k2 in M.MX_BWD_FIELDS])
            rc = lib.moe_grouped_mlp_bwd(f, f, f, f, f, f, f, f, f, 8, 2, 4, 128, 64, 1024, 0, stage,
                                         f, f, f, f, f, f, f, 1 << 20, C.byref(mx), None)
            assert rc == M.MOE_ERR_INVALID_ARG, (stage, key)
    # the transposed copy of dX_perm needs its scales and the row-wise copy beside it
    for drop in ("dxt_s", "dx_q"):
        mx = M.moe_mx_bwd(*[None if k2 in (drop, "dx_s" if drop == "dx_q" else "") else full[k2]
                            for k2 in M.MX_BWD_FIELDS])
        rc = lib.moe_grouped_mlp_bwd(f, f, f, f, f, f, f, f, f, 8, 2, 4, 128, 64, 1024, 0, 0x10,
                                     f, f, f, f, f, f, f, 1 << 20, C.byref(mx), None)
        assert rc == M.MOE_ERR_INVALID_ARG, drop
    # likewise the transposed copy of Y in the forward
    fwd = {key: f for key in M.MX_FWD_FIELDS}
    for drop in ("yt_s", "y_q"):
        mxf = M.moe_mx_fwd(*[None if k2 in (drop, "y_s" if drop == "y_q" else "") else fwd[k2]
                             for k2 in M.MX_FWD_FIELDS])
        rc = lib.moe_grouped_mlp_fwd(f, f, f, f, None, 0, 0, 4, 128, 128, 1024, 0, 2, None, f, f,
                                     C.byref(mxf), None)
        assert rc == M.MOE_ERR_INVALID_ARG, drop
    mx = M.moe_mx_bwd(*[_fake(0x1001) if k2 == "w1_q" else full[k2] for k2 in M.MX_BWD_FIELDS])
    rc = lib.moe_grouped_mlp_bwd(f, f, f, f, f, f, f, f, f, 8, 2, 4, 128, 64, 1024, 0, 0x10,
                                 f, f, f, f, f, f, f, 1 << 20, C.byref(mx), None)
    assert rc == M.MOE_ERR_INVALID_ARG             # misaligned codes
    # fused permute + quant: shape and capacity checks
    rc = lib.moe_permute_quant_mxfp8(f, f, 8, 2, 4, 48, 1024, 3, f, f, f, f, None)
    assert rc == M.MOE_ERR_UNSUPPORTED              # d % 32
    rc = lib.moe_permute_quant_mxfp8(f, f, 8, 2, 4, 64, 256, 3, f, f, f, f, None)
    assert rc == M.MOE_ERR_WORKSPACE                # M_cap below capacity
    rc = lib.moe_permute_quant_mxfp8(f, None, 8, 2, 4, 64, 1024, 3, f, f, f, f, None)
    assert rc == M.MOE_ERR_INVALID_ARG              # no src_of
    rc = lib.moe_permute_quant_mxfp8(f, f, 8, 2, 4, 64, 1024, 1, None, f, None, None, None)
    assert rc == M.MOE_ERR_INVALID_ARG              # row-wise without codes
    # quant: bad mode / shape
    rc = lib.moe_quant_mxfp8(f, 1, 64, 64, 0, f, f, f, f, None)
    assert rc == M.MOE_ERR_INVALID_ARG
    rc = lib.moe_quant_mxfp8(f, 1, 64, 48, 1, f, f, None, None, None)
    assert rc == M.MOE_ERR_UNSUPPORTED
    rc = lib.moe_quant_mxfp8(f, 1, 40, 64, 2, None, None, f, f, None)
    assert rc == M.MOE_ERR_UNSUPPORTED


def test_binding_refuses_operands_of_the_wrong_shape():
    """The C ABI takes bare pointers; the binding checks every operand it sizes (raises
    before any call), so a W1 of another layout cannot make the kernels write past H."""
    import torch
    E, d, n, M_cap = 2, 256, 64, 512
    bf = torch.bfloat16
    x = torch.zeros(M_cap, d, dtype=bf)
    w1, w2 = torch.zeros(E, d, 2 * n, dtype=bf), torch.zeros(E, n, d, dtype=bf)
    offs = torch.zeros(E + 1, dtype=torch.int32)
    h, a, y = torch.zeros(M_cap, 2 * n, dtype=bf), torch.zeros(M_cap, n, dtype=bf), torch.zeros(M_cap, d, dtype=bf)
    w1t = w1.transpose(1, 2).contiguous()     # [E, 2n, d]: read as d = 2n, n1 = d
    with pytest.raises(ValueError):
        M.moe_grouped_mlp_fwd(x, w1t, w2, offs, h, a, y, M.MOE_STAGE_FC1)
    with pytest.raises(ValueError):
        M.moe_grouped_mlp_fwd(x, w1, w2, offs, h[:, :n], a, y, M.MOE_STAGE_FC1)
    with pytest.raises(ValueError):
        M.moe_grouped_mlp_fwd(x[:, :64], w1, w2, offs, h, a, y, M.MOE_STAGE_FC1)
    with pytest.raises(ValueError):
        M.moe_grouped_mlp_fwd(x, w1, w2.transpose(1, 2), offs, h, a, y, M.MOE_STAGE_FC2)
