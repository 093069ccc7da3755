"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and host-side validation returns the documented status codes
before anything is launched (no GPU is touched)."""
import ctypes
import os
import re

import pytest

from fp4_block_scaled_route_amd import ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libnvfp4.so not built")
    return ops.lib()


def test_header_declares_the_binding_entry_points():
    assert _declared() == sorted(ops.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == ops.ABI_VERSION
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.nvfp4_status_string(code) != b"unknown status"
    assert lib.nvfp4_status_string(-99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)   # 16-byte aligned, never dereferenced: validation fails first


def test_linear_validation(lib):
    L = lib
    args = lambda **kw: dict(dict(x=FAKE, xq=None, xs=None, gsa=None, w=FAKE, ws=FAKE, gsb=FAKE,  # noqa: E731
                                  M=8, N=128, K=256, y=FAKE, work=FAKE, wb=1 << 20), **kw)

    def call(a):
        return L.nvfp4_linear(a["x"], a["xq"], a["xs"], a["gsa"], a["w"], a["ws"], a["gsb"],
                              a["M"], a["N"], a["K"], a["y"], a["work"], a["wb"], None)
    assert call(args(K=200)) == -2          # K not a multiple of 256
    assert call(args(N=100)) == -2          # N not a multiple of 16
    assert call(args(M=-1)) == -2
    assert call(args(M=0)) == 0             # nothing to do, nothing launched
    assert call(args(w=None)) == -1
    assert call(args(x=None)) == -1
    assert call(args(xq=FAKE)) == -6        # both activation forms
    assert call(args(y=ctypes.c_void_p(0x1004))) == -3
    assert call(args(work=None)) == -4
    assert call(args(wb=4)) == -4


def test_linear_small_row_counts_need_no_workspace(lib):
    """Up to 4 rows per group the linear is one launch that converts its
    activations in LDS and adds its K ranges there: no workspace.  More rows
    take the staged kernels."""
    L = lib
    for m in (1, 2, 3, 4):
        assert L.nvfp4_linear_workspace_size(m, 1536, 7168) == 0
        assert L.nvfp4_linear_workspace_size(m, 24576, 1536) == 0
        assert L.nvfp4_linear_workspace_size(m, 64, 8448) == 0
        assert L.nvfp4_linear_workspace_size(m, 16, 256) == 0
    assert L.nvfp4_grouped_linear_workspace_size(4, 8, 1024, 4096) == 0
    assert L.nvfp4_linear_workspace_size(1, 64, 16384) == 0
    assert L.nvfp4_linear_workspace_size(4, 64, 16384) > 0     # 16 waves x 2 slots x 4 rows exceed the LDS
    assert L.nvfp4_linear_workspace_size(5, 1536, 7168) > 0
    assert L.nvfp4_grouped_linear_workspace_size(5, 8, 1024, 4096) > 0


def test_grouped_linear_validation(lib):
    L = lib
    ws = L.nvfp4_grouped_linear_workspace_size(64, 8, 1024, 4096)
    assert ws >= 64 * 8 * 4096 * 2
    args = lambda **kw: dict(dict(x=FAKE, xq=None, xs=None, gsa=None, w=FAKE, ws=FAKE, ws2=FAKE,  # noqa: E731
                                  T=64, G=8, N=1024, K=4096, y=FAKE, work=FAKE, wb=ws), **kw)

    def call(a):
        return L.nvfp4_grouped_linear(a["x"], a["xq"], a["xs"], a["gsa"], a["w"], a["ws"], a["ws2"],
                                      a["T"], a["G"], a["N"], a["K"], a["y"], a["work"], a["wb"], None)
    assert call(args(K=4000)) == -2         # K not a multiple of 256
    assert call(args(N=1000)) == -2         # N not a multiple of 16
    assert call(args(G=0)) == -2
    assert call(args(T=-1)) == -2
    assert call(args(T=0)) == 0             # nothing to do, nothing launched
    assert call(args(ws2=None)) == -1
    assert call(args(x=None)) == -1
    assert call(args(xq=FAKE)) == -6        # both activation forms
    assert call(args(x=None, xq=FAKE, xs=FAKE)) == -1       # NVFP4 activations without their global scale
    assert call(args(y=ctypes.c_void_p(0x1004))) == -3
    assert call(args(ws2=ctypes.c_void_p(0x1002))) == -3
    assert call(args(work=None)) == -4
    assert call(args(wb=ws - 1)) == -4


def test_rmsnorm_quantize_validation(lib):
    L = lib
    ws = L.nvfp4_rmsnorm_quantize_workspace_size(64)
    assert ws >= 64 * 4

    def call(x=FAKE, w=FAKE, eps=1e-6, T=64, K=7168, y=None, gs=FAKE, comp=1, q=FAKE, sf=FAKE, work=FAKE, wb=ws):
        return L.nvfp4_rmsnorm_quantize(x, w, eps, T, K, y, gs, comp, q, sf, work, wb, None)
    assert call(K=100) == -2                 # K not a multiple of 16
    assert call(T=-1) == -2
    assert call(eps=0.0) == -6               # eps must be positive
    assert call(eps=float("nan")) == -6
    assert call(T=0, comp=0) == 0            # empty batch, supplied gs: nothing to launch
    assert call(T=0, x=None, w=None, q=None, sf=None, work=None, comp=0) == 0
    assert call(T=0, gs=None) == -1          # empty batch still writes a computed gs
    assert call(T=0, gs=ctypes.c_void_p(0x1002)) == -3
    assert call(w=None) == -1
    assert call(gs=None) == -1
    assert call(x=ctypes.c_void_p(0x1008)) == -3
    assert call(y=ctypes.c_void_p(0x1004)) == -3
    assert call(work=None) == -4
    assert call(wb=ws - 1) == -4


def test_quantize_validation(lib):
    L = lib
    ws = L.nvfp4_quantize_act_workspace_size(4, 64)
    assert ws > 0 and L.nvfp4_quantize_act_workspace_size(0, 64) == 0
    assert L.nvfp4_quantize_act(FAKE, 4, 40, FAKE, 1, FAKE, FAKE, FAKE, ws, None) == -2
    assert L.nvfp4_quantize_act(FAKE, 4, 64, None, 1, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.nvfp4_quantize_act(None, 4, 64, FAKE, 1, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.nvfp4_quantize_act(ctypes.c_void_p(0x1002), 4, 64, FAKE, 1, FAKE, FAKE, FAKE, ws, None) == -3
    assert L.nvfp4_quantize_act(FAKE, 4, 64, FAKE, 1, FAKE, FAKE, None, 0, None) == -4     # computed gs needs it
    assert L.nvfp4_quantize_act(FAKE, 4, 64, FAKE, 1, FAKE, FAKE, FAKE, ws - 1, None) == -4


def test_moe_validation(lib):
    L = lib
    ws_shared = L.nvfp4_moe_workspace_size(64, 7168, 2048, 384, 8, 1, 0)
    ws = L.nvfp4_moe_workspace_size(64, 7168, 2048, 384, 8, 0, 0)      # no shared expert, fp32 h
    ws4 = L.nvfp4_moe_workspace_size(64, 7168, 2048, 384, 8, 0, 1)     # NVFP4 h
    assert ws_shared > ws > ws4 > 0

    def base(**kw):
        a = ops.MoeArgs()
        a.T, a.H, a.I, a.E, a.topk = 64, 7168, 2048, 384, 8
        for f in ("x", "topk_ids", "topk_w", "w1", "w1_sf", "w1_ws2", "w2", "w2_sf", "w2_ws2", "y", "workspace"):
            setattr(a, f, FAKE)
        a.workspace_bytes = ws
        for k, v in kw.items():
            setattr(a, k, v)
        return L.nvfp4_moe_grouped(ctypes.byref(a), None)
    assert base(H=7000) == -2
    assert base(I=100) == -2
    assert base(E=1000) == -2               # more experts than the permutation supports
    assert base(topk=400) == -2
    assert base(T=0) == 0
    assert base(w1=None) == -1
    assert base(x=None) == -1
    assert base(x_fp4=FAKE, x_sf=FAKE, a1_gs=FAKE) == -6     # both activation forms
    assert base(s1=FAKE) == -1                                # half a shared expert
    assert base(s2=FAKE) == -6
    assert base(a2_gs=FAKE, a2_gs_out=FAKE) == -6
    assert base(workspace_bytes=ws - 1) == -4
    assert base(y=ctypes.c_void_p(0x1008)) == -3


def test_moe_noalloc_validation(lib):
    """Host-side checks of the no-allocation entry point: the same argument
    checks as nvfp4_moe_grouped, no workspace accepted, and calls needing
    more than the static scratch array rejected before any launch."""
    L = lib

    def call(**kw):
        a = ops.MoeArgs()
        a.T, a.H, a.I, a.E, a.topk = 64, 7168, 2048, 384, 8
        for f in ("x", "topk_ids", "topk_w", "w1", "w1_sf", "w1_ws2", "w2", "w2_sf", "w2_ws2", "y"):
            setattr(a, f, FAKE)
        for k, v in kw.items():
            setattr(a, k, v)
        return L.nvfp4_moe_grouped_noalloc(ctypes.byref(a), None)
    assert call(T=0) == 0
    assert call(H=7000) == -2
    assert call(w1=None) == -1
    assert call(workspace=FAKE, workspace_bytes=1 << 30) == -6    # no workspace is taken
    limit = 72 << 20
    assert L.nvfp4_moe_workspace_size(298, 7168, 2048, 384, 8, 1, 0) > limit
    assert L.nvfp4_moe_workspace_size(297, 7168, 2048, 384, 8, 1, 0) <= limit
    assert call(T=298, s1=FAKE, s1_sf=FAKE, s1_ws2=FAKE, s2=FAKE, s2_sf=FAKE, s2_ws2=FAKE) == -7
    assert call(T=4096, x=None, x_fp4=FAKE, x_sf=FAKE, a1_gs=FAKE, a2_gs=FAKE) == -7


def test_router_validation(lib):
    L = lib
    mis = ctypes.c_void_p(0x1002)
    assert L.nvfp4_router_prepare(FAKE, 384, 200, FAKE, FAKE, None) == -2     # H not a multiple of 256
    assert L.nvfp4_router_prepare(FAKE, 0, 256, FAKE, FAKE, None) == -2
    assert L.nvfp4_router_prepare(None, 384, 256, FAKE, FAKE, None) == -1
    assert L.nvfp4_router_prepare(mis, 384, 256, FAKE, FAKE, None) == -3

    def topk(**kw):
        a = dict(x=FAKE, w=FAKE, T=64, H=7168, E=384, k=8, lg=FAKE, ids=FAKE, wt=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return L.nvfp4_router_topk(a["x"], a["w"], a["T"], a["H"], a["E"], a["k"], a["lg"], a["ids"], a["wt"],
                                   a["ws"], a["wsb"], None)
    assert topk(E=513) == -2                 # more experts than the selection kernel holds
    assert topk(k=0) == -2
    assert topk(k=65) == -2
    assert topk(E=4, k=5) == -2
    assert topk(H=100) == -2
    assert topk(T=0) == 0                    # nothing to do
    assert topk(ids=None) == -1
    assert topk(lg=ctypes.c_void_p(0x1001)) == -3
    need = L.nvfp4_router_workspace_size(64, 7168, 384)
    assert need > 0
    assert topk(wsb=need - 1) == -4
    assert topk(ws=None) == -4
