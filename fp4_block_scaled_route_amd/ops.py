"""ctypes binding of libnvfp4.so (declared in include/nvfp4.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch is used for device memory (outputs and workspace are
allocated here when the caller does not pass them) and for the current HIP
stream.  If the library has not been built, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p

EXPORTED = (
    "nvfp4_status_string",
    "nvfp4_abi_version",
    "nvfp4_quantize_act_workspace_size",
    "nvfp4_quantize_act",
    "nvfp4_rmsnorm_quantize_workspace_size",
    "nvfp4_rmsnorm_quantize",
    "nvfp4_linear_workspace_size",
    "nvfp4_linear",
    "nvfp4_grouped_linear_workspace_size",
    "nvfp4_grouped_linear",
    "nvfp4_moe_workspace_size",
    "nvfp4_moe_grouped",
    "nvfp4_moe_grouped_noalloc",
    "nvfp4_router_prepare",
    "nvfp4_router_workspace_size",
    "nvfp4_router_topk",
)
ABI_VERSION = 2


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"nvfp4 status {status}: {msg}")
        self.status = status


class MoeArgs(ctypes.Structure):
    """Mirror of nvfp4_moe_args (field order and types as in include/nvfp4.h)."""
    _fields_ = [
        ("T", _c_i64), ("H", _c_i64), ("I", _c_i64), ("E", _c_i64), ("topk", _c_i64),
        ("x", _c_ptr), ("x_fp4", _c_ptr), ("x_sf", _c_ptr), ("a1_gs", _c_ptr),
        ("a2_gs", _c_ptr), ("a2_gs_out", _c_ptr),
        ("topk_ids", _c_ptr), ("topk_w", _c_ptr),
        ("w1", _c_ptr), ("w1_sf", _c_ptr), ("w1_ws2", _c_ptr),
        ("w2", _c_ptr), ("w2_sf", _c_ptr), ("w2_ws2", _c_ptr),
        ("s1", _c_ptr), ("s1_sf", _c_ptr), ("s1_ws2", _c_ptr),
        ("s2", _c_ptr), ("s2_sf", _c_ptr), ("s2_ws2", _c_ptr),
        ("workspace", _c_ptr), ("workspace_bytes", ctypes.c_size_t),
        ("offsets_out", _c_ptr), ("perm_out", _c_ptr),
        ("y", _c_ptr),
        ("stage_events", ctypes.POINTER(_c_ptr)),
    ]


# ---------------------------------------------------------------------------
# argument checks: the C ABI takes raw pointers and cannot see dtypes, shapes,
# strides or devices, so every tensor is checked here before its pointer is
# passed: dtypes, shapes (consistent with the sizes the call derives from its
# weights and ids) and contiguity of all arguments first, then that they all
# live on one GPU.  Size rules (multiples of 256, ranges) are the library's
# own checks, reported as Nvfp4Error.
# ---------------------------------------------------------------------------

_U8, _I32, _F32, _BF16 = torch.uint8, torch.int32, torch.float32, torch.bfloat16
SCALAR = "scalar"   # shape spec: a one-element tensor


def _validate(specs):
    """specs: (name, tensor or None, dtype, shape, required).  ``shape`` is a
    tuple (exact), SCALAR (one element) or ("min", n) (1-D with at least n
    elements).  Returns the device shared by the given tensors (None if none)."""
    given = []
    for name, t, dtype, shape, required in specs:
        if t is None:
            if required:
                raise ValueError(f"{name} is required")
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            hint = " (call .int() on the ids)" if dtype == _I32 and t.dtype == torch.int64 else ""
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}{hint}")
        if shape == SCALAR:
            if t.numel() != 1:
                raise ValueError(f"{name} must hold exactly one element, has {t.numel()}")
        elif isinstance(shape, tuple) and len(shape) == 2 and shape[0] == "min":
            if t.dim() != 1 or t.numel() < shape[1]:
                raise ValueError(f"{name} must be 1-D with at least {shape[1]} elements, "
                                 f"has shape {tuple(t.shape)}")
        elif tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        given.append((name, t))
    dev = None
    for name, t in given:
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}; every tensor must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _one_of(bf16_name, bf16, fp4_names, fp4):
    """Exactly one activation form: the bf16 tensor, or all the NVFP4 parts."""
    if (bf16 is None) == all(v is None for v in fp4):
        raise ValueError(f"pass either {bf16_name} or {' + '.join(fp4_names)}")
    if bf16 is None and any(v is None for v in fp4):
        raise ValueError(f"NVFP4 activations need all of {', '.join(fp4_names)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp4_block_scaled_route_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_status_string.argtypes = [ctypes.c_int]
        L.nvfp4_abi_version.restype = ctypes.c_int
        L.nvfp4_abi_version.argtypes = []
        L.nvfp4_quantize_act_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_quantize_act_workspace_size.argtypes = [_c_i64, _c_i64]
        L.nvfp4_quantize_act.restype = ctypes.c_int
        L.nvfp4_quantize_act.argtypes = [_c_ptr, _c_i64, _c_i64, _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr,
                                         ctypes.c_size_t, _c_ptr]
        L.nvfp4_rmsnorm_quantize_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_rmsnorm_quantize_workspace_size.argtypes = [_c_i64]
        L.nvfp4_rmsnorm_quantize.restype = ctypes.c_int
        L.nvfp4_rmsnorm_quantize.argtypes = [_c_ptr, _c_ptr, ctypes.c_float, _c_i64, _c_i64, _c_ptr, _c_ptr,
                                             ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]
        L.nvfp4_linear_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_linear_workspace_size.argtypes = [_c_i64, _c_i64, _c_i64]
        L.nvfp4_linear.restype = ctypes.c_int
        L.nvfp4_linear.argtypes = [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                   _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]
        L.nvfp4_grouped_linear_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_grouped_linear_workspace_size.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64]
        L.nvfp4_grouped_linear.restype = ctypes.c_int
        L.nvfp4_grouped_linear.argtypes = [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                           _c_i64, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]
        L.nvfp4_moe_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_moe_workspace_size.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int]
        L.nvfp4_moe_grouped.restype = ctypes.c_int
        L.nvfp4_moe_grouped.argtypes = [ctypes.POINTER(MoeArgs), _c_ptr]
        L.nvfp4_moe_grouped_noalloc.restype = ctypes.c_int
        L.nvfp4_moe_grouped_noalloc.argtypes = [ctypes.POINTER(MoeArgs), _c_ptr]
        L.nvfp4_router_prepare.restype = ctypes.c_int
        L.nvfp4_router_prepare.argtypes = [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]
        L.nvfp4_router_workspace_size.restype = ctypes.c_size_t
        L.nvfp4_router_workspace_size.argtypes = [_c_i64, _c_i64, _c_i64]
        L.nvfp4_router_topk.restype = ctypes.c_int
        L.nvfp4_router_topk.argtypes = [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                        _c_ptr, ctypes.c_size_t, _c_ptr]
        if L.nvfp4_abi_version() != ABI_VERSION:
            raise RuntimeError("libnvfp4.so ABI version does not match the binding")
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise Nvfp4Error(status, lib().nvfp4_status_string(status).decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else _c_ptr(t.data_ptr())


def _stream(dev=None):
    return _c_ptr(torch.cuda.current_stream(dev).cuda_stream)


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


# ---------------------------------------------------------------------------


def quantize_act(x: torch.Tensor, gs: Optional[torch.Tensor] = None,
                 out: Optional[Sequence[torch.Tensor]] = None, gs_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """NVFP4-quantize bf16 activations [M, K].  ``gs`` None: the global scale is
    computed on the device (max|x| / 2688) into ``gs_out`` (allocated if not
    given) and returned; otherwise ``gs`` (a 1-element fp32 device tensor) is
    used.  ``workspace``: nvfp4_quantize_act_workspace_size bytes (allocated if
    not given).  Returns (codes [M,K/2] u8, scales [M,K/16] u8, gs [1] fp32)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [M, K]")
    m, k = x.shape
    q, sf = out if out is not None else (None, None)
    dev = _validate([("x", x, _BF16, (m, k), True), ("gs", gs, _F32, SCALAR, False),
                     ("out[0]", q, _U8, (m, k // 2), False), ("out[1]", sf, _U8, (m, k // 16), False),
                     ("gs_out", gs_out, _F32, SCALAR, False), ("workspace", workspace, _U8, ("min", 0), False)])
    if out is None:
        q = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    compute = gs is None
    if compute:
        gsb = gs_out if gs_out is not None else torch.empty(1, dtype=torch.float32, device=dev)
    else:
        gsb = gs
    need = lib().nvfp4_quantize_act_workspace_size(m, k) if compute else 0
    if workspace is not None and workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() if workspace is not None else 0
    _check(lib().nvfp4_quantize_act(_p(x), m, k, _p(gsb), int(compute), _p(q), _p(sf), _p(workspace), wsb,
                                    _stream(dev)))
    return q, sf, gsb


def rmsnorm_quantize(x: torch.Tensor, w: torch.Tensor, eps: float, gs: Optional[torch.Tensor] = None,
                     y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     gs_out: Optional[torch.Tensor] = None):
    """RMSNorm of bf16 rows x [T, K] with weight w [K], quantized to NVFP4.
    Returns (codes [T, K/2], scale bytes [T, K/16], gs [1]); gs is computed
    into ``gs_out`` (allocated if not given) unless given; ``y`` (bf16
    [T, K]) receives the RMSNorm output if given."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, K]")
    t, k = x.shape
    dev = _validate([("x", x, _BF16, (t, k), True), ("w", w, _BF16, (k,), True),
                     ("gs", gs, _F32, SCALAR, False), ("y", y, _BF16, (t, k), False),
                     ("workspace", workspace, _U8, ("min", 1), False), ("gs_out", gs_out, _F32, SCALAR, False)])
    q = torch.empty((t, k // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((t, k // 16), dtype=torch.uint8, device=dev)
    compute = gs is None
    if compute:
        g = gs_out if gs_out is not None else torch.empty(1, dtype=torch.float32, device=dev)
    else:
        g = gs
    if workspace is None:
        workspace = torch.empty(max(16, lib().nvfp4_rmsnorm_quantize_workspace_size(t)), dtype=torch.uint8,
                                device=dev)
    wsb = workspace.numel()
    _check(lib().nvfp4_rmsnorm_quantize(_p(x), _p(w), float(eps), t, k, _p(y), _p(g), int(compute), _p(q), _p(sf),
                                        _p(workspace), wsb, _stream(dev)))
    return q, sf, g


def linear(w: torch.Tensor, w_sf: torch.Tensor, ws2: torch.Tensor, x: Optional[torch.Tensor] = None,
           x_fp4: Optional[torch.Tensor] = None, x_sf: Optional[torch.Tensor] = None,
           gsa: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[M, N] = x @ W^T (bf16 out).  Activations: ``x`` bf16 [M, K], or
    ``x_fp4`` [M, K/2] + ``x_sf`` [M, K/16] + ``gsa`` [1]."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w must be a 2-D tensor [N, K/2]")
    n, k = w.shape[0], w.shape[1] * 2
    _one_of("x", x, ("x_fp4", "x_sf", "gsa"), (x_fp4, x_sf, gsa))
    act = x if x is not None else x_fp4
    if act.dim() != 2:
        raise ValueError("activations must be 2-D [M, K] (NVFP4: [M, K/2])")
    m = act.shape[0]
    dev = _validate([("w", w, _U8, (n, k // 2), True), ("w_sf", w_sf, _U8, (n, k // 16), True),
                     ("ws2", ws2, _F32, SCALAR, True),
                     ("x", x, _BF16, (m, k), False), ("x_fp4", x_fp4, _U8, (m, k // 2), False),
                     ("x_sf", x_sf, _U8, (m, k // 16), False), ("gsa", gsa, _F32, SCALAR, False),
                     ("out", out, _BF16, (m, n), False), ("workspace", workspace, _U8, ("min", 0), False)])
    need = lib().nvfp4_linear_workspace_size(m, n, k)
    if workspace is not None and workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() if workspace is not None else 0
    _check(lib().nvfp4_linear(_p(x), _p(x_fp4), _p(x_sf), _p(gsa), _p(w), _p(w_sf), _p(ws2),
                              m, n, k, _p(y), _p(workspace), wsb, _stream(dev)))
    return y


def grouped_linear_workspace_size(t: int, g: int, n: int, k: int) -> int:
    return int(lib().nvfp4_grouped_linear_workspace_size(t, g, n, k))


def grouped_linear(w: torch.Tensor, w_sf: torch.Tensor, ws2: torch.Tensor, x: Optional[torch.Tensor] = None,
                   x_fp4: Optional[torch.Tensor] = None, x_sf: Optional[torch.Tensor] = None,
                   gsa: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[T, G, N] with y[:, g] = x[:, g] @ W[g]^T (bf16 out).  Weights
    ``w`` [G, N, K/2], ``w_sf`` [G, N, K/16], ``ws2`` [G].  Activations: ``x``
    bf16 [T, G, K], or ``x_fp4`` [T, G, K/2] + ``x_sf`` [T, G, K/16] + ``gsa`` [1]."""
    if not isinstance(w, torch.Tensor) or w.dim() != 3:
        raise ValueError("w must be a 3-D tensor [G, N, K/2]")
    g, n, kh = w.shape
    k = kh * 2
    _one_of("x", x, ("x_fp4", "x_sf", "gsa"), (x_fp4, x_sf, gsa))
    act = x if x is not None else x_fp4
    if act.dim() != 3:
        raise ValueError("activations must be 3-D [T, G, K] (NVFP4: [T, G, K/2])")
    t = act.shape[0]
    dev = _validate([("w", w, _U8, (g, n, k // 2), True), ("w_sf", w_sf, _U8, (g, n, k // 16), True),
                     ("ws2", ws2, _F32, (g,), True),
                     ("x", x, _BF16, (t, g, k), False), ("x_fp4", x_fp4, _U8, (t, g, k // 2), False),
                     ("x_sf", x_sf, _U8, (t, g, k // 16), False), ("gsa", gsa, _F32, SCALAR, False),
                     ("out", out, _BF16, (t, g, n), False), ("workspace", workspace, _U8, ("min", 0), False)])
    need = lib().nvfp4_grouped_linear_workspace_size(t, g, n, k)
    if workspace is not None and workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    y = out if out is not None else torch.empty((t, g, n), dtype=torch.bfloat16, device=dev)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() if workspace is not None else 0
    _check(lib().nvfp4_grouped_linear(_p(x), _p(x_fp4), _p(x_sf), _p(gsa), _p(w), _p(w_sf), _p(ws2),
                                      t, g, n, k, _p(y), _p(workspace), wsb, _stream(dev)))
    return y


def moe_workspace_size(t: int, h: int, i: int, e: int, topk: int, has_shared: bool, h_fp4: bool) -> int:
    return int(lib().nvfp4_moe_workspace_size(t, h, i, e, topk, int(has_shared), int(h_fp4)))


def _moe_specs(topk_ids, topk_w, w1, w1_sf, w1_ws2, w2, w2_sf, w2_ws2, x, x_fp4, x_sf, a1_gs, shared,
               a2_gs, a2_gs_out, workspace, offsets_out, perm_out, out):
    """Shape (T, H, I, E, topk) of a MoE call and the checks of its tensors."""
    for name, t, dim in (("topk_ids", topk_ids, 2), ("w1", w1, 3)):
        if not isinstance(t, torch.Tensor) or t.dim() != dim:
            raise ValueError(f"{name} must be a {dim}-D tensor")
    e, two_i, h_half = w1.shape
    if two_i % 2:
        raise ValueError(f"w1 has {two_i} rows per expert; gate and up need an even count")
    h, i = h_half * 2, two_i // 2
    t, topk = topk_ids.shape
    _one_of("x", x, ("x_fp4", "x_sf", "a1_gs"), (x_fp4, x_sf, a1_gs))
    if shared is not None and len(shared) != 6:
        raise ValueError("shared must be (s1, s1_sf, s1_ws2, s2, s2_sf, s2_ws2)")
    s = shared if shared is not None else (None,) * 6
    has = shared is not None
    specs = [
        ("topk_ids", topk_ids, _I32, (t, topk), True), ("topk_w", topk_w, _F32, (t, topk), True),
        ("w1", w1, _U8, (e, 2 * i, h // 2), True), ("w1_sf", w1_sf, _U8, (e, 2 * i, h // 16), True),
        ("w1_ws2", w1_ws2, _F32, (e,), True),
        ("w2", w2, _U8, (e, h, i // 2), True), ("w2_sf", w2_sf, _U8, (e, h, i // 16), True),
        ("w2_ws2", w2_ws2, _F32, (e,), True),
        ("x", x, _BF16, (t, h), False), ("x_fp4", x_fp4, _U8, (t, h // 2), False),
        ("x_sf", x_sf, _U8, (t, h // 16), False), ("a1_gs", a1_gs, _F32, SCALAR, False),
        ("shared[0] (s1)", s[0], _U8, (2 * i, h // 2), has), ("shared[1] (s1_sf)", s[1], _U8, (2 * i, h // 16), has),
        ("shared[2] (s1_ws2)", s[2], _F32, SCALAR, has),
        ("shared[3] (s2)", s[3], _U8, (h, i // 2), has), ("shared[4] (s2_sf)", s[4], _U8, (h, i // 16), has),
        ("shared[5] (s2_ws2)", s[5], _F32, SCALAR, has),
        ("a2_gs", a2_gs, _F32, SCALAR, False), ("a2_gs_out", a2_gs_out, _F32, SCALAR, False),
        ("workspace", workspace, _U8, ("min", 0), False),
        ("offsets_out", offsets_out, _I32, (e + 2,), False), ("perm_out", perm_out, _I32, (t * topk + t,), False),
        ("out", out, _BF16, (t, h), False),
    ]
    return (t, h, i, e, topk), specs


def moe_grouped(topk_ids: torch.Tensor, topk_w: torch.Tensor,
                w1: torch.Tensor, w1_sf: torch.Tensor, w1_ws2: torch.Tensor,
                w2: torch.Tensor, w2_sf: torch.Tensor, w2_ws2: torch.Tensor,
                x: Optional[torch.Tensor] = None,
                x_fp4: Optional[torch.Tensor] = None, x_sf: Optional[torch.Tensor] = None,
                a1_gs: Optional[torch.Tensor] = None,
                shared: Optional[Sequence[torch.Tensor]] = None,
                a2_gs: Optional[torch.Tensor] = None, a2_gs_out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                offsets_out: Optional[torch.Tensor] = None, perm_out: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stage_events: Optional[Sequence[int]] = None,
                noalloc: bool = False) -> torch.Tensor:
    """One MoE layer (see nvfp4_moe_grouped in include/nvfp4.h).
    ``shared`` = (s1, s1_sf, s1_ws2, s2, s2_sf, s2_ws2) or None.
    ``noalloc``: call nvfp4_moe_grouped_noalloc instead (no workspace; the
    library's static scratch array; ``out`` must then be given too, so that
    nothing is allocated)."""
    (t, h, i, e, topk), specs = _moe_specs(topk_ids, topk_w, w1, w1_sf, w1_ws2, w2, w2_sf, w2_ws2, x, x_fp4, x_sf,
                                           a1_gs, shared, a2_gs, a2_gs_out, workspace, offsets_out, perm_out, out)
    dev = _validate(specs)
    if stage_events is not None and len(stage_events) != 8:
        raise ValueError("stage_events must hold 8 hipEvent_t handles (0 to skip one)")
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc calls take no workspace")
        if out is None:
            raise ValueError("noalloc calls need `out` (nothing is allocated)")
        y = out
    else:
        need = moe_workspace_size(t, h, i, e, topk, shared is not None, a2_gs is not None)
        if workspace is not None and workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
        y = out if out is not None else torch.empty((t, h), dtype=torch.bfloat16, device=dev)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    a = MoeArgs()
    a.T, a.H, a.I, a.E, a.topk = t, h, i, e, topk
    a.x, a.x_fp4, a.x_sf, a.a1_gs = _p(x), _p(x_fp4), _p(x_sf), _p(a1_gs)
    a.a2_gs, a.a2_gs_out = _p(a2_gs), _p(a2_gs_out)
    a.topk_ids, a.topk_w = _p(topk_ids), _p(topk_w)
    a.w1, a.w1_sf, a.w1_ws2 = _p(w1), _p(w1_sf), _p(w1_ws2)
    a.w2, a.w2_sf, a.w2_ws2 = _p(w2), _p(w2_sf), _p(w2_ws2)
    if shared is not None:
        s1, s1_sf, s1_ws2, s2, s2_sf, s2_ws2 = shared
        a.s1, a.s1_sf, a.s1_ws2 = _p(s1), _p(s1_sf), _p(s1_ws2)
        a.s2, a.s2_sf, a.s2_ws2 = _p(s2), _p(s2_sf), _p(s2_ws2)
    a.workspace = _p(workspace)
    a.workspace_bytes = workspace.numel() if workspace is not None else 0
    a.offsets_out, a.perm_out = _p(offsets_out), _p(perm_out)
    a.y = _p(y)
    if stage_events is not None:
        arr = (_c_ptr * len(stage_events))(*[_c_ptr(int(v)) for v in stage_events])
        a.stage_events = ctypes.cast(arr, ctypes.POINTER(_c_ptr))
    fn = lib().nvfp4_moe_grouped_noalloc if noalloc else lib().nvfp4_moe_grouped
    _check(fn(ctypes.byref(a), _stream(dev)))
    return y


def router_prepare(w: torch.Tensor, out: Optional[torch.Tensor] = None,
                   scale_out: Optional[torch.Tensor] = None):
    """FP8-E4M3 round trip of a bf16 router weight [E, H] (see
    nvfp4_router_prepare).  Returns (w_rt bf16 [E, H], scale fp32 [1])."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w must be a 2-D tensor [E, H]")
    e, h = w.shape
    dev = _validate([("w", w, _BF16, (e, h), True), ("out", out, _BF16, (e, h), False),
                     ("scale_out", scale_out, _F32, SCALAR, False)])
    w_rt = out if out is not None else torch.empty_like(w)
    scale = scale_out if scale_out is not None else torch.empty(1, dtype=torch.float32, device=dev)
    _check(lib().nvfp4_router_prepare(_p(w), e, h, _p(scale), _p(w_rt), _stream(dev)))
    return w_rt, scale


def router_workspace_size(t: int, h: int, e: int) -> int:
    return int(lib().nvfp4_router_workspace_size(t, h, e))


def router_topk(x: torch.Tensor, w_rt: torch.Tensor, topk: int, logits: Optional[torch.Tensor] = None,
                ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None):
    """Router logits and top-k softmax (see nvfp4_router_topk).
    Returns (logits fp32 [T, E], topk_ids int32 [T, k], topk_w fp32 [T, k])."""
    for name, v in (("x", x), ("w_rt", w_rt)):
        if not isinstance(v, torch.Tensor) or v.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    t, h = x.shape
    e = w_rt.shape[0]
    dev = _validate([("x", x, _BF16, (t, h), True), ("w_rt", w_rt, _BF16, (e, h), True),
                     ("logits", logits, _F32, (t, e), False), ("ids", ids, _I32, (t, topk), False),
                     ("weights", weights, _F32, (t, topk), False),
                     ("workspace", workspace, _U8, ("min", 0), False)])
    need = router_workspace_size(t, h, e)
    if workspace is not None and workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    logits = logits if logits is not None else torch.empty((t, e), dtype=torch.float32, device=dev)
    ids = ids if ids is not None else torch.empty((t, topk), dtype=torch.int32, device=dev)
    weights = weights if weights is not None else torch.empty((t, topk), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    _check(lib().nvfp4_router_topk(_p(x), _p(w_rt), t, h, e, topk, _p(logits), _p(ids), _p(weights),
                                   _p(workspace), workspace.numel(), _stream(dev)))
    return logits, ids, weights
