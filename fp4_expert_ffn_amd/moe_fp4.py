"""Python binding of the C ABI in ``include/moe_fp4.h`` (ctypes, argument marshalling only).

Every compute step runs in the HIP library ``libmoe_fp4.so``; this module only turns
torch tensors (device memory) and streams into the raw pointers the C functions take,
and raises :class:`MoeFp4Error` on a non-OK status. It fails loudly when the library has
not been built: there is no fallback path.

Functions carry the C names. Tensor arguments may also be given as raw integer device
addresses; ``stream`` is a ``torch.cuda.Stream``, a raw ``hipStream_t`` integer, or None
for torch's current stream.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmoe_fp4.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_BAD_SHAPE = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE = -4
ERR_HIP = -5
ERR_TOO_LARGE = -6
NOALLOC_SCRATCH_BYTES = 16 << 20  # MOE_FP4_NOALLOC_SCRATCH_BYTES

KERNEL_PACK, KERNEL_ROUTER_GEMV, KERNEL_TOPK, KERNEL_GATE_UP, KERNEL_DOWN_COMBINE = range(5)
KERNEL_NAMES = ("pack", "router_gemv", "topk", "gate_up", "down_combine", "route_decode",
                "grouped_sort", "grouped_quant", "grouped_gate_up", "grouped_down", "grouped_combine",
                "norm", "probe_stream", "probe_mfma", "small_m_gate_up", "small_m_down", "fp8_gemv",
                "prefetch")
PROBE_MFMA_CHAINS = 8  # independent block-scaled MFMAs per wavefront per loop iteration


class MoeFp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({strerror(status)})")


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

_SIGNATURES = {
    "moe_fp4_version": (_I, []),
    "moe_fp4_strerror": (ctypes.c_char_p, [_I]),
    "moe_fp4_packed_bytes": (_Z, [_I, _I, _I]),
    "moe_fp4_packed_expert_stride": (_Z, [_I, _I]),
    "moe_fp4_pack": (_I, [_P, _P, _I, _I, _I, _P, _Z, _P]),
    "moe_fp4_route_workspace_bytes": (_Z, [_I, _I]),
    "moe_fp4_route": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "moe_fp4_route_logits": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_fp4_route_status": (_I, [_P, _Z, _P, _P]),
    "moe_fp4_route_reset": (_I, [_P, _Z, _P]),
    "moe_fp4_debug_route_spin_limit": (_I, [ctypes.c_longlong]),
    "moe_fp4_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "moe_fp4_expert_ffn": (_I, [_P, _P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _Z, _P]),
    "moe_fp4_expert_ffn_ex": (_I, [_P, _P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _Z, _I, _P]),
    "moe_fp4_residual_init": (_I, [_P, _P, _I, _I, _P]),
    "moe_fp4_residual_rmsnorm": (_I, [_P, _P, _P, _I, _I, ctypes.c_float, _P]),
    "moe_fp4_route_residual": (_I, [_P, _P, _P, _P, ctypes.c_float, _P, _I, _I, _I, _I, _P, _P, _P,
                                    _Z, _P]),
    "moe_fp4_moe_forward_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "moe_fp4_moe_forward": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _Z, _P]),
    "moe_fp4_moe_forward_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P]),
    "moe_fp4_validate_ids": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_fp4_prefetch_experts": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P]),
    "moe_fp4_debug_dequant": (_I, [_P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_fp4_debug_act_quant_bytes": (ctypes.c_size_t, [_I, _I]),
    "moe_fp4_fp8_packed_bytes": (ctypes.c_size_t, [_I, _I]),
    "moe_fp4_fp8_pack": (_I, [_P, _P, _I, _I, _P, ctypes.c_size_t, _P]),
    "moe_fp4_fp8_linear": (_I, [_P, _I, _P, _I, _I, _P, _P]),
    "moe_fp4_fp8_swiglu": (_I, [_P, _I, _P, _P, _I, _I, _P, _P]),
    "moe_fp4_shared_expert_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "moe_fp4_shared_expert": (_I, [_P, _I, _P, _P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]),
    "moe_fp4_debug_act_quant": (_I, [_P, _I, _I, _I, _P, ctypes.c_size_t, _P, _P]),
    "moe_fp4_debug_stream_read": (_I, [_P, _Z, _P, _P]),
    "moe_fp4_debug_mfma_loop": (_I, [_I, _I, _I, _P, _P]),
    "moe_fp4_timing_enable": (_I, [_I]),
    "moe_fp4_timing_reset": (_I, []),
    "moe_fp4_timing_read": (_I, [_I, ctypes.POINTER(_I), ctypes.POINTER(ctypes.c_double)]),
}


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m fp4_expert_ffn_amd.build` "
                "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_names() -> Tuple[str, ...]:
    return tuple(_SIGNATURES)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != OK:
        raise MoeFp4Error(status, where)


def strerror(status: int) -> str:
    return lib().moe_fp4_strerror(status).decode()


def moe_fp4_version() -> int:
    return lib().moe_fp4_version()


def moe_fp4_packed_bytes(n_experts: int, hidden: int, inter: int) -> int:
    return lib().moe_fp4_packed_bytes(n_experts, hidden, inter)


def moe_fp4_packed_expert_stride(hidden: int, inter: int) -> int:
    return lib().moe_fp4_packed_expert_stride(hidden, inter)


def moe_fp4_pack(codes, scales, n_experts: int, hidden: int, inter: int, packed,
                 packed_bytes: Optional[int] = None, stream=None) -> None:
    if packed_bytes is None:
        packed_bytes = packed.numel() * packed.element_size()
    _check(lib().moe_fp4_pack(_ptr(codes), _ptr(scales), n_experts, hidden, inter, _ptr(packed),
                              packed_bytes, _stream(stream)), "moe_fp4_pack")


def moe_fp4_route_workspace_bytes(T: int, n_experts: int) -> int:
    return lib().moe_fp4_route_workspace_bytes(T, n_experts)


def moe_fp4_route(x, w_router, T: int, hidden: int, n_experts: int, k: int, topk_ids, topk_w,
                  workspace, workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_fp4_route(_ptr(x), _ptr(w_router), T, hidden, n_experts, k, _ptr(topk_ids),
                               _ptr(topk_w), _ptr(workspace), workspace_bytes, _stream(stream)),
           "moe_fp4_route")


def _nbytes(t, given: Optional[int]) -> int:
    return t.numel() * t.element_size() if given is None else given


def moe_fp4_route_status(workspace, status, workspace_bytes: Optional[int] = None,
                         stream=None) -> None:
    _check(lib().moe_fp4_route_status(_ptr(workspace), _nbytes(workspace, workspace_bytes),
                                      _ptr(status), _stream(stream)), "moe_fp4_route_status")


def moe_fp4_route_reset(workspace, workspace_bytes: Optional[int] = None, stream=None) -> None:
    _check(lib().moe_fp4_route_reset(_ptr(workspace), _nbytes(workspace, workspace_bytes),
                                     _stream(stream)), "moe_fp4_route_reset")


def moe_fp4_debug_route_spin_limit(polls: int) -> None:
    _check(lib().moe_fp4_debug_route_spin_limit(polls), "moe_fp4_debug_route_spin_limit")


def moe_fp4_route_logits(logits, T: int, n_experts: int, k: int, topk_ids, topk_w,
                         stream=None) -> None:
    _check(lib().moe_fp4_route_logits(_ptr(logits), T, n_experts, k, _ptr(topk_ids), _ptr(topk_w),
                                      _stream(stream)), "moe_fp4_route_logits")


def moe_fp4_workspace_bytes(T: int, k: int, n_experts: int, hidden: int, inter: int) -> int:
    return lib().moe_fp4_workspace_bytes(T, k, n_experts, hidden, inter)


def moe_fp4_expert_ffn(x, topk_ids, topk_w, T: int, k: int, packed, n_experts: int, hidden: int,
                       inter: int, y, workspace, workspace_bytes: Optional[int] = None,
                       stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_fp4_expert_ffn(_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, k, _ptr(packed),
                                    n_experts, hidden, inter, _ptr(y), _ptr(workspace),
                                    workspace_bytes, _stream(stream)), "moe_fp4_expert_ffn")


PATH_AUTO, PATH_DECODE, PATH_GROUPED, PATH_SMALL_M, PATH_GROUPED_FP8 = 0, 1, 2, 3, 4


def moe_fp4_residual_init(x, residual, T: int, hidden: int, stream=None) -> None:
    _check(lib().moe_fp4_residual_init(_ptr(x), _ptr(residual), T, hidden, _stream(stream)),
           "moe_fp4_residual_init")


def moe_fp4_residual_rmsnorm(residual, y, x_out, T: int, hidden: int, eps: float = 1e-6,
                             stream=None) -> None:
    _check(lib().moe_fp4_residual_rmsnorm(_ptr(residual), _ptr(y), _ptr(x_out), T, hidden, eps,
                                          _stream(stream)), "moe_fp4_residual_rmsnorm")


def moe_fp4_route_residual(residual_in, y_prev, residual_out, x_out, eps: float, w_router, T: int,
                           hidden: int, n_experts: int, k: int, topk_ids, topk_w, workspace,
                           stream=None) -> None:
    _check(lib().moe_fp4_route_residual(_ptr(residual_in), _ptr(y_prev), _ptr(residual_out),
                                        _ptr(x_out), eps, _ptr(w_router), T, hidden, n_experts, k,
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "moe_fp4_route_residual")


def moe_fp4_expert_ffn_ex(x, topk_ids, topk_w, T: int, k: int, packed, n_experts: int,
                          hidden: int, inter: int, y, workspace, path: int,
                          workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_fp4_expert_ffn_ex(_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, k, _ptr(packed),
                                       n_experts, hidden, inter, _ptr(y), _ptr(workspace),
                                       workspace_bytes, path, _stream(stream)),
           "moe_fp4_expert_ffn_ex")


def moe_fp4_moe_forward_workspace_bytes(T: int, k: int, n_experts: int, hidden: int,
                                        inter: int) -> int:
    return lib().moe_fp4_moe_forward_workspace_bytes(T, k, n_experts, hidden, inter)


def moe_fp4_moe_forward(x, w_router, T: int, hidden: int, n_experts: int, k: int, packed,
                        inter: int, topk_ids, topk_w, y, workspace,
                        workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_fp4_moe_forward(_ptr(x), _ptr(w_router), T, hidden, n_experts, k, _ptr(packed),
                                     inter, _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(workspace),
                                     workspace_bytes, _stream(stream)), "moe_fp4_moe_forward")


def moe_fp4_moe_forward_noalloc(x, w_router, T: int, hidden: int, n_experts: int, k: int, packed,
                                inter: int, topk_ids, topk_w, y, stream=None) -> None:
    _check(lib().moe_fp4_moe_forward_noalloc(_ptr(x), _ptr(w_router), T, hidden, n_experts, k,
                                             _ptr(packed), inter, _ptr(topk_ids), _ptr(topk_w),
                                             _ptr(y), _stream(stream)), "moe_fp4_moe_forward_noalloc")


def moe_fp4_prefetch_experts(ids, n_ids: int, packed, n_experts: int, hidden: int, inter: int,
                             matrices: int, sink, stream=None) -> None:
    _check(lib().moe_fp4_prefetch_experts(_ptr(ids), n_ids, _ptr(packed), n_experts, hidden, inter,
                                          matrices, _ptr(sink), _stream(stream)),
           "moe_fp4_prefetch_experts")


def moe_fp4_validate_ids(topk_ids, T: int, k: int, n_experts: int, bad_count, stream=None) -> None:
    _check(lib().moe_fp4_validate_ids(_ptr(topk_ids), T, k, n_experts, _ptr(bad_count),
                                      _stream(stream)), "moe_fp4_validate_ids")


def moe_fp4_fp8_packed_bytes(rows: int, cols: int) -> int:
    return lib().moe_fp4_fp8_packed_bytes(rows, cols)


def moe_fp4_fp8_pack(codes, scale_inv, rows: int, cols: int, packed, packed_bytes: int,
                     stream=None) -> None:
    _check(lib().moe_fp4_fp8_pack(_ptr(codes), _ptr(scale_inv), rows, cols, _ptr(packed),
                                  packed_bytes, _stream(stream)), "moe_fp4_fp8_pack")


def moe_fp4_fp8_linear(x, T: int, packed, rows: int, cols: int, y, stream=None) -> None:
    _check(lib().moe_fp4_fp8_linear(_ptr(x), T, _ptr(packed), rows, cols, _ptr(y), _stream(stream)),
           "moe_fp4_fp8_linear")


def moe_fp4_fp8_swiglu(x, T: int, gate, up, inter: int, hidden: int, h, stream=None) -> None:
    _check(lib().moe_fp4_fp8_swiglu(_ptr(x), T, _ptr(gate), _ptr(up), inter, hidden, _ptr(h),
                                    _stream(stream)), "moe_fp4_fp8_swiglu")


def moe_fp4_shared_expert_workspace_bytes(T: int, inter: int) -> int:
    return lib().moe_fp4_shared_expert_workspace_bytes(T, inter)


def moe_fp4_shared_expert(x, T: int, gate, up, down, hidden: int, inter: int, y, workspace,
                          workspace_bytes: int, stream=None) -> None:
    _check(lib().moe_fp4_shared_expert(_ptr(x), T, _ptr(gate), _ptr(up), _ptr(down), hidden, inter,
                                       _ptr(y), _ptr(workspace), workspace_bytes, _stream(stream)),
           "moe_fp4_shared_expert")


def moe_fp4_debug_act_quant_bytes(T: int, hidden: int) -> int:
    return lib().moe_fp4_debug_act_quant_bytes(T, hidden)


def moe_fp4_debug_act_quant(x, T: int, hidden: int, terms: int, workspace,
                            workspace_bytes: int, out, stream=None) -> None:
    _check(lib().moe_fp4_debug_act_quant(_ptr(x), T, hidden, terms, _ptr(workspace),
                                         workspace_bytes, _ptr(out), _stream(stream)),
           "moe_fp4_debug_act_quant")


def moe_fp4_debug_dequant(packed, n_experts: int, hidden: int, inter: int, expert: int,
                          matrix: int, out, stream=None) -> None:
    _check(lib().moe_fp4_debug_dequant(_ptr(packed), n_experts, hidden, inter, expert, matrix,
                                       _ptr(out), _stream(stream)), "moe_fp4_debug_dequant")


def moe_fp4_debug_stream_read(src, nbytes: int, sink, stream=None) -> None:
    _check(lib().moe_fp4_debug_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "moe_fp4_debug_stream_read")


def moe_fp4_debug_mfma_loop(fmt_a: int, n_workgroups: int, iters: int, sink, stream=None) -> None:
    _check(lib().moe_fp4_debug_mfma_loop(fmt_a, n_workgroups, iters, _ptr(sink), _stream(stream)),
           "moe_fp4_debug_mfma_loop")


def moe_fp4_timing_enable(enable: bool) -> None:
    _check(lib().moe_fp4_timing_enable(1 if enable else 0), "moe_fp4_timing_enable")


def moe_fp4_timing_reset() -> None:
    _check(lib().moe_fp4_timing_reset(), "moe_fp4_timing_reset")


def moe_fp4_timing_read(kind: int) -> Tuple[int, float]:
    n = _I(0)
    ms = ctypes.c_double(0.0)
    _check(lib().moe_fp4_timing_read(kind, ctypes.byref(n), ctypes.byref(ms)), "moe_fp4_timing_read")
    return n.value, ms.value
