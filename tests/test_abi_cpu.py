"""CPU-only checks of the C ABI: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any HIP call (fake, never
dereferenced pointer values are used, so no GPU is needed)."""

import ctypes
import os
import re

import pytest

from fp4_expert_ffn_amd import moe_fp4 as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp4.h")

A = 0x10000  # an aligned fake device address (never dereferenced)
MIS = 0x10008  # misaligned for 16-byte pointers
MIS4 = 0x10002  # misaligned for 4-byte pointers (ids, weights, fp32 logits)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_fp4_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    try:
        return C.lib()
    except RuntimeError as e:  # not built yet
        pytest.fail(str(e))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(C.exported_names())


def test_status_strings_and_version(L):
    """moe_fp4_strerror: its own text for every status the header defines, "unknown status"
    for any other value."""
    assert C.moe_fp4_version() >= 100
    codes = (C.OK, C.ERR_INVALID_ARG, C.ERR_BAD_SHAPE, C.ERR_MISALIGNED, C.ERR_WORKSPACE,
             C.ERR_HIP, C.ERR_TOO_LARGE)
    texts = [C.strerror(st) for st in codes]
    assert all(texts) and "unknown status" not in texts
    assert len(set(texts)) == len(codes)
    for st in (-7, -99, 1, 2**31 - 1):
        assert C.strerror(st) == "unknown status"


def test_packed_sizes():
    stride = C.moe_fp4_packed_expert_stride(4096, 2880)
    assert stride == 18_800_640 and stride % 256 == 0
    assert C.moe_fp4_packed_bytes(384, 4096, 2880) == 384 * stride
    assert C.moe_fp4_packed_expert_stride(256, 128) == 3 * 256 * 128 // 2 + 3 * 256 * 128 // 32
    assert C.moe_fp4_packed_expert_stride(100, 128) == 0
    assert C.moe_fp4_packed_bytes(0, 4096, 2880) == 0


def test_workspace_sizes():
    assert C.moe_fp4_workspace_bytes(1, 6, 384, 4096, 2880) >= 6 * 2880 * 2
    assert C.moe_fp4_workspace_bytes(8192, 6, 384, 4096, 2880) >= 8192 * 6 * 2880 * 2
    assert C.moe_fp4_route_workspace_bytes(1, 384) >= 384 * 8
    assert C.moe_fp4_workspace_bytes(1, 6, 384, 4010, 2880) == 0  # hidden not a multiple of 32


def ffn(L, x=A, ids=A, w=A, T=1, k=6, packed=A, E=384, H=4096, I=2880, y=A, ws=A, wsb=1 << 20):
    return L.moe_fp4_expert_ffn(x, ids, w, T, k, packed, E, H, I, y, ws, wsb, None)


def test_expert_ffn_argument_checks(L):
    assert ffn(L, x=None) == C.ERR_INVALID_ARG
    assert ffn(L, y=None) == C.ERR_INVALID_ARG
    assert ffn(L, ws=None) == C.ERR_INVALID_ARG
    assert ffn(L, T=-1) == C.ERR_INVALID_ARG
    assert ffn(L, k=0) == C.ERR_INVALID_ARG
    assert ffn(L, k=9) == C.ERR_INVALID_ARG
    assert ffn(L, k=4, E=3) == C.ERR_INVALID_ARG
    assert ffn(L, H=4010) == C.ERR_BAD_SHAPE
    assert ffn(L, I=2881) == C.ERR_BAD_SHAPE
    assert ffn(L, H=16384 + 32) == C.ERR_BAD_SHAPE
    # k * inter > 32768 does not fit the decode path's LDS: the automatic choice takes the
    # grouped path (the argument checks pass and the workspace check fires)
    assert ffn(L, k=8, I=8192, wsb=8) == C.ERR_WORKSPACE
    assert ffn(L, x=MIS) == C.ERR_MISALIGNED
    assert ffn(L, packed=MIS) == C.ERR_MISALIGNED
    assert ffn(L, ids=MIS4) == C.ERR_MISALIGNED
    assert ffn(L, w=MIS4) == C.ERR_MISALIGNED
    assert ffn(L, ids=A + 4, w=A + 12, wsb=8) == C.ERR_WORKSPACE
    assert ffn(L, wsb=100) == C.ERR_WORKSPACE
    # T = 0 is a no-op: OK without touching any pointer
    assert ffn(L, T=0, wsb=0) == C.OK


def test_expert_ffn_path_checks(L):
    def ffn_ex(path, k=6, E=384, I=2880, wsb=1 << 40, T=1):
        return L.moe_fp4_expert_ffn_ex(A, A, A, T, k, A, E, 4096, I, A, A, wsb, path, None)
    assert ffn_ex(C.PATH_DECODE, k=8, I=8192) == C.ERR_BAD_SHAPE       # decode LDS limit
    assert ffn_ex(C.PATH_GROUPED, E=4096, k=6) == C.ERR_BAD_SHAPE      # sort table limit
    assert ffn_ex(7) == C.ERR_INVALID_ARG
    assert ffn_ex(-1) == C.ERR_INVALID_ARG
    for path in (C.PATH_AUTO, C.PATH_DECODE, C.PATH_GROUPED):
        assert ffn_ex(path, wsb=8) == C.ERR_WORKSPACE
        assert ffn_ex(path, T=0, wsb=0) == C.OK
    # the workspace covers the grouped path: sort tables, MX x and h, fp32 per-pair y
    need = C.moe_fp4_workspace_bytes(64, 6, 384, 4096, 2880)
    assert need >= 64 * 6 * (4096 * 4 + 2 * 2944) + 64 * 2 * 4096
    assert C.moe_fp4_workspace_bytes(0, 6, 384, 4096, 2880) == 0


def test_route_argument_checks(L):
    def route(x=A, wr=A, T=1, H=4096, E=384, k=6, ids=A, w=A, ws=A, wsb=1 << 20):
        return L.moe_fp4_route(x, wr, T, H, E, k, ids, w, ws, wsb, None)
    assert route(wr=None) == C.ERR_INVALID_ARG
    assert route(k=0) == C.ERR_INVALID_ARG
    assert route(k=7, E=6) == C.ERR_INVALID_ARG
    assert route(E=4096) == C.ERR_BAD_SHAPE
    assert route(H=31) == C.ERR_BAD_SHAPE
    assert route(x=MIS) == C.ERR_MISALIGNED
    assert route(ids=MIS4) == C.ERR_MISALIGNED
    assert route(w=MIS4) == C.ERR_MISALIGNED
    # ids / weights only need 4-byte alignment: the check passes and the workspace one fires
    assert route(ids=A + 4, w=A + 8, wsb=8) == C.ERR_WORKSPACE
    assert route(wsb=8) == C.ERR_WORKSPACE
    assert route(T=0) == C.OK
    assert L.moe_fp4_route_logits(A, 0, 384, 6, A, A, None) == C.OK
    assert L.moe_fp4_route_logits(None, 1, 384, 6, A, A, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_route_logits(A, 1, 384, 9, A, A, None) == C.ERR_INVALID_ARG


def test_pack_and_debug_argument_checks(L):
    assert L.moe_fp4_pack(None, A, 1, 256, 128, A, 1 << 30, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_pack(A, A, 0, 256, 128, A, 1 << 30, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_pack(A, A, 1, 250, 128, A, 1 << 30, None) == C.ERR_BAD_SHAPE
    assert L.moe_fp4_pack(A, MIS, 1, 256, 128, A, 1 << 30, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_pack(A, A, 2, 256, 128, A, 1000, None) == C.ERR_WORKSPACE
    assert L.moe_fp4_debug_dequant(A, 2, 256, 128, 2, 0, A, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_debug_dequant(A, 2, 256, 128, 0, 3, A, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_validate_ids(None, 1, 6, 384, A, None) == C.ERR_INVALID_ARG


def test_act_quant_argument_checks(L):
    """Workspace size of the activation-quantiser helper (two terms and two scale rows per
    token, hidden padded to 128) and its argument checks, none of which launches work."""
    assert L.moe_fp4_debug_act_quant_bytes(3, 4096) == 2 * 3 * 4096 + 2 * 3 * 128
    assert L.moe_fp4_debug_act_quant_bytes(1, 96) == 2 * 128 + 2 * 4
    assert L.moe_fp4_debug_act_quant_bytes(1, 100) == 0
    assert L.moe_fp4_debug_act_quant_bytes(-1, 128) == 0
    big = 1 << 30
    q = L.moe_fp4_debug_act_quant
    assert q(None, 1, 256, 2, A, big, A, None) == C.ERR_INVALID_ARG
    assert q(A, -1, 256, 2, A, big, A, None) == C.ERR_INVALID_ARG
    assert q(A, 1, 256, 0, A, big, A, None) == C.ERR_INVALID_ARG
    assert q(A, 1, 256, 3, A, big, A, None) == C.ERR_INVALID_ARG
    assert q(A, 1, 250, 1, A, big, A, None) == C.ERR_BAD_SHAPE
    assert q(MIS, 1, 256, 1, A, big, A, None) == C.ERR_MISALIGNED
    assert q(A, 1, 256, 1, A, 100, A, None) == C.ERR_WORKSPACE
    assert q(A, 0, 256, 2, A, 0, A, None) == C.OK


def test_fp8_entry_points_argument_checks(L):
    """Packed sizes of the FP8 matrices and the argument checks of the dense FP8 calls, none
    of which launches work."""
    # 2880 x 4096: 180 tiles x 32 chunks x 2 KB of codes, then 180 x 32 fp32 multipliers
    assert L.moe_fp4_fp8_packed_bytes(2880, 4096) == 180 * 32 * 2048 + (180 * 32 * 4 + 255) // 256 * 256
    # 4096 x 2880: K = 2880 is 22.5 chunks, padded to 23
    assert L.moe_fp4_fp8_packed_bytes(4096, 2880) == 256 * 23 * 2048 + (256 * 23 * 4 + 255) // 256 * 256
    assert L.moe_fp4_fp8_packed_bytes(100, 128) == 0
    assert L.moe_fp4_fp8_packed_bytes(128, 32768) == 0
    big = 1 << 30
    assert L.moe_fp4_fp8_pack(None, A, 128, 128, A, big, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_fp8_pack(A, A, 130, 128, A, big, None) == C.ERR_BAD_SHAPE
    assert L.moe_fp4_fp8_pack(MIS, A, 128, 128, A, big, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_fp8_pack(A, MIS4, 128, 128, A, big, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_fp8_pack(A, A, 128, 128, A, 1000, None) == C.ERR_WORKSPACE
    assert L.moe_fp4_fp8_linear(A, -1, A, 128, 128, A, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_fp8_linear(A, 1, A, 128, 100, A, None) == C.ERR_BAD_SHAPE
    assert L.moe_fp4_fp8_linear(A, 1, MIS, 128, 128, A, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_fp8_linear(A, 0, A, 128, 128, A, None) == C.OK
    assert L.moe_fp4_fp8_swiglu(A, 1, None, A, 128, 128, A, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_fp8_swiglu(A, 0, A, A, 128, 128, A, None) == C.OK
    assert L.moe_fp4_shared_expert_workspace_bytes(3, 2880) == (3 * 2880 * 2 + 255) // 256 * 256
    se = L.moe_fp4_shared_expert
    assert se(A, 3, A, A, A, 4096, 2880, A, A, 100, None) == C.ERR_WORKSPACE
    assert se(A, 3, A, A, A, 4096, 2888, A, A, big, None) == C.ERR_BAD_SHAPE
    assert se(A, 3, A, A, A, 4096, 2880, A, MIS, big, None) == C.ERR_MISALIGNED
    assert se(A, 0, A, A, A, 4096, 2880, A, A, 0, None) == C.OK


def test_timing_read_without_records(L):
    C.moe_fp4_timing_reset()
    assert C.moe_fp4_timing_read(C.KERNEL_GATE_UP) == (0, 0.0)
    with pytest.raises(C.MoeFp4Error):
        C.moe_fp4_timing_read(99)


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        C.moe_fp4_expert_ffn(torch.zeros(4), A, A, 1, 6, A, 384, 4096, 2880, A, A, 1 << 20, stream=0)


def test_residual_helpers_argument_checks(L):
    assert L.moe_fp4_residual_init(None, A, 1, 64, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_residual_init(A, A, -1, 64, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_residual_init(A, A + 2, 1, 64, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_residual_init(A, A, 0, 64, None) == C.OK
    f = L.moe_fp4_residual_rmsnorm
    assert f(A, None, A, 1, 64, 1e-6, None) == C.ERR_INVALID_ARG
    assert f(A, A, A, 1, 0, 1e-6, None) == C.ERR_INVALID_ARG
    assert f(A, A, A, 1, 64, -1.0, None) == C.ERR_INVALID_ARG
    assert f(A + 4, A, A, 1, 64, 1e-6, None) == C.ERR_MISALIGNED
    assert f(A, A + 2, A, 1, 64, 1e-6, None) == C.ERR_MISALIGNED
    assert f(A, A, A, 1, 60, 1e-6, None) == C.ERR_BAD_SHAPE
    assert f(A, A, A, 1, 16384 + 8, 1e-6, None) == C.ERR_BAD_SHAPE
    assert f(A, A, A, 0, 64, 1e-6, None) == C.OK


def test_probe_helpers_argument_checks(L):
    f = L.moe_fp4_debug_stream_read
    assert f(None, 1024, A, None) == C.ERR_INVALID_ARG
    assert f(A, 1024, None, None) == C.ERR_INVALID_ARG
    assert f(A, 0, A, None) == C.ERR_INVALID_ARG
    assert f(A, 1000, A, None) == C.ERR_INVALID_ARG
    assert f(MIS, 1024, A, None) == C.ERR_MISALIGNED
    assert f(A, 1024, MIS4, None) == C.ERR_MISALIGNED
    g = L.moe_fp4_debug_mfma_loop
    assert g(4, 1, 1, None, None) == C.ERR_INVALID_ARG
    assert g(2, 1, 1, A, None) == C.ERR_INVALID_ARG
    assert g(4, 0, 1, A, None) == C.ERR_INVALID_ARG
    assert g(0, 1, 0, A, None) == C.ERR_INVALID_ARG
    assert g(0, 1, (1 << 20) + 1, A, None) == C.ERR_INVALID_ARG
    assert g(4, 1, 1, MIS4, None) == C.ERR_MISALIGNED
    assert C.PROBE_MFMA_CHAINS == 8
    kinds = int(re.search(r"#define MOE_FP4_KERNEL_KINDS (\d+)", open(HEADER).read()).group(1))
    assert len(C.KERNEL_NAMES) == kinds


def test_route_residual_argument_checks(L):
    f = L.moe_fp4_route_residual
    B = 0x20000  # a second aligned fake address, far from A
    big = 1 << 20
    Y, XO = 0x30000, 0x40000  # y_prev and x_out: distinct from every other buffer
    args = lambda **kw: dict(dict(ri=A, y=Y, ro=B, xo=XO, eps=1e-6, wr=A, T=1, H=64, E=8, k=2,
                                  ids=A, w=A, ws=A, wsb=big), **kw)
    def call(**kw):
        a = args(**kw)
        return f(a["ri"], a["y"], a["ro"], a["xo"], a["eps"], a["wr"], a["T"], a["H"], a["E"],
                 a["k"], a["ids"], a["w"], a["ws"], a["wsb"], None)
    assert call(T=0) == C.OK
    assert call(ri=None) == C.ERR_INVALID_ARG
    assert call(y=None) == C.ERR_INVALID_ARG
    assert call(eps=-1.0) == C.ERR_INVALID_ARG
    assert call(eps=float("nan")) == C.ERR_INVALID_ARG
    assert call(ro=A) == C.ERR_INVALID_ARG  # residual_in and residual_out overlap (checked before any launch)
    assert call(ro=A + 64 * 4 - 16, T=1) == C.ERR_INVALID_ARG
    # no output may overlap an input or the other output (x_out in y_prev's buffer is the
    # natural reuse, and a race at T == 1)
    assert call(xo=Y) == C.ERR_INVALID_ARG
    assert call(xo=Y + 64 * 2 - 16) == C.ERR_INVALID_ARG
    assert call(xo=A + 16) == C.ERR_INVALID_ARG             # x_out inside residual_in
    assert call(ro=Y - 64 * 4 + 16) == C.ERR_INVALID_ARG    # residual_out over y_prev
    assert call(xo=B + 64) == C.ERR_INVALID_ARG             # x_out inside residual_out
    assert call(k=9) == C.ERR_INVALID_ARG
    assert call(H=100) == C.ERR_BAD_SHAPE
    assert call(ri=MIS) == C.ERR_MISALIGNED
    assert call(ids=MIS4) == C.ERR_MISALIGNED
    assert call(wsb=16) == C.ERR_WORKSPACE


def test_route_status_reset_argument_checks(L):
    assert L.moe_fp4_route_status(None, 1 << 14, A, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_route_status(A, 1 << 14, None, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_route_status(MIS, 1 << 14, A, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_route_status(A, 1 << 14, MIS4, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_route_status(A, (1 << 14) - 1, A, None) == C.ERR_WORKSPACE
    assert L.moe_fp4_route_reset(None, 1 << 14, None) == C.ERR_INVALID_ARG
    assert L.moe_fp4_route_reset(MIS, 1 << 14, None) == C.ERR_MISALIGNED
    assert L.moe_fp4_route_reset(A, 100, None) == C.ERR_WORKSPACE
    assert L.moe_fp4_debug_route_spin_limit(-1) == C.OK  # the default bound


def test_prefetch_argument_checks(L):
    f = L.moe_fp4_prefetch_experts
    assert f(A, 0, A, 384, 4096, 2880, 3, A, None) == C.OK          # no ids: nothing enqueued
    assert f(None, 2, A, 384, 4096, 2880, 3, A, None) == C.ERR_INVALID_ARG
    assert f(A, -1, A, 384, 4096, 2880, 3, A, None) == C.ERR_INVALID_ARG
    assert f(A, 2, A, 384, 4096, 2880, 0, A, None) == C.ERR_INVALID_ARG
    assert f(A, 2, A, 384, 4096, 2880, 8, A, None) == C.ERR_INVALID_ARG
    assert f(A, 2, A, 384, 4100, 2880, 3, A, None) == C.ERR_BAD_SHAPE   # 4100 % 32 != 0
    assert f(MIS4, 2, A, 384, 4096, 2880, 3, A, None) == C.ERR_MISALIGNED
    assert f(A, 2, MIS, 384, 4096, 2880, 3, A, None) == C.ERR_MISALIGNED
