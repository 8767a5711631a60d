"""GPU parity of the dense FP8 calls (the shared expert and the dense projections) against
the oracle's FP8 section: E4M3 codes with one fp32 multiplier per 128 x 128 block, converted
to bf16 matrix-core operands in registers. Products are exact, sums are fp32, outputs bf16,
so the bar is the FFN one (normwise 2e-2 and cosine 0.9995 per token); a one-hot input
checks the element order of every column exactly up to the output rounding."""

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import moe_inputs as S

from tests.gpu_helpers import check_ffn, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import moe_fp4 as C
    C.lib()
    return C


def _pack(C, codes, scales):
    rows, cols = codes.shape
    dev = torch.device("cuda:0")
    c = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).to(dev)
    nbytes = C.moe_fp4_fp8_packed_bytes(rows, cols)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    C.moe_fp4_fp8_pack(c, s, rows, cols, packed, nbytes)
    return packed


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0")


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols,T", [(256, 512, 1), (2880, 4096, 1), (4096, 2880, 3), (96, 7168, 5),
                                         (64, 32, 2), (160, 16384, 1), (1024, 1024, 9)])
def test_fp8_linear_matches_oracle(C, rows, cols, T):
    """y = x W^T: ragged last 128-element chunk (K 2880, 96 -> blocks past K), ragged last
    128-row block (2880, 160, 96 rows), the largest K (16384: one token per workgroup), and
    token counts that leave a partial group of four."""
    codes, scales = S.fp8_matrix(rows, cols, seed=rows + cols)
    packed = _pack(C, codes, scales)
    x_bits = O.f64_to_bf16_bits(np.random.default_rng(rows * 3 + T).standard_normal((T, cols)))
    y = torch.empty((T, rows), dtype=torch.int16, device="cuda:0")
    C.moe_fp4_fp8_linear(_bf16(x_bits), T, packed, rows, cols, y)
    torch.cuda.synchronize()
    ref = O.dense_fp8(x_bits, codes, scales)
    err, cos = check_ffn(_bits(y), ref, f"fp8 linear {rows}x{cols} T={T}")
    log(f"fp8 linear {rows}x{cols} T={T}: normwise {err:.2e} cosine {cos:.7f}")


@pytest.mark.parametrize("rows,cols", [(256, 512), (96, 2880)])
def test_fp8_linear_one_hot_columns(C, rows, cols):
    """One-hot rows of x pick single columns of W: every output equals its weight times the
    block multiplier, rounded once to bf16 (the fp32 product of an E4M3 value and an fp32
    multiplier may round first, so one bf16 unit of difference is allowed). Any mistake in
    the byte order of the packed words or the K order of the operands picks other columns."""
    codes, scales = S.fp8_matrix(rows, cols, seed=11)
    packed = _pack(C, codes, scales)
    ks = np.array([0, 1, 7, 8, 15, 16, 31, 32, 100, 127, 128, cols - 33, cols - 1])
    x = np.zeros((ks.size, cols))
    x[np.arange(ks.size), ks] = 1.0
    x_bits = O.f64_to_bf16_bits(x)
    y = torch.empty((ks.size, rows), dtype=torch.int16, device="cuda:0")
    C.moe_fp4_fp8_linear(_bf16(x_bits), ks.size, packed, rows, cols, y)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(_bits(y))
    ref = O.dequant_fp8(codes, scales)[:, ks].T
    tol = np.abs(ref) * 2.0 ** -7  # one bf16 unit of the value: zero weights give exact zeros
    bad = np.argwhere(np.abs(got - ref) > tol)
    assert bad.size == 0, f"{bad.shape[0]} outputs off, first {bad[:4].tolist()}"


@pytest.mark.parametrize("hidden,inter,T", [(4096, 2880, 1), (512, 256, 6), (7168, 2048, 2)])
def test_shared_expert_matches_oracle(C, hidden, inter, T):
    """The FP8 SwiGLU shared expert (two launches, h bf16 in the workspace) against the
    oracle's fp64 FFN."""
    gate = S.fp8_matrix(inter, hidden, seed=1)
    up = S.fp8_matrix(inter, hidden, seed=2)
    down = S.fp8_matrix(hidden, inter, seed=3)
    pg, pu, pd = (_pack(C, *m) for m in (gate, up, down))
    x_bits = O.f64_to_bf16_bits(np.random.default_rng(hidden + T).standard_normal((T, hidden)) * 0.5)
    y = torch.empty((T, hidden), dtype=torch.int16, device="cuda:0")
    wsb = C.moe_fp4_shared_expert_workspace_bytes(T, inter)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    C.moe_fp4_shared_expert(_bf16(x_bits), T, pg, pu, pd, hidden, inter, y, ws, wsb)
    torch.cuda.synchronize()
    ref = O.shared_expert_fp8(x_bits, gate, up, down)
    err, cos = check_ffn(_bits(y), ref, f"shared expert H{hidden} I{inter} T={T}")
    log(f"shared expert H{hidden} I{inter} T={T}: normwise {err:.2e} cosine {cos:.7f}")
    # the first launch alone: h against silu(g) * u
    h = torch.empty((T, inter), dtype=torch.int16, device="cuda:0")
    C.moe_fp4_fp8_swiglu(_bf16(x_bits), T, pg, pu, inter, hidden, h)
    torch.cuda.synchronize()
    x = O.bf16_to_f64(x_bits)
    h_ref = O.silu(x @ O.dequant_fp8(*gate).T) * (x @ O.dequant_fp8(*up).T)
    check_ffn(_bits(h), h_ref, "fp8 swiglu h")


def test_fp8_repeat_determinism(C):
    codes, scales = S.fp8_matrix(2880, 4096, seed=5)
    packed = _pack(C, codes, scales)
    x_bits = O.f64_to_bf16_bits(np.random.default_rng(5).standard_normal((7, 4096)))
    outs = []
    for _ in range(4):
        y = torch.empty((7, 2880), dtype=torch.int16, device="cuda:0")
        C.moe_fp4_fp8_linear(_bf16(x_bits), 7, packed, 2880, 4096, y)
        torch.cuda.synchronize()
        outs.append(_bits(y))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
