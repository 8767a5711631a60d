"""Plain CPU oracle for the routed FP4 expert FFN of a DeepSeek-style MoE decoder layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The product path
(``fp4_expert_ffn_amd``: HIP kernels behind a C ABI) never imports it, and this module
imports nothing from the product path: NumPy and the standard library only.

Everything here is fp64 and written for checking by eye, not for speed: no blocking, no
fusion, no reordering beyond what each definition states. Library primitives used as steps:
``numpy.matmul`` (a plain fp64 matrix product), ``numpy.exp`` and ``numpy.ldexp``.

Sources. The pages this follows, cited by title and section:

* [A100-FP4] shi3z, "DeepSeek v4.1 Flashを動かしたくてFP4に対応していないA100を、33tok/sから
  673 tok/sまで持っていって気がつくと公式APIより速くなっていた話" (note.com), and its Chinese
  translation "把不支持 FP4 的 A100 拉到 673 tok/s". Section 「FP4非対応」という言葉を疑う
  (Chinese: 质疑「不支持 FP4」这句话): E2M1 has 2 exponent bits and 1 mantissa bit; twice
  its values are the small integers 0, ±1, ±2, ±3, ±4, ±6, ±8, ±12; a 4-bit by 4-bit product
  has only 256 cases.
* [8GB-GPU] "在 8 GB 显卡上运行 510 GB 的 DeepSeek-V4.1-Flash——以及三个从不抛错的 Bug".
  Section 每 token 字节数决定一切: 384 experts per layer, 6 chosen per token, 17.93 MiB per
  FP4 expert with scales. Section 方案：不重写模型，只迁移其存储: the three matrices of an
  expert are stored next to each other (17.7 MB) and the scales are a separate block
  (1.1 MB). Section RTX 50xx 上的三个从不抛错的 Bug: the scale format is ue8m0.
* [A100-FP4], Chinese translation, section A100 也没有 FP8: the dense weights (the shared
  expert, the dense projections) are FP8 E4M3, kept as a storage format and turned into bf16
  matrix-core operands in registers.

Readings taken where the pages are silent (each is listed with its reason in the design notes):

* E2M1 code layout is the OCP MX one: bit 3 sign, bits 2:1 exponent with bias 1, bit 0
  mantissa. Two codes per byte, the low nibble holds the even K index.
* A ue8m0 scale byte ``e`` means 2**(e - 127); e == 255 means NaN.
* One scale per 32 consecutive elements along K (the only block size that gives 1.1 MB of
  one-byte scales next to 17.7 MB of codes for hidden 4096 and intermediate 2880).
* Matrices per expert, in this order: gate [I x H], up [I x H], down [H x I], each row-major
  [out x in] (K = in is the contiguous axis).
* Router: logits = W_r x accumulated in fp64; the k largest logits, ordered by descending
  logit with ties going to the lower expert id; weights = softmax over those k logits only
  (a full softmax renormalised over the chosen k gives the same numbers, since the full
  denominator cancels).
* SwiGLU: h = silu(g) * u with silu(z) = z / (1 + exp(-z)); no clamp, routed scaling factor
  1; the routed FFN has no shared expert term (the FP8 shared expert is computed on its own,
  section 6a).
* Combine: y = sum_j w_j * y_{e_j}, summed in ascending expert id. Ids outside [0, E)
  contribute nothing. Duplicate ids are legal and add up.
"""

from __future__ import annotations

import math
from typing import Callable, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------------------
# 1. Number formats
# ---------------------------------------------------------------------------------------

#: The 16-entry E2M1 value table, indexed by the 4-bit code. Codes 0..7 are the positive
#: values (exponent field 0 is subnormal: 0 and 0.5), codes 8..15 the same magnitudes with
#: the sign bit set ([A100-FP4], 「FP4非対応」という言葉を疑う; code layout per the OCP MX reading).
E2M1_VALUES: Tuple[float, ...] = (
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
)

#: Elements per ue8m0 scale block along K.
BLOCK = 32

#: Matrix order inside one expert blob ([8GB-GPU], 方案：不重写模型，只迁移其存储).
GATE, UP, DOWN = 0, 1, 2


def e2m1_table() -> np.ndarray:
    """The E2M1 table as a float64 array of 16 entries."""
    return np.array(E2M1_VALUES, dtype=np.float64)


def ue8m0_to_f64(e: np.ndarray) -> np.ndarray:
    """Decode ue8m0 scale bytes: 2**(e - 127) exactly in fp64, NaN for e == 255
    ([8GB-GPU], RTX 50xx 上的三个从不抛错的 Bug names the format; the meaning is the OCP
    E8M0 reading)."""
    e = np.asarray(e, dtype=np.int64)
    out = np.ldexp(np.ones(e.shape, dtype=np.float64), e - 127)
    return np.where(e == 255, np.nan, out)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly: a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 (round to nearest, ties to even, subnormals kept,
    overflow to infinity) and return the bit patterns. One value at a time, on the exact
    binary value, so no double rounding through fp32 can occur."""
    v = np.asarray(v, dtype=np.float64)
    flat = v.ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    for i in range(flat.shape[0]):
        out[i] = _f64_to_bf16_scalar(float(flat[i]))
    return out.reshape(v.shape)


def _f64_to_bf16_scalar(val: float) -> int:
    if math.isnan(val):
        return 0x7FC0
    sign = 1 if math.copysign(1.0, val) < 0 else 0
    if val == 0.0:
        return sign << 15
    if math.isinf(val):
        return (sign << 15) | 0x7F80
    m, q = math.frexp(abs(val))  # abs(val) = m * 2**q, 0.5 <= m < 1
    # bf16 normal: 1.f (7 bits) * 2**(E-127), E in 1..254; subnormal: 0.f * 2**-126.
    exp = q - 1  # abs(val) = (2m) * 2**exp with 1 <= 2m < 2
    if exp < -126:
        exp_eff = -126
    else:
        exp_eff = exp
    # quantum of the target grid at this exponent: 2**(exp_eff - 7)
    scaled = abs(val) / math.ldexp(1.0, exp_eff - 7)  # exact: power-of-two division
    lo = math.floor(scaled)
    frac = scaled - lo
    if frac > 0.5 or (frac == 0.5 and (lo & 1)):
        lo += 1
    # lo is the integer significand on the 2**(exp_eff-7) grid (may carry into next binade)
    if exp < -126:
        # subnormal range: lo in [0, 128]; 128 means the smallest normal
        bits = lo  # exponent field 0 plus mantissa, or 0x80 -> exponent field 1
    else:
        if lo == 256:  # carried into the next binade
            lo = 128
            exp_eff += 1
        if exp_eff > 127:
            return (sign << 15) | 0x7F80  # overflow to infinity
        bits = ((exp_eff + 127) << 7) | (lo - 128)
    return (sign << 15) | bits


def dequant_fp4(codes: np.ndarray, scales: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Dequantise one FP4 matrix to fp64.

    codes:  uint8 [N, K/2]; byte b of a row holds element 2b in its low nibble and element
            2b+1 in its high nibble.
    scales: uint8 [N, K/32]; one ue8m0 byte per 32 consecutive elements along K.
    Returns W [N, K] with W[n, k] = E2M1_VALUES[code[n, k]] * 2**(scale[n, k // 32] - 127),
    which is exact in fp64. ``out`` (float64 [N, K]) may be given to reuse memory.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half_k = codes.shape
    k = 2 * half_k
    if scales.shape != (n, k // BLOCK) or k % BLOCK:
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape}")
    # byte -> (value of its low nibble, value of its high nibble): element order 2b, 2b+1
    table = e2m1_table()
    byte = np.arange(256)
    pair_values = np.stack([table[byte & 0x0F], table[byte >> 4]], axis=1)   # [256, 2]
    if out is None:
        out = np.empty((n, k), dtype=np.float64)
    np.take(pair_values, codes, axis=0, out=out.reshape(n, half_k, 2))
    blocks = out.reshape(n, k // BLOCK, BLOCK)
    blocks *= ue8m0_to_f64(scales)[:, :, None]
    return out


# ---------------------------------------------------------------------------------------
# 2. Expert blobs
# ---------------------------------------------------------------------------------------

def expert_matrix_shapes(hidden: int, inter: int) -> Tuple[Tuple[int, int], ...]:
    """(rows, K) of gate, up and down for one expert."""
    return ((inter, hidden), (inter, hidden), (hidden, inter))


def expert_bytes(hidden: int, inter: int) -> Tuple[int, int]:
    """(code bytes, scale bytes) of one expert: 3 matrices of hidden*inter elements, half a
    byte per code and one byte per 32 elements ([8GB-GPU], 每 token 字节数决定一切 and
    方案：不重写模型，只迁移其存储)."""
    n = 3 * hidden * inter
    return n // 2, n // BLOCK


def split_expert(codes_flat: np.ndarray, scales_flat: np.ndarray, hidden: int, inter: int):
    """Split one canonical expert blob (codes: gate|up|down row-major, scales likewise) into
    three (codes [N, K/2], scales [N, K/32]) pairs."""
    out = []
    c_off = s_off = 0
    for rows, k in expert_matrix_shapes(hidden, inter):
        nc, ns = rows * k // 2, rows * k // BLOCK
        out.append((codes_flat[c_off:c_off + nc].reshape(rows, k // 2),
                    scales_flat[s_off:s_off + ns].reshape(rows, k // BLOCK)))
        c_off += nc
        s_off += ns
    return out


def dequant_expert(codes_flat: np.ndarray, scales_flat: np.ndarray, hidden: int, inter: int,
                   bufs: Optional[list] = None):
    """Dequantised (W_gate [I,H], W_up [I,H], W_down [H,I]) of one canonical expert blob.
    ``bufs`` (a list, filled on first use) lets consecutive calls reuse three fp64 buffers."""
    mats = split_expert(codes_flat, scales_flat, hidden, inter)
    if bufs is None:
        return tuple(dequant_fp4(c, s) for c, s in mats)
    if not bufs:
        bufs.extend(np.empty((r, kk), dtype=np.float64) for r, kk in expert_matrix_shapes(hidden, inter))
    return tuple(dequant_fp4(c, s, out=b) for (c, s), b in zip(mats, bufs))


# ---------------------------------------------------------------------------------------
# 3. Router
# ---------------------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h W_r[e, h] * x[t, h] in fp64. Every bf16 x bf16 product is exact
    in fp64; only the sum rounds."""
    x = bf16_to_f64(x_bits)
    wr = bf16_to_f64(w_router_bits)
    return np.matmul(x, wr.T)


def topk_softmax(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k selection with renormalised softmax weights, per token.

    ids[t]: the k experts with the largest logits, ordered by descending logit, equal logits
            ordered by ascending expert id.
    w[t, j] = exp(l_j - l_max) / sum over the k chosen of exp(l_i - l_max)   (fp64).
    """
    logits = np.asarray(logits, dtype=np.float64)
    t_count, n_exp = logits.shape
    if not 1 <= k <= n_exp:
        raise ValueError("k out of range")
    ids = np.empty((t_count, k), dtype=np.int32)
    w = np.empty((t_count, k), dtype=np.float64)
    expert_ids = np.arange(n_exp)
    for t in range(t_count):
        # lexsort: last key is primary -> primary descending logit, secondary ascending id
        order = np.lexsort((expert_ids, -logits[t]))[:k]
        ids[t] = order
        chosen = logits[t, order]
        ex = np.exp(chosen - chosen.max())
        w[t] = ex / ex.sum()
    return ids, w


def route(x_bits: np.ndarray, w_router_bits: np.ndarray, k: int):
    """Router GEMV then top-k softmax. Returns (ids int32 [T,k], w fp64 [T,k], logits)."""
    logits = router_logits(x_bits, w_router_bits)
    ids, w = topk_softmax(logits, k)
    return ids, w, logits


# ---------------------------------------------------------------------------------------
# 4. Expert FFN and combine
# ---------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)). For very negative z, exp(-z) overflows to inf and the
    quotient is the correct limit -0."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on a batch of rows x [T, H]: g = x W_g^T, u = x W_u^T,
    h = silu(g) * u, y = h W_d^T. All fp64."""
    g = np.matmul(x, w_gate.T)
    u = np.matmul(x, w_up.T)
    h = silu(g) * u
    return np.matmul(h, w_down.T)


ExpertSource = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def expert_ffn(x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, expert_source: ExpertSource,
               n_experts: int, hidden: int, inter: int) -> np.ndarray:
    """The routed expert FFN with the router-weighted combine, fp64.

    x_bits: bf16 bits [T, H]; ids: int [T, k]; w: float [T, k] (used as given);
    expert_source(e) returns the canonical (codes, scales) of expert e.
    y[t] = sum over j, in ascending expert id, of w[t, j] * expert_{ids[t, j]}(x[t]).
    Ids outside [0, n_experts) contribute nothing.
    """
    x = bf16_to_f64(x_bits)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    t_count = x.shape[0]
    y = np.zeros((t_count, hidden), dtype=np.float64)
    valid = (ids >= 0) & (ids < n_experts)
    bufs: list = []
    # Visiting experts in ascending id makes every token's sum run in ascending id order.
    for e in np.unique(ids[valid]):
        rows_t, slots = np.nonzero(ids == e)
        wg, wu, wd = dequant_expert(*expert_source(int(e)), hidden, inter, bufs)
        # one token may pick the same expert twice: each (t, slot) pair adds its own term
        ye = swiglu_expert(x[rows_t], wg, wu, wd)
        for r in range(rows_t.shape[0]):
            y[rows_t[r]] += w[rows_t[r], slots[r]] * ye[r]
    return y


def moe_layer(x_bits: np.ndarray, w_router_bits: np.ndarray, k: int, expert_source: ExpertSource,
              n_experts: int, hidden: int, inter: int):
    """Route then expert FFN: returns (y fp64 [T,H], ids, w)."""
    ids, w, _ = route(x_bits, w_router_bits, k)
    return expert_ffn(x_bits, ids, w, expert_source, n_experts, hidden, inter), ids, w


# ---------------------------------------------------------------------------------------
# 5. MX activation formats: the reading taken for activations that enter block-scaled
#    matrix cores. DeepSeek quantises activations to FP8 with ue8m0 block scales
#    ([8GB-GPU], RTX 50xx 上的三个从不抛错的 Bug names the act_quant step and its ue8m0 format);
#    the pages give no block size, scale rule or rounding. The reading taken here: blocks of
#    32 along K, one power-of-two scale 2^X per block, X the SMALLEST integer with
#    max|v| <= vmax * 2^X (vmax the element format's largest value), elements rounded to the
#    nearest value of the element format with ties to the even code. This scale rule is this
#    project's own choice, not the OCP MX v1.0 one: OCP takes X = floor(log2(max|v|)) - emax
#    (emax = 8 for E4M3) and saturates the elements that then exceed vmax. The two agree
#    unless the block maximum's significand exceeds vmax's (1.75 for E4M3, 1.875 for E2M3,
#    1.5 for E2M1); there this rule picks X one larger, so no element is ever clipped.
# ---------------------------------------------------------------------------------------

#: element formats: (exponent bits, mantissa bits, exponent bias, largest finite value)
MX_FORMATS = {
    "e4m3": (4, 3, 7, 448.0),  # FP8; the all-ones code is NaN, so 448 = 1.75 * 2^8 is the top
    "e2m3": (2, 3, 1, 7.5),    # FP6
    "e2m1": (2, 1, 1, 6.0),    # FP4 (the weight format)
}


def mx_grid(fmt: str) -> np.ndarray:
    """Non-negative values of an element format in code order (code i -> grid[i]):
    subnormals m / 2^mb * 2^(1 - bias), then normals (1 + m / 2^mb) * 2^(e - bias), up to
    the largest finite value."""
    eb, mb, bias, vmax = MX_FORMATS[fmt]
    vals = [m / 2.0 ** mb * 2.0 ** (1 - bias) for m in range(2 ** mb)]
    for e in range(1, 2 ** eb):
        for m in range(2 ** mb):
            vals.append((1.0 + m / 2.0 ** mb) * 2.0 ** (e - bias))
    vals = [v for v in vals if v <= vmax]
    return np.array(vals, dtype=np.float64)


def mx_round(v: np.ndarray, fmt: str) -> np.ndarray:
    """Round to the nearest value of the format, ties to the even code (|v| <= max)."""
    grid = mx_grid(fmt)
    a = np.abs(np.asarray(v, dtype=np.float64))
    if np.any(a > grid[-1]):
        raise ValueError("value outside the format's range")
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, grid.size - 1)
    lo = np.clip(hi - 1, 0, grid.size - 1)
    d_hi = grid[hi] - a
    d_lo = a - grid[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    q = np.where(pick_lo, grid[lo], grid[hi])
    return np.copysign(q, v)


def mx_scale_exponent(amax: float, vmax: float) -> int:
    """Smallest integer X with amax <= vmax * 2^X, clamped to the ue8m0 range [-127, 127];
    amax == 0 gives -127. (This project's scale rule; see the section note: it is one larger
    than the OCP MX rule's exponent when amax's significand exceeds vmax's.)"""
    if amax == 0.0:
        return -127
    x = math.frexp(amax)[1] - math.frexp(vmax)[1] - 1
    while amax > math.ldexp(vmax, x):
        x += 1
    while x > -127 and amax <= math.ldexp(vmax, x - 1):
        x -= 1
    return max(-127, min(127, x))


def mx_scale_exponents(amax: np.ndarray, vmax: float) -> np.ndarray:
    """mx_scale_exponent for an array of block maxima (same rule, all blocks at once)."""
    amax = np.asarray(amax, dtype=np.float64)
    x = np.frexp(amax)[1].astype(np.int64) - math.frexp(vmax)[1] - 1
    for _ in range(3):  # x starts at most two below the answer
        x = np.where(amax > np.ldexp(vmax, x), x + 1, x)
    x = np.where(amax == 0.0, -127, x)
    return np.clip(x, -127, 127)


def mx_quantize(v: np.ndarray, fmt: str, terms: int = 1) -> np.ndarray:
    """Dequantised value of v [..., K] (K a multiple of 32) after MX quantisation along
    the last axis: one term q1 = 2^X round(v / 2^X), or two terms q1 + q2 where q2 is the
    same quantisation of the residual v - q1 with its own block exponent."""
    v = np.asarray(v, dtype=np.float64)
    vmax = MX_FORMATS[fmt][3]
    rem = v.reshape(-1, BLOCK).copy()
    out = np.zeros_like(rem)
    for _ in range(terms):
        x = mx_scale_exponents(np.max(np.abs(rem), axis=1), vmax)[:, None]
        q = np.ldexp(mx_round(np.ldexp(rem, -x), fmt), x)
        out += q
        rem -= q
    return out.reshape(v.shape)


def expert_ffn_mx(x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, expert_source: ExpertSource,
                  n_experts: int, hidden: int, inter: int, fmt: str, terms: int) -> np.ndarray:
    """expert_ffn with the activations x and h replaced by their MX quantisation (fmt,
    terms) before each projection: the numerics of a block-scaled matrix-core path, for
    the activation-format study. fp64 otherwise."""
    x = mx_quantize(bf16_to_f64(x_bits), fmt, terms)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    y = np.zeros((x.shape[0], hidden), dtype=np.float64)
    valid = (ids >= 0) & (ids < n_experts)
    bufs: list = []
    for e in np.unique(ids[valid]):
        rows_t, slots = np.nonzero(ids == e)
        wg, wu, wd = dequant_expert(*expert_source(int(e)), hidden, inter, bufs)
        xe = x[rows_t]
        h = silu(np.matmul(xe, wg.T)) * np.matmul(xe, wu.T)
        ye = np.matmul(mx_quantize(h, fmt, terms), wd.T)
        for r in range(rows_t.shape[0]):
            y[rows_t[r]] += w[rows_t[r], slots[r]] * ye[r]
    return y


# ---------------------------------------------------------------------------------------
# 6a. Dense FP8 weights: the shared expert and the dense projections. [A100-FP4], Chinese
# translation, section A100 也没有 FP8: the dense weights are FP8 (E4M3), used as a storage
# format only: each weight goes from memory into registers and becomes a bf16 matrix-core
# operand there. Readings (the pages name FP8 E4M3 but not its encoding details or its
# scaling): the OCP "FN" E4M3 encoding (bit 7 sign, bits 6:3 exponent with bias 7, bits
# 2:0 mantissa; exponent field 0 is subnormal; S.1111.111 is NaN; no infinities; largest
# finite value 448), and one fp32 multiplier per 128 x 128 block of the [out x in] matrix,
# the block-scaled FP8 layout of DeepSeek's checkpoints.
# ---------------------------------------------------------------------------------------

#: Rows and columns per fp32 scale block of an FP8 matrix.
FP8_BLOCK = 128


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[n, k] = e4m3(codes[n, k]) * scales[n // 128, k // 128], fp64 [N x K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    scales = np.asarray(scales, dtype=np.float64)
    assert scales.shape == ((n + FP8_BLOCK - 1) // FP8_BLOCK, (k + FP8_BLOCK - 1) // FP8_BLOCK)
    w = e4m3_table()[codes]
    rows = np.arange(n) // FP8_BLOCK
    cols = np.arange(k) // FP8_BLOCK
    return w * scales[rows[:, None], cols[None, :]]


def dense_fp8(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y = x W^T for bf16 x [T x K] and an FP8 matrix W [N x K]; fp64 [T x N]."""
    return np.matmul(bf16_to_f64(x_bits), dequant_fp8(codes, scales).T)


def shared_expert_fp8(x_bits: np.ndarray, gate, up, down) -> np.ndarray:
    """SwiGLU FFN with FP8 matrices (each a (codes, scales) pair): gate, up [I x H],
    down [H x I]; y = W_d (silu(W_g x) * (W_u x)), fp64 [T x H] (h is not rounded)."""
    x = bf16_to_f64(x_bits)
    return swiglu_expert(x, dequant_fp8(*gate), dequant_fp8(*up), dequant_fp8(*down))


# ---------------------------------------------------------------------------------------
# 6. Layer chaining used by the multi-layer decode workload
# ---------------------------------------------------------------------------------------

def residual_rmsnorm(r: np.ndarray, y: np.ndarray, eps: float = 1e-6):
    """r' = r + y; x' = bf16(r' / sqrt(mean(r'^2) + eps)) with unit gain.
    Returns (r' fp64, x' bf16 bits). The pages name RMSNorm among the per-layer kernels
    ([A100-FP4], 然后又发现每 token 启动 2000 次内核); residual and eps are the plain reading."""
    r2 = np.asarray(r, dtype=np.float64) + np.asarray(y, dtype=np.float64)
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True) + eps)
    return r2, f64_to_bf16_bits(r2 / rms)


def expert_sources_from_arrays(codes: np.ndarray, scales: np.ndarray) -> ExpertSource:
    """Expert source over in-memory canonical arrays codes [E, nc], scales [E, ns]."""
    def src(e: int):
        return codes[e], scales[e]
    return src


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def normwise_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max_h |y - ref| / max_h |ref| for one token (0 if both are zero)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(y - ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)
