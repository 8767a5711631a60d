"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test is chosen so that a plausible mistake in the oracle (a wrong table entry, a swapped
nibble, a dropped term, a transposed operand, a wrong sign) fails at least one of them.
CPU only.
"""

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import moe_inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints():
    with open(os.path.join(GOLDEN, "e2m1_doubled_integers.txt")) as f:
        line = [l for l in f if l.strip() and not l.startswith("#")][0]
    return [int(v) for v in line.split()]


# --------------------------------------------------------------------------- decode table

def test_e2m1_doubled_values_are_the_pages_integer_set():
    ints = _golden_ints()
    doubled = [2.0 * v for v in O.E2M1_VALUES]
    assert all(d == int(d) for d in doubled)
    assert sorted(set(int(d) for d in doubled)) == sorted(set(ints))
    # 16 codes onto 15 values: only +0 and -0 coincide
    assert len(set(int(d) for d in doubled)) == 15


def test_e2m1_code_order_sign_and_monotonicity():
    # The integer set does not fix which code maps to which value; the OCP layout does:
    # codes 0..7 ascend, and code 8+i is the negation of code i (sign bit 3).
    v = O.E2M1_VALUES
    assert all(v[i] < v[i + 1] for i in range(7))
    for i in range(8):
        assert v[8 + i] == -v[i]
        assert math.copysign(1.0, v[8 + i]) == -1.0
    # exponent field 0 is the subnormal pair {0, 0.5}; code 2 (exponent 1, mantissa 0) is 1.0
    assert v[0] == 0.0 and v[1] == 0.5 and v[2] == 1.0 and v[7] == 6.0


def test_all_256_products_are_exact_small_integers_over_4():
    ints = set(_golden_ints())
    pair_products = {a * b for a in ints for b in ints}
    seen = set()
    for a in range(16):
        for b in range(16):
            p4 = 4.0 * O.E2M1_VALUES[a] * O.E2M1_VALUES[b]
            assert p4 == int(p4) and -144 <= p4 <= 144
            assert int(p4) == int(2 * O.E2M1_VALUES[a]) * int(2 * O.E2M1_VALUES[b])
            seen.add(int(p4))
    assert seen == pair_products


def test_ue8m0_scale_decoding():
    e = np.arange(256)
    s = O.ue8m0_to_f64(e)
    assert s[127] == 1.0 and s[128] == 2.0 and s[126] == 0.5
    assert s[0] == 2.0 ** -127 and s[254] == 2.0 ** 127
    assert np.isnan(s[255])
    assert np.all(s[1:255] == 2.0 * s[0:254])


def test_dequant_matches_per_element_bitfield_decode():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(5, 32), dtype=np.uint8)       # [5 rows, K=64]
    scales = rng.integers(100, 150, size=(5, 2), dtype=np.uint8)
    w = O.dequant_fp4(codes, scales)
    assert w.shape == (5, 64)
    for n in range(5):
        for k in range(64):
            byte = int(codes[n, k // 2])
            c = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
            sign, exp, man = c >> 3, (c >> 1) & 3, c & 1
            mag = man * 0.5 if exp == 0 else 2.0 ** (exp - 1) * (1 + man / 2)
            ref = (-mag if sign else mag) * 2.0 ** (int(scales[n, k // 32]) - 127)
            assert w[n, k] == ref


# --------------------------------------------------------------------------- sizes

def test_expert_byte_counts_match_the_pages():
    with open(os.path.join(GOLDEN, "expert_bytes.json")) as f:
        g = json.load(f)
    codes, scales = O.expert_bytes(g["hidden"], g["intermediate"])
    assert codes == 17_694_720 and scales == 1_105_920
    assert round(codes / 1e6, 1) == g["expert_weight_MB"]
    assert round(scales / 1e6, 1) == g["expert_scale_MB"]
    assert round((codes + scales) / 2 ** 20, 2) == g["expert_MiB"]
    per_token = g["layers"] * g["experts_per_token"] * (codes + scales)
    assert round(per_token / 2 ** 30, 1) == g["per_token_GiB"]
    full = g["layers"] * g["experts_per_layer"] * (codes + scales)
    assert round(full / 2 ** 30) == g["full_expert_set_GiB"]
    # a 16- or 64-element block would not give 1.1 MB of scales
    n = 3 * g["hidden"] * g["intermediate"]
    assert round(n / 16 / 1e6, 1) != g["expert_scale_MB"]
    assert round(n / 64 / 1e6, 1) != g["expert_scale_MB"]


def test_synthetic_blob_sizes_and_determinism():
    wl = S.small_workload(64, 32, 4, 2, 3)
    c1, s1 = S.expert_blob(wl, 0, 2)
    c2, s2 = S.expert_blob(wl, 0, 2)
    assert c1.shape == (3 * 64 * 32 // 2,) and s1.shape == (3 * 64 * 32 // 32,)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    c3, _ = S.expert_blob(wl, 0, 3)
    assert not np.array_equal(c1, c3)
    assert s1.min() >= 120 and s1.max() <= 130


# --------------------------------------------------------------------------- brute force

def _bf16(x):
    return O.bf16_to_f64(x)


def _brute_ffn_token(x, ids, w, src, H, I):
    """Exact rational arithmetic for the linear parts, 50-digit decimal for SiLU."""
    getcontext().prec = 50
    xs = [Fraction(float(v)) for v in x]
    total = [Decimal(0)] * H
    for e, wj in sorted(zip(ids, w), key=lambda p: p[0]):
        codes, scales = src(int(e))
        mats = O.split_expert(codes, scales, H, I)
        wmat = []
        for c, s in mats:
            rows, hk = c.shape
            m = []
            for r in range(rows):
                row = []
                for k in range(2 * hk):
                    byte = int(c[r, k // 2])
                    code = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
                    val = Fraction(O.E2M1_VALUES[code]) * Fraction(2) ** (int(s[r, k // 32]) - 127)
                    row.append(val)
                m.append(row)
            wmat.append(m)
        g = [sum(wmat[0][i][k] * xs[k] for k in range(H)) for i in range(I)]
        u = [sum(wmat[1][i][k] * xs[k] for k in range(H)) for i in range(I)]
        h = []
        for i in range(I):
            gd = Decimal(g[i].numerator) / Decimal(g[i].denominator)
            ud = Decimal(u[i].numerator) / Decimal(u[i].denominator)
            h.append(gd / (Decimal(1) + (-gd).exp()) * ud)
        for n in range(H):
            acc = Decimal(0)
            for i in range(I):
                f = wmat[2][n][i]
                acc += Decimal(f.numerator) / Decimal(f.denominator) * h[i]
            total[n] += Decimal(repr(float(wj))) * acc
    return np.array([float(v) for v in total])


def test_ffn_matches_exact_brute_force_on_tiny_shapes():
    H, I, E, k, T = 64, 32, 4, 2, 2
    wl = S.small_workload(H, I, E, k, T, wid=101)
    src = S.expert_source(wl)
    x = S.activations(wl, 0, 0)
    ids = np.array([[3, 1], [2, 2]], dtype=np.int32)   # second token: a duplicated id
    w = np.array([[0.625, 0.375], [0.5, 0.25]])
    y = O.expert_ffn(x, ids, w, src, E, H, I)
    xf = _bf16(x)
    for t in range(T):
        ref = _brute_ffn_token(xf[t], ids[t], w[t], src, H, I)
        assert O.normwise_rel_err(y[t], ref) < 1e-12
        assert np.max(np.abs(y[t] - ref)) <= 1e-12 * np.max(np.abs(ref))


# --------------------------------------------------------------------------- closed forms

def _identity_expert(H, I):
    """gate = up = [I x H] with 1.0 on the diagonal, down = [H x I] with 1.0 on the
    diagonal, every scale 127 (factor 1)."""
    def mat(rows, k):
        c = np.zeros((rows, k // 2), dtype=np.uint8)
        for r in range(min(rows, k)):
            byte_idx, hi = divmod(r, 2)
            c[r, byte_idx] |= (0x2 << 4) if hi else 0x2      # code 0b0010 = 1.0
        s = np.full((rows, k // 32), 127, dtype=np.uint8)
        return c, s
    parts = [mat(I, H), mat(I, H), mat(H, I)]
    codes = np.concatenate([p[0].ravel() for p in parts])
    scales = np.concatenate([p[1].ravel() for p in parts])
    return codes, scales


def test_identity_weights_give_w_silu_x_times_x():
    H, I = 64, 32
    codes, scales = _identity_expert(H, I)
    rng = np.random.default_rng(5)
    x = S.f32_to_bf16_bits(rng.standard_normal((3, H), dtype=np.float32))
    ids = np.zeros((3, 1), dtype=np.int32)
    w = np.array([[0.75], [1.0], [-2.0]])
    y = O.expert_ffn(x, ids, w, lambda e: (codes, scales), 1, H, I)
    xf = _bf16(x)
    for t in range(3):
        z = xf[t, :I]
        expect = w[t, 0] * (z / (1 + np.exp(-z))) * z
        assert np.allclose(y[t, :I], expect, rtol=1e-15, atol=0)
        assert np.all(y[t, I:] == 0.0)


def test_zero_input_gives_zero_output():
    wl = S.small_workload(64, 32, 3, 2, 2, wid=102)
    x = np.zeros((2, 64), dtype=np.uint16)
    y = O.expert_ffn(x, np.array([[0, 1], [2, 0]]), np.ones((2, 2)), S.expert_source(wl), 3, 64, 32)
    assert np.all(y == 0.0)


def test_one_hot_input_selects_scaled_columns():
    H, I = 64, 32
    wl = S.small_workload(H, I, 1, 1, 1, wid=103)
    codes, scales = S.expert_blob(wl, 0, 0)
    wg, wu, wd = O.dequant_expert(codes, scales, H, I)
    c, a = 17, 1.5
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, c] = S.f32_to_bf16_bits(np.array([a], dtype=np.float32))[0]
    y = O.expert_ffn(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), lambda e: (codes, scales), 1, H, I)
    g, u = a * wg[:, c], a * wu[:, c]
    h = g / (1 + np.exp(-g)) * u
    assert np.allclose(y[0], wd @ h, rtol=1e-13, atol=1e-300)


def test_k_copies_of_one_expert_equal_that_expert():
    H, I, E = 64, 32, 3
    wl = S.small_workload(H, I, E, 4, 2, wid=104)
    src = S.expert_source(wl)
    x = S.activations(wl, 0, 0)
    single = O.expert_ffn(x, np.full((2, 1), 1, np.int32), np.ones((2, 1)), src, E, H, I)
    copies = O.expert_ffn(x, np.full((2, 4), 1, np.int32), np.full((2, 4), 0.25), src, E, H, I)
    assert np.allclose(copies, single, rtol=1e-14, atol=0)


@pytest.mark.parametrize("mat", [O.UP, O.DOWN])
def test_adding_one_to_every_up_or_down_scale_doubles_y_exactly(mat):
    H, I, E = 64, 32, 2
    wl = S.small_workload(H, I, E, 2, 3, wid=105)
    src = S.expert_source(wl)
    x = S.activations(wl, 0, 0)
    ids = np.array([[0, 1], [1, 0], [1, 1]], np.int32)
    w = np.array([[0.3, 0.7], [0.6, 0.4], [0.5, 0.5]])
    y = O.expert_ffn(x, ids, w, src, E, H, I)
    n_gu = I * H // 32

    def src2(e):
        c, s = src(e)
        s = s.copy()
        lo = mat * n_gu
        s[lo:lo + n_gu] += 1
        return c, s
    y2 = O.expert_ffn(x, ids, w, src2, E, H, I)
    assert np.array_equal(y2, 2.0 * y)


def test_permuting_pairs_and_relabelling_experts():
    H, I, E, k, T = 64, 32, 5, 3, 4
    wl = S.small_workload(H, I, E, k, T, wid=106)
    src = S.expert_source(wl)
    x = S.activations(wl, 0, 0)
    rng = np.random.default_rng(7)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    y = O.expert_ffn(x, ids, w, src, E, H, I)
    perm_slots = np.stack([rng.permutation(k) for _ in range(T)])
    ids_p = np.take_along_axis(ids, perm_slots, 1)
    w_p = np.take_along_axis(w, perm_slots, 1)
    assert np.array_equal(O.expert_ffn(x, ids_p, w_p, src, E, H, I), y)
    # relabel: blob'[pi(e)] = blob[e], ids' = pi(ids)
    pi = rng.permutation(E)
    inv = np.argsort(pi)
    y_r = O.expert_ffn(x, pi[ids].astype(np.int32), w, lambda e: src(int(inv[e])), E, H, I)
    assert np.allclose(y_r, y, rtol=1e-14, atol=1e-300)


def test_invalid_ids_contribute_nothing():
    H, I, E = 64, 32, 3
    wl = S.small_workload(H, I, E, 2, 2, wid=107)
    src = S.expert_source(wl)
    x = S.activations(wl, 0, 0)
    y = O.expert_ffn(x, np.array([[1, -1], [E, 2]], np.int32), np.ones((2, 2)), src, E, H, I)
    y1 = O.expert_ffn(x, np.array([[1], [2]], np.int32), np.ones((2, 1)), src, E, H, I)
    assert np.array_equal(y, y1)


# --------------------------------------------------------------------------- router

def test_topk_against_python_sort_with_exact_ties():
    rng = np.random.default_rng(11)
    T, E, k = 40, 64, 6
    logits = rng.standard_normal((T, E))
    # exact ties around the selection boundary
    logits[0, 5] = logits[0, 9] = logits[0, 40] = 10.0
    logits[1, :] = 0.0
    logits[2, 3] = logits[2, 60]
    ids, w = O.topk_softmax(logits, k)
    for t in range(T):
        ref = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        assert list(ids[t]) == ref
    assert list(ids[1]) == [0, 1, 2, 3, 4, 5]
    assert list(ids[0][:3]) == [5, 9, 40]


def test_softmax_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((10, 384)) * 3
    ids, w = O.topk_softmax(logits, 6)
    full = np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-14, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_router_logits_against_exact_rational_sum():
    rng = np.random.default_rng(13)
    x = S.f32_to_bf16_bits(rng.standard_normal((2, 96), dtype=np.float32))
    wr = S.f32_to_bf16_bits(0.02 * rng.standard_normal((5, 96), dtype=np.float32))
    lg = O.router_logits(x, wr)
    xf, wf = _bf16(x), _bf16(wr)
    for t in range(2):
        for e in range(5):
            exact = sum(Fraction(float(wf[e, h])) * Fraction(float(xf[t, h])) for h in range(96))
            assert abs(lg[t, e] - float(exact)) <= 1e-15 * max(1.0, abs(float(exact)))


# --------------------------------------------------------------------------- bf16 helpers

def test_bf16_round_trip_and_rounding_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    v = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3e-39, -1e-40, 3.4e38, 0.0, -0.0])])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(v.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(O.bf16_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())
    # the generator's fp32 -> bf16 rounding agrees with torch too
    assert np.array_equal(S.f32_to_bf16_bits(v), ref)


# ------------------------------------------------------------------------- MX activations

def test_mx_grids_match_the_format_definitions():
    """Value counts and extremes of the element formats, and E2M1 equal to the weight
    table (itself pinned to the pages' integer set above)."""
    g8, g6, g4 = O.mx_grid("e4m3"), O.mx_grid("e2m3"), O.mx_grid("e2m1")
    # E4M3: zero, 7 subnormals, 15 binades x 8 minus the NaN code
    assert g8.size == 127 and g8[-1] == 448.0 and g8[1] == 2.0 ** -9
    assert g6.size == 32 and g6[-1] == 7.5 and g6[1] == 0.125
    assert np.array_equal(g4, O.e2m1_table()[:8])
    for g in (g8, g6, g4):
        assert np.all(np.diff(g) > 0)


def test_mx_round_e4m3_matches_torch_float8():
    """Round-to-nearest-even onto E4M3 against torch's float8_e4m3fn conversion (an
    independent implementation), including exact midpoints between grid values."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    g = O.mx_grid("e4m3")
    mids = (g[:-1] + g[1:]) / 2.0
    vals = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-1, 1, 2000) * 2.0 ** -6,
                           mids, -mids, g, -g]).astype(np.float32).astype(np.float64)
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.mx_round(vals, "e4m3"), ref)


def test_mx_round_e2m3_hand_derived_midpoints():
    """E2M3 (FP6) rounding on hand-derived values: grid points stay, the midpoint between two
    neighbouring codes goes to the even code (0.0625 -> 0, 0.1875 -> 0.25, 0.9375 -> 1,
    1.9375 -> 2, 2.125 -> 2, 2.375 -> 2.5, 3.875 -> 4, 4.25 -> 4, 4.75 -> 5, 7.25 -> 7), values
    just off a midpoint go to the nearer code, and negative values mirror."""
    g = O.mx_grid("e2m3")
    assert np.array_equal(O.mx_round(g, "e2m3"), g)
    mids = np.array([0.0625, 0.1875, 0.9375, 1.9375, 2.125, 2.375, 3.875, 4.25, 4.75, 7.25])
    want = np.array([0.0, 0.25, 1.0, 2.0, 2.0, 2.5, 4.0, 4.0, 5.0, 7.0])
    assert np.array_equal(O.mx_round(mids, "e2m3"), want)
    assert np.array_equal(O.mx_round(-mids, "e2m3"), -want)
    up = np.array([0.0625, 2.125, 7.25]) * (1 + 2.0 ** -20)
    assert np.array_equal(O.mx_round(up, "e2m3"), [0.125, 2.25, 7.5])
    down = np.array([0.1875, 2.375, 4.75]) * (1 - 2.0 ** -20)
    assert np.array_equal(O.mx_round(down, "e2m3"), [0.125, 2.25, 4.5])
    assert np.array_equal(O.mx_round(np.array([1.2, 5.2, 0.3]), "e2m3"), [1.25, 5.0, 0.25])


def test_mx_e2m3_scale_rule_and_two_terms_hand_derived():
    """The scale rule for E2M3 (largest value 7.5 = 1.875 * 4) and one two-term block worked
    by hand: the block [1.0, 0.3, 0, ...] takes 2^-2 (7.5 / 4 = 1.875 >= 1 > 0.9375), 0.3 / 0.25
    = 1.2 rounds to 1.25, so hi = 0.3125; the residual -0.0125 takes 2^-9 (7.5 * 2^-9 >= 0.0125
    > 7.5 * 2^-10) and -0.0125 * 2^9 = -6.4 rounds to -6.5, so lo = -6.5 * 2^-9."""
    assert O.mx_scale_exponent(7.5, 7.5) == 0
    assert O.mx_scale_exponent(7.6, 7.5) == 1
    assert O.mx_scale_exponent(1.0, 7.5) == -2
    assert O.mx_scale_exponent(1.875, 7.5) == -2
    assert O.mx_scale_exponent(1.876, 7.5) == -1
    assert O.mx_scale_exponent(0.9375, 7.5) == -3
    v = np.zeros((1, 32))
    v[0, 0], v[0, 1] = 1.0, 0.3
    q1 = O.mx_quantize(v, "e2m3", 1)
    assert q1[0, 0] == 1.0 and q1[0, 1] == 0.3125 and np.all(q1[0, 2:] == 0.0)
    q2 = O.mx_quantize(v, "e2m3", 2)
    assert q2[0, 0] == 1.0 and q2[0, 1] == 0.3125 - 6.5 * 2.0 ** -9


def test_mx_scale_exponent_is_the_smallest_fitting_power():
    for n in (-20, -8, 0, 7):
        top = np.ldexp(448.0, n)
        assert O.mx_scale_exponent(top, 448.0) == n
        assert O.mx_scale_exponent(np.nextafter(top, np.inf), 448.0) == n + 1
    assert O.mx_scale_exponent(1.0, 448.0) == -8      # 448 * 2^-9 = 0.875 < 1 <= 1.75
    assert O.mx_scale_exponent(1.76, 448.0) == -7
    assert O.mx_scale_exponent(0.0, 448.0) == -127
    assert O.mx_scale_exponent(6.0, 6.0) == 0 and O.mx_scale_exponent(6.5, 6.0) == 1


def test_mx_two_terms_bound_and_one_term_exactness():
    """Two E4M3 terms reproduce a block to within 2^-7 of its maximum; values already on
    the scaled grid survive one term exactly."""
    rng = np.random.default_rng(6)
    v = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    q2 = O.mx_quantize(v, "e4m3", 2)
    amax = np.abs(v).reshape(-1, 32).max(axis=1)
    err = np.abs(q2 - v).reshape(-1, 32).max(axis=1)
    assert np.all(err <= amax * 2.0 ** -7)
    q1 = O.mx_quantize(v, "e4m3", 1)
    assert np.array_equal(O.mx_quantize(q1, "e4m3", 1), q1)
    # a whole block of zeros stays zero
    assert np.all(O.mx_quantize(np.zeros((1, 32)), "e4m3", 2) == 0.0)


def test_mx_scale_exponents_vector_form_matches_scalar_rule():
    rng = np.random.default_rng(7)
    a = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 500), rng.integers(-140, 120, 500)),
                        np.ldexp(448.0, np.arange(-20, 20)), [0.0, 448.0, 449.0, 1.75]])
    for vmax in (448.0, 7.5, 6.0):
        vec = O.mx_scale_exponents(a, vmax)
        assert [O.mx_scale_exponent(float(v), vmax) for v in a] == list(vec)


# --------------------------------------------------------------------------- layer chaining

def test_residual_rmsnorm_hand_derived_cases():
    """Hand-derived values of the residual update and the unit-gain RMSNorm:
    - a constant row c normalises to c / |c| = 1 (eps = 1e-6 is far below bf16 resolution);
    - the row pattern [3, 4, 0, 0] has mean square 25 / 4, so RMS 2.5 and normalised values
      1.2 and 1.6, whose bf16 encodings are 0x3F9A (1.203125) and 0x3FCD (1.6015625);
    - scaling the residual by 2^10 leaves x unchanged; the residual update is an exact sum."""
    r = np.zeros((2, 64))
    y = np.full((2, 64), 5.0)
    y[1] = -5.0
    r2, x = O.residual_rmsnorm(r, y)
    assert np.array_equal(r2, y)
    assert np.all(x[0] == 0x3F80) and np.all(x[1] == 0xBF80)

    pat = np.tile(np.array([3.0, 4.0, 0.0, 0.0]), 16)[None, :]
    r2, x = O.residual_rmsnorm(np.zeros_like(pat), pat)
    assert x.tolist()[0][:4] == [0x3F9A, 0x3FCD, 0, 0]
    assert np.array_equal(x[0].reshape(16, 4), np.tile(x[0][:4], (16, 1)))

    _, x_big = O.residual_rmsnorm(np.zeros_like(pat), pat * 1024.0)
    assert np.array_equal(x_big, x)

    a = np.array([[1.5, -2.25, 0.0, 8.0]])
    b = np.array([[0.25, 2.25, -1.0, 0.5]])
    r2, _ = O.residual_rmsnorm(a, b)
    assert r2.tolist() == [[1.75, 0.0, -1.0, 8.5]]


# ------------------------------------------------------------------------------ dense FP8 weights

def test_e4m3_table_matches_torch_float8_e4m3fn():
    """All 256 E4M3 codes against an independent decoder (torch's float8_e4m3fn, CPU)."""
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_table()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_hand_derived_codes():
    t = O.e4m3_table()
    assert t[0x38] == 1.0 and t[0xB8] == -1.0          # exponent 7 = bias, mantissa 0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0      # the largest finite value
    assert t[0x08] == 2.0 ** -6                         # the smallest normal
    assert t[0x01] == 2.0 ** -9                         # the smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                     # the largest subnormal
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # codes 0..126 increase


def test_fp8_block_scales_apply_per_128_block():
    """Every code 1.0, a distinct power-of-ten multiplier per 128 x 128 block of a
    260 x 300 matrix: each element carries its own block's multiplier, including the
    ragged last blocks and the elements on both sides of each block edge."""
    n, k = 260, 300
    codes = np.full((n, k), 0x38, dtype=np.uint8)
    scales = np.array([[10.0 ** (3 * i + j) for j in range(3)] for i in range(3)], dtype=np.float32)
    w = O.dequant_fp8(codes, scales)
    for (r, c) in [(0, 0), (127, 127), (128, 127), (127, 128), (128, 128), (255, 255), (256, 256),
                   (259, 299)]:
        assert w[r, c] == np.float64(scales[r // 128, c // 128]), (r, c)


def test_shared_expert_fp8_reduces_to_the_routed_expert_oracle():
    """An FP4 expert re-encoded exactly in FP8 (every FP4 value times its ue8m0 scale is an
    E4M3 value for scale bytes 120..130; block multipliers 1): the FP8 SwiGLU FFN equals the
    routed-expert oracle with one slot of weight 1, bit for bit."""
    wl = S.small_workload(256, 160, 1, 1, 3, wid=901)
    codes_flat, scales_flat = S.expert_blob(wl, 0, 0)
    table = O.e4m3_table()
    finite = ~np.isnan(table)
    value_to_code = {float(v): c for c, v in enumerate(table) if finite[c] and not (v == 0 and c)}
    mats = []
    for (c, s) in O.split_expert(codes_flat, scales_flat, wl.hidden, wl.inter):
        w = O.dequant_fp4(c, s)
        fp8 = np.vectorize(lambda v: value_to_code[float(v)] if v != 0 else 0)(w).astype(np.uint8)
        ones = np.ones(((w.shape[0] + 127) // 128, (w.shape[1] + 127) // 128), dtype=np.float32)
        assert np.array_equal(O.dequant_fp8(fp8, ones), np.where(w == 0, 0.0, w))
        mats.append((fp8, ones))
    x_bits = S.activations(wl, 0, 0)
    y8 = O.shared_expert_fp8(x_bits, *mats)
    y4 = O.expert_ffn(x_bits, np.zeros((3, 1), np.int32), np.ones((3, 1)), S.expert_source(wl),
                      1, wl.hidden, wl.inter)
    assert np.array_equal(y8, y4)


# ------------------------------------------------------------------ MX oracle mode: hand values

def _signed_identity_expert(H, I):
    """gate = +identity [I x H], up = -identity (code 0b1010 = -1.0), down = +identity
    [H x I], every scale byte 127: with inputs q >= 38 (where silu(q) == q exactly in fp64,
    since exp(-38) is below half an ulp of 1.0) the expert gives h = -q * q exactly."""
    def mat(rows, k, code):
        c = np.zeros((rows, k // 2), dtype=np.uint8)
        for r in range(min(rows, k)):
            byte_idx, hi = divmod(r, 2)
            c[r, byte_idx] |= (code << 4) if hi else code
        return c, np.full((rows, k // 32), 127, dtype=np.uint8)
    parts = [mat(I, H, 0x2), mat(I, H, 0xA), mat(H, I, 0x2)]
    return (np.concatenate([p[0].ravel() for p in parts]),
            np.concatenate([p[1].ravel() for p in parts]))


# One 32-block of x, every value exact in bf16 and >= 38. Its maximum 61 = 1.90625 * 2^5 has
# a significand above 1.75, so the scale rule matters: the smallest X with 61 <= 448 * 2^X is
# X = -2 (448 / 8 = 56 < 61), so x / 2^X = 4x is rounded on the E4M3 grid (step 16 on
# [128, 256)). The OCP MX rule would take X = -3 and clip 488 to 448 (q = 56, not 60).
_X_BLOCK = [61, 40, 41, 42, 43, 44, 46, 50, 54, 60.5, 38, 39, 58, 48, 56, 52,
            45, 47, 49, 51, 53, 55, 57, 59, 38.5, 40.5, 44.5, 48.5, 52.5, 56.5, 60, 47.5]
# 4x -> nearest grid value, ties to the even mantissa:
#   244->240, 160, 164->160, 168->160 (tie: 160 is m=2), 172->176, 176, 184->192 (tie: m=4),
#   200->192 (tie: m=4), 216->224 (tie: m=6), 242->240, 152->160 (tie: m=2), 156->160,
#   232->224 (tie: m=6), 192, 224, 208, 180->176, 188->192, 196->192, 204->208, 212->208,
#   220->224, 228->224, 236->240, 154->160, 162->160, 178->176, 194->192, 210->208,
#   226->224, 240, 190->192; divided by 4:
_Q_BLOCK = [60, 40, 40, 40, 44, 44, 48, 48, 56, 60, 40, 40, 56, 48, 56, 52,
            44, 48, 48, 52, 52, 56, 56, 60, 40, 40, 44, 48, 52, 56, 60, 48]
# h = -q^2 over I: squares 3600, 1600, 1936, 2304, 2704, 3136. Block maximum 3600 =
# 1.7578 * 2^11 (again above 1.75): X = 4 (448 * 8 = 3584 < 3600). |h| / 16 on the grid:
# 225->224, 100->96 (tie between 96 = m4 and 104 = m5), 121->120, 144, 169->176, 196->192;
# times 16:
_HQ = {3600: 3584, 1600: 1536, 1936: 1920, 2304: 2304, 2704: 2816, 3136: 3072}


def test_expert_ffn_mx_one_term_hand_derived():
    """The one-term MX oracle mode on a signed identity expert: x is quantised per 32-block
    with the scale rule above, h = -q^2 is quantised again along I before the down
    projection; every value worked by hand. Catches an unquantised x or h, the OCP scale
    rule (elements 0, 9, 23, 30 would give 56 instead of 60) and a wrong rounding tie."""
    H = I = 32
    codes, scales = _signed_identity_expert(H, I)
    x = O.f64_to_bf16_bits(np.array([_X_BLOCK], dtype=np.float64))
    assert np.array_equal(O.bf16_to_f64(x)[0], _X_BLOCK)  # every value exact in bf16
    y = O.expert_ffn_mx(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), lambda e: (codes, scales),
                        1, H, I, "e4m3", 1)
    expect = [-_HQ[q * q] for q in _Q_BLOCK]
    assert y[0].tolist() == expect


# A sparse block for the two-term case: x = [61, 41, 50, 60.5, 0 ...].
#  x hi: 60, 40, 48, 60 (as above); residual 1, 1, 2, 0.5 has maximum 2, X = -7 (3.5 >= 2 >
#  1.75), 2^7 r = 128, 128, 256, 64 all on the grid: x is reproduced exactly, so h = -x^2 =
#  -3721, -1681, -2500, -3660.25.
#  h hi: X = 4 (3721 > 3584); |h| / 16 = 232.5625 -> 240, 105.0625 -> 104, 156.25 -> 160,
#  228.765625 -> 224: hi = -3840, -1664, -2560, -3584.
#  h lo: residual 119, -17, 60, -76.25, maximum 119, X = -1 (112 < 119 <= 224); times 2:
#  238 -> 240, -34 -> -32 (tie between 32 = m0 and 36 = m1), 120, -152.5 -> -160: lo = 120,
#  -16, 60, -80. h = hi + lo = -3720, -1680, -2500, -3664.
#  One term: q = 60, 40, 48, 60, h = -3600, -1600, -2304, -3600 -> -3584, -1536, -2304, -3584.
_SPARSE_X = [61, 41, 50, 60.5]
_SPARSE_Y = {1: [-3584, -1536, -2304, -3584], 2: [-3720, -1680, -2500, -3664]}


@pytest.mark.parametrize("terms", [1, 2])
def test_expert_ffn_mx_blocks_and_tokens_get_their_own_scales(terms):
    """Two tokens, H = I = 64: token t holds the sparse block A in its first 32-block times
    2^(20 t) and in its second times 2^(20 t + 20). Each 32-block along K (x) and along I (h)
    of each token has its own scale, and power-of-two factors commute with the rounding, so
    y of block b of token t is the hand-derived block result times 2^(40 (t + b)). A scale
    shared across the two blocks, or blocks running along the token axis, would flush the
    smaller block to zero (2^-20 lies below E4M3's smallest subnormal relative to 448)."""
    H = I = 64
    codes, scales = _signed_identity_expert(H, I)
    blk = np.zeros(32)
    blk[:4] = _SPARSE_X
    x = np.stack([np.concatenate([blk * 2.0 ** (20 * t), blk * 2.0 ** (20 * t + 20)]) for t in range(2)])
    xb = O.f64_to_bf16_bits(x)
    assert np.array_equal(O.bf16_to_f64(xb), x)
    y = O.expert_ffn_mx(xb, np.zeros((2, 1), np.int32), np.ones((2, 1)), lambda e: (codes, scales),
                        1, H, I, "e4m3", terms)
    for t in range(2):
        for b in range(2):
            expect = np.zeros(32)
            expect[:4] = np.array(_SPARSE_Y[terms]) * 2.0 ** (40 * (t + b))
            assert np.array_equal(y[t, 32 * b:32 * b + 32], expect), (t, b)


def test_expert_ffn_mx_slot_weights_and_invalid_ids():
    """The MX mode keeps the combine of the exact mode: weights scale each pair's result,
    duplicate ids add, ids outside [0, E) contribute nothing (hand values from the sparse
    block, one term)."""
    H = I = 32
    codes, scales = _signed_identity_expert(H, I)
    blk = np.zeros(32)
    blk[:4] = _SPARSE_X
    xb = O.f64_to_bf16_bits(blk[None, :])
    ids = np.array([[0, 0, 1, -1]], np.int32)
    w = np.array([[0.5, 0.25, 9.0, 9.0]])
    y = O.expert_ffn_mx(xb, ids, w, lambda e: (codes, scales), 1, H, I, "e4m3", 1)
    assert y[0, :4].tolist() == [0.75 * v for v in _SPARSE_Y[1]]
    assert np.all(y[0, 4:] == 0.0)


# ------------------------------------------------------------------ dense FP8: one-hot columns

def test_dense_fp8_one_hot_columns_hand_values():
    """y = x W^T with x one-hot selects one column of W, times the input value: each element
    is e4m3(code) times the multiplier of its own (row block, column block). W is 200 x 300
    (row blocks 128 + 72, column blocks 128 + 128 + 44); token 0 is 2.0 at column 130
    (column block 1), token 1 is -1.0 at column 5 (column block 0). A transposed product or
    a multiplier indexed [column block, row block] fails."""
    n, k = 200, 300
    codes = np.full((n, k), 0x3A, dtype=np.uint8)           # 1.25 everywhere else
    mult = np.array([[0.5, 3.0, 0.25], [1.5, 10.0, 0.125]], dtype=np.float32)
    col = {0: 0x38, 127: 0x40, 128: 0xC4, 199: 0x7E, 5: 0x01, 6: 0x00}  # 1, 2, -3, 448, 2^-9, 0
    for r, c in col.items():
        codes[r, 130] = c
    codes[:, 5] = 0x38                                      # column 5: all 1.0
    codes[150, 5] = 0xB8                                    # -1.0
    x = np.zeros((2, k))
    x[0, 130] = 2.0
    x[1, 5] = -1.0
    y = O.dense_fp8(O.f64_to_bf16_bits(x), codes, mult)
    # token 0: 2 * value * mult[row block, 1]
    assert y[0, 0] == 2 * 1.0 * 3.0
    assert y[0, 127] == 2 * 2.0 * 3.0
    assert y[0, 128] == 2 * -3.0 * 10.0
    assert y[0, 199] == 2 * 448.0 * 10.0
    assert y[0, 5] == 2 * 2.0 ** -9 * 3.0
    assert y[0, 6] == 0.0
    assert y[0, 1] == 2 * 1.25 * 3.0 and y[0, 150] == 2 * 1.25 * 10.0
    # token 1: -1 * value * mult[row block, 0]
    assert y[1, 0] == -0.5 and y[1, 127] == -0.5
    assert y[1, 128] == -1.5 and y[1, 150] == 1.5 and y[1, 199] == -1.5


# ------------------------------------------------------------------ the parity checkers

def test_cosine_hand_values():
    assert O.cosine([1.0, 0.0], [0.0, 1.0]) == 0.0                 # orthogonal
    assert O.cosine([1.0, 2.0, 3.0], [2.0, 4.0, 6.0]) == pytest.approx(1.0, abs=1e-15)
    assert O.cosine([1.0, 2.0], [-1.0, -2.0]) == pytest.approx(-1.0, abs=1e-15)
    assert O.cosine([3.0, 4.0], [4.0, 3.0]) == pytest.approx(24.0 / 25.0, abs=1e-15)
    assert O.cosine([0.0, 0.0], [0.0, 0.0]) == 1.0                 # both zero: equal
    assert O.cosine([0.0, 0.0], [1.0, 2.0]) == 0.0                 # one zero
    assert O.cosine([[1.0, 0.0], [0.0, 1.0]], [[1.0, 0.0], [0.0, 1.0]]) == pytest.approx(1.0, abs=1e-15)


def test_normwise_rel_err_hand_values():
    assert O.normwise_rel_err([1.0, 2.0], [1.0, 4.0]) == 0.5       # max |diff| 2 / max |ref| 4
    assert O.normwise_rel_err([-7.0, 2.0], [-8.0, 2.0]) == 0.125   # signs: |ref| max is 8
    assert O.normwise_rel_err([3.0, -1.0], [2.0, -4.0]) == 0.75    # max diff 3 at another index
    assert O.normwise_rel_err([5.0, 5.0], [5.0, 5.0]) == 0.0
    assert O.normwise_rel_err([0.0], [0.0]) == 0.0                 # zero reference, zero output
    assert O.normwise_rel_err([1.0], [0.0]) == math.inf            # zero reference, non-zero
