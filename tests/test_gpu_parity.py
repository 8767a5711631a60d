"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars: router ids bit-exact (same order), router weights within 2^-22 relative, dequantised
weights bit-exact in fp32, FFN outputs per token within normwise relative error 2e-2 and
cosine >= 0.9995, repeated runs bit-identical.
"""

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import moe_inputs as S
from tests.gpu_helpers import check_ffn, check_route, log, oracle_ffn_parallel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import moe_fp4 as C
    C.lib()  # fail loudly if the library is missing
    return torch.device("cuda:0")


def _mods():
    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C
    return C, D


def _layer(wl, dev, layer=0):
    C, D = _mods()
    packed = D.upload_experts(S.expert_source(wl, layer), wl.n_experts, wl.hidden, wl.inter, dev)
    wr = D.upload_bf16(S.router_weights(wl, layer), dev)
    return D.MoeFp4Layer(packed, wl.n_experts, wl.hidden, wl.inter, wl.k, wr)


def _random_routing(rng, T, k, E, distinct=True):
    if distinct:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
    return ids, w


DECODE, GROUPED, SMALL_M, GROUPED_FP8 = 1, 2, 3, 4  # moe_fp4_expert_ffn_ex paths
PATHS = pytest.mark.parametrize("path", [DECODE, GROUPED, SMALL_M, GROUPED_FP8],
                                ids=["decode", "grouped", "small_m", "grouped_fp8"])


def _ref(path, x_bits, ids, w, src, E, H, I):
    """The oracle result a path is held to: the exact FFN, or for the opt-in single-term FP8
    path the FFN on x and h quantised to one MXFP8 term (its own numerics)."""
    if path == GROUPED_FP8:
        return O.expert_ffn_mx(x_bits, ids, w, src, E, H, I, "e4m3", 1)
    return O.expert_ffn(x_bits, ids, w, src, E, H, I)


def _run_ffn(layer, x_bits, ids, w, dev, path=None):
    _, D = _mods()
    T, k = ids.shape
    if path == SMALL_M and (T < 2 or T * k > 256):
        pytest.skip("the small-M path takes 2 <= T and T * k <= 256")
    if path == SMALL_M and max(layer.hidden, layer.inter) > 8192:
        # groups of two bf16 rows no longer fit the path's 32 KB of LDS: refused, not run
        C, _ = _mods()
        with pytest.raises(C.MoeFp4Error) as err:
            layer.ffn(D.upload_bf16(x_bits, dev), torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev),
                      torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev), path=path)
        assert err.value.status == C.ERR_BAD_SHAPE
        pytest.skip("max(hidden, inter) > 8192: the small-M path refuses the shape")
    x = D.upload_bf16(x_bits, dev)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev)
    w_d = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev)
    y = layer.ffn(x, ids_d, w_d, path=path)
    torch.cuda.synchronize()
    return D.bf16_bits(y)


# ------------------------------------------------------------------------------ dequant

def _bf16_dequant_ref(c, s):
    """The oracle's exact value rounded to bf16 (the FFN kernels' operand format), as fp32:
    exact except where the magnitude reaches 2^128 (+-inf); NaN for scale byte 255."""
    return O.bf16_to_f64(O.f64_to_bf16_bits(O.dequant_fp4(c, s))).astype(np.float32)


def _assert_same_bits(got, ref, label):
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{label}: NaN positions differ"
    gb, rb = got.view(np.uint32)[~nan_g], ref.view(np.uint32)[~nan_r]
    bad = np.nonzero(gb != rb)[0]
    assert bad.size == 0, f"{label}: {bad.size} mismatches, first {got[~nan_g][bad[:4]]} vs {ref[~nan_r][bad[:4]]}"


def test_dequant_all_codes_and_scales_bit_exact(dev):
    """moe_fp4_debug_dequant runs the FFN kernels' own decode (the FP4 -> bf16 conversion
    with the ue8m0 byte as its scale operand). Every code pair meets every scale byte
    0..255 in each of gate, up and down: bit-exact against the oracle rounded to bf16,
    i.e. exact 2^(e-127) scaling including e = 0 and 1 (bf16 subnormals), +-inf where the
    value reaches 2^128 (e = 253 with |v| >= 4, e = 254 with |v| >= 2), NaN for e = 255."""
    C, D = _mods()
    H, I = 256, 128
    # gate and up: block b has bytes 16b..16b+15 (mod 256), so every code byte occurs, and
    # scale byte b mod 256 (1024 blocks: every (code, scale) pair four times); down: the
    # same pattern over its own 1024 blocks, shifted by one byte so the pairing differs.
    n = I * H // 2
    base_codes = (np.arange(n) % 256).astype(np.uint8)
    base_scales = (np.arange(I * H // 32) % 256).astype(np.uint8)
    codes = np.concatenate([base_codes, base_codes[::-1], (base_codes + 1).astype(np.uint8)])
    scales = np.concatenate([base_scales, base_scales[::-1], (base_scales + 7).astype(np.uint8)])
    packed = D.upload_experts(lambda e: (codes, scales), 1, H, I, dev)
    mats = O.split_expert(codes, scales, H, I)
    for m, (c, s) in enumerate(mats):
        assert set(np.unique(s).tolist()) == set(range(256))
        out = torch.empty(c.shape[0] * c.shape[1] * 2, dtype=torch.float32, device=dev)
        C.moe_fp4_debug_dequant(packed, 1, H, I, 0, m, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(c.shape[0], -1)
        _assert_same_bits(got, _bf16_dequant_ref(c, s), f"matrix {m}")
    log("dequant: the FFN decode of all 16 codes x 256 scale bytes bit-exact (bf16)")


@pytest.mark.parametrize("H,I,E", [(256, 128, 3), (4096, 2880, 2), (320, 96, 4)])
def test_pack_round_trip_bit_exact(dev, H, I, E):
    C, D = _mods()
    wl = S.small_workload(H, I, E, 1, 1, wid=201)
    packed = D.upload_experts(S.expert_source(wl), E, H, I, dev, chunk=2)
    for e in range(E):
        mats = O.split_expert(*S.expert_blob(wl, 0, e), H, I)
        for m, (c, s) in enumerate(mats):
            out = torch.empty(c.shape[0] * c.shape[1] * 2, dtype=torch.float32, device=dev)
            C.moe_fp4_debug_dequant(packed, E, H, I, e, m, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy().reshape(c.shape[0], -1)
            assert np.array_equal(got, _bf16_dequant_ref(c, s)), (e, m)


# ------------------------------------------------------------------------------ activation quantiser

@pytest.mark.parametrize("terms", [1, 2])
@pytest.mark.parametrize("H", [4096, 2880, 96])
def test_act_quant_bit_exact(dev, terms, H):
    """The grouped path's activation quantiser (x -> MX hi [+ lo], ue8m0 per 32), decoded
    back to fp32, equals the oracle's MX quantisation bit for bit: codes and scales are
    rounding decisions on the same bf16 inputs. terms 1 is the one-term E4M3 (FP8) mode,
    terms 2 the default grouped path's two E2M3 (FP6) terms. Blocks with zeros, a single
    value, E4M3 and E2M3 grid ties, values 2^-12 below their block maximum, rows scaled over
    2^-40 .. 2^40, blocks at 2^-98, 2^-110, bf16-subnormal magnitudes (block exponent
    clamped to -127) and 2^124, and a ragged last 128-chunk (H 96, 2880)."""
    C, D = _mods()
    rng = np.random.default_rng(H + terms)
    T = 37
    v = rng.standard_normal((T, H)) * np.exp2(rng.integers(-40, 40, size=(T, 1)).astype(np.float64))
    v[0, :32] = 0.0
    v[1, :32] = 0.0
    v[1, 5] = -3.0
    v[2, :32] = np.arange(32) / 4.0               # E4M3 ties after scaling
    v[3, :32] = np.where(np.arange(32) % 2 == 0, 1.0, 2.0 ** -12)
    v[4, :32] = -(np.arange(32) + 0.5) * 0.0625   # every half-step between grid values
    g6 = O.mx_grid("e2m3")
    v[5, :32] = np.append((g6[:-1] + g6[1:]) / 2.0, 7.5)  # E2M3 midpoints at scale 1
    z = rng.standard_normal((4, 32))
    v[6, :32] = z[0] * 2.0 ** -98    # block exponent near -100
    v[7, :32] = z[1] * 2.0 ** -110   # block exponent near -112
    v[8, :32] = z[2] * 2.0 ** -129   # bf16 subnormals: exponent clamped to -127
    v[9, :32] = z[3] * 2.0 ** 124    # near the top of the range
    x_bits = O.f64_to_bf16_bits(v)
    x = D.upload_bf16(x_bits, dev)
    nbytes = C.moe_fp4_debug_act_quant_bytes(T, H)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    C.moe_fp4_debug_act_quant(x, T, H, terms, ws, nbytes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = O.mx_quantize(O.bf16_to_f64(x_bits), "e2m3" if terms == 2 else "e4m3", terms)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[:3].tolist()}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"


# ------------------------------------------------------------------------------ router

def test_route_ids_bit_exact_full_size(dev):
    C, D = _mods()
    wl = S.WORKLOADS["layer_decode_h4096_i2880_e384"]
    wr_bits = S.router_weights(wl, 0)
    # exact ties: rows 12 and 300 equal row 7; token 0 points along row 7
    wr_bits[12] = wr_bits[7]
    wr_bits[300] = wr_bits[7]
    T = 256
    x_bits = np.concatenate([S.activations(wl, 0, s) for s in range(T)])
    x_bits[0] = wr_bits[7]
    ids_ref, w_ref, _ = O.route(x_bits, wr_bits, wl.k)
    assert list(ids_ref[0][:3]) == [7, 12, 300]
    layer = D.MoeFp4Layer(torch.empty(256, dtype=torch.uint8, device=dev), wl.n_experts,
                          wl.hidden, wl.inter, wl.k, D.upload_bf16(wr_bits, dev))
    ids, w = layer.route(D.upload_bf16(x_bits, dev))
    torch.cuda.synchronize()
    check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, "route")


@pytest.mark.parametrize("n_experts,k", [(384, 6), (20, 3), (64, 8), (200, 1)])
def test_route_batch1_sequence(dev, n_experts, k):
    """Batch-1 routing takes the one-launch path (its workspace keeps synchronisation words
    from call to call): consecutive calls on one workspace with different tokens must each
    match the oracle, including a token with exact ties among the top scores."""
    C, D = _mods()
    wl = S.WORKLOADS["layer_decode_h4096_i2880_e384"]
    wr_bits = S.router_weights(wl, 0)[:n_experts].copy()
    wr_bits[n_experts - 1] = wr_bits[3]
    layer = D.MoeFp4Layer(torch.empty(256, dtype=torch.uint8, device=dev), n_experts,
                          wl.hidden, wl.inter, k, D.upload_bf16(wr_bits, dev))
    for step in range(12):
        x_bits = S.activations(wl, 0, 1000 + step)
        if step == 5:
            x_bits = wr_bits[3:4].copy()
        ids_ref, w_ref, _ = O.route(x_bits, wr_bits, k)
        ids, w = layer.route(D.upload_bf16(x_bits, dev))
        torch.cuda.synchronize()
        check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, f"step {step}")
        if step == 5 and k >= 2:
            assert list(ids_ref[0][:2]) == [3, n_experts - 1]


@pytest.mark.parametrize("n_experts", [1020, 1021])
def test_route_batch1_record_area_edge(dev, n_experts):
    """The one-launch batch-1 route keeps one 16-byte logit record per expert in the route
    workspace's synchronisation area: 1020 experts are the most it holds, 1021 take the
    two-launch route. Both must match the oracle over consecutive calls on one workspace,
    including a token with an exact tie between the first and the last expert."""
    C, D = _mods()
    k = 6
    wl = S.small_workload(4096, 128, n_experts, k, 1, wid=920)
    wr_bits = S.router_weights(wl, 0).copy()
    wr_bits[n_experts - 1] = wr_bits[0]
    layer = D.MoeFp4Layer(torch.empty(256, dtype=torch.uint8, device=dev), n_experts,
                          wl.hidden, wl.inter, k, D.upload_bf16(wr_bits, dev))
    for step in range(6):
        x_bits = S.activations(wl, 0, step)
        if step == 3:
            x_bits = wr_bits[0:1].copy()
        ids_ref, w_ref, _ = O.route(x_bits, wr_bits, k)
        C.moe_fp4_timing_reset()
        C.moe_fp4_timing_enable(True)
        ids, w = layer.route(D.upload_bf16(x_bits, dev))
        torch.cuda.synchronize()
        C.moe_fp4_timing_enable(False)
        launched = {n for kind, n in enumerate(C.KERNEL_NAMES) if C.moe_fp4_timing_read(kind)[0]}
        C.moe_fp4_timing_reset()
        # the kernels that ran: one launch up to 1020 experts, GEMV + selection above
        expect = {"route_decode"} if n_experts <= 1020 else {"router_gemv", "topk"}
        assert launched == expect, (n_experts, launched)
        check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, f"E {n_experts} step {step}")
        if step == 3:
            assert list(ids_ref[0][:2]) == [0, n_experts - 1]


def test_route_batch1_give_up_is_reported_and_sticky(dev):
    """A batch-1 route whose wait for the logit records gives up (forced from the host: a
    spin bound of 0 polls, so every kernel still runs to its normal end) writes ids -1 and
    weights 0, marks its workspace, and keeps doing so on later calls, also with the normal
    bound, until moe_fp4_route_reset; the routed FFN then contributes nothing (y = 0), and
    after the reset the route matches the oracle again."""
    C, D = _mods()
    wl = S.WORKLOADS["layer_decode_h4096_i2880_e384"]
    wr_bits = S.router_weights(wl, 0)[:64].copy()
    k = 6
    layer = D.MoeFp4Layer(torch.empty(256, dtype=torch.uint8, device=dev), 64, wl.hidden,
                          wl.inter, k, D.upload_bf16(wr_bits, dev))
    status = torch.full((1,), 7, dtype=torch.int32, device=dev)

    def route_and_status(step):
        x_bits = S.activations(wl, 0, 2000 + step)
        ids, w = layer.route(D.upload_bf16(x_bits, dev))
        C.moe_fp4_route_status(layer._rws, status)
        torch.cuda.synchronize()
        return x_bits, ids.cpu().numpy(), w.cpu().numpy(), int(status.item())

    try:
        x_bits, ids, w, st = route_and_status(0)
        ids_ref, w_ref, _ = O.route(x_bits, wr_bits, k)
        check_route(ids, w, ids_ref, w_ref, "before")
        assert st == 0
        C.moe_fp4_debug_route_spin_limit(0)
        _, ids, w, st = route_and_status(1)
        assert np.all(ids == -1) and np.all(w == 0.0) and st == 1, (ids, w, st)
        C.moe_fp4_debug_route_spin_limit(-1)  # the normal bound again: still failed
        _, ids, w, st = route_and_status(2)
        assert np.all(ids == -1) and np.all(w == 0.0) and st == 1
        bad = torch.zeros(1, dtype=torch.int32, device=dev)
        C.moe_fp4_validate_ids(torch.from_numpy(ids).to(dev), 1, k, 64, bad)
        torch.cuda.synchronize()
        assert int(bad.item()) == k
        C.moe_fp4_route_reset(layer._rws)
        for step in (3, 4, 5):
            x_bits, ids, w, st = route_and_status(step)
            ids_ref, w_ref, _ = O.route(x_bits, wr_bits, k)
            check_route(ids, w, ids_ref, w_ref, f"after reset, step {step}")
            assert st == 0
    finally:
        C.moe_fp4_debug_route_spin_limit(-1)


def test_moe_forward_give_up_outputs_zero(dev):
    """The one-call layer on a workspace whose batch-1 route gave up: ids -1, weights 0 and
    y exactly 0 (the FFN skips every slot), then correct again after moe_fp4_route_reset."""
    C, D = _mods()
    wl = S.small_workload(256, 128, 8, 2, 1, wid=960)
    layer = _layer(wl, dev)
    x_bits = S.activations(wl, 0, 0)
    x = D.upload_bf16(x_bits, dev)
    try:
        C.moe_fp4_debug_route_spin_limit(0)
        y, ids, w = layer.forward_fused(x)
        torch.cuda.synchronize()
        assert torch.all(ids == -1) and torch.all(w == 0) and torch.all(y.float() == 0)
    finally:
        C.moe_fp4_debug_route_spin_limit(-1)
    C.moe_fp4_route_reset(layer._fws)
    y, ids, w = layer.forward_fused(x)
    torch.cuda.synchronize()
    ids_ref, w_ref, _ = O.route(x_bits, S.router_weights(wl, 0), wl.k)
    check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, "forward after reset")
    ref = O.expert_ffn(x_bits, ids_ref, w_ref, S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter)
    check_ffn(D.bf16_bits(y), ref, "forward after reset")


@pytest.mark.parametrize("routing", ["zipf", "uniform", "ties"])
def test_route_logits_bit_exact(dev, routing):
    C, D = _mods()
    if routing == "ties":
        wl = S.WORKLOADS["batched64_zipf"]
        lg = S.router_logits(wl, 0, 0, tokens=300)
        lg = np.round(lg * 2) / 2  # many exact ties
        lg[0, :] = 0.0
        lg = lg.astype(np.float32)
    else:
        wl = S.WORKLOADS["batched64_zipf" if routing == "zipf" else "prefill8192_uniform"]
        lg = S.router_logits(wl, 0, 0, tokens=1000)
    T = lg.shape[0]
    ids_ref, w_ref = O.topk_softmax(lg.astype(np.float64), 6)
    layer = D.MoeFp4Layer(torch.empty(256, dtype=torch.uint8, device=dev), 384, 4096, 2880, 6)
    ids, w = layer.route_logits(torch.from_numpy(lg).to(dev))
    torch.cuda.synchronize()
    check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, routing)
    if routing == "ties":
        assert list(ids.cpu().numpy()[0]) == [0, 1, 2, 3, 4, 5]


# ------------------------------------------------------------------------------ FFN

def test_single_expert_h256_i128(dev):
    wl = S.WORKLOADS["expert_h256_i128"]
    layer = _layer(wl, dev)
    x_bits = S.activations(wl, 0, 0)
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1), np.float32)
    y = _run_ffn(layer, x_bits, ids, w, dev)
    ref = O.expert_ffn(x_bits, ids, w, S.expert_source(wl), 1, 256, 128)
    err, cos = check_ffn(y, ref, "expert_h256_i128")
    log(f"single expert: normwise {err:.2e} cosine {cos:.7f}")


SMALL_SHAPES = [
    # H, I, E, k, T: ragged K tails (K % 128 != 0), tiles of 16 rows, ragged token counts
    (64, 32, 4, 2, 3),
    (320, 96, 5, 3, 7),
    (512, 2880, 8, 6, 5),
    (4096, 256, 7, 6, 2),
    (7168, 512, 4, 4, 2),
    (16384, 64, 3, 2, 2),
    (96, 16384, 3, 2, 2),
    (1024, 1024, 16, 8, 17),
    # grouped-path shapes: H and I = 32 mod 64 (last 64-row tile half used), K padded to
    # 128, one and several 64-row blocks per expert, a partial last block
    (160, 96, 8, 3, 50),
    (256, 128, 4, 2, 200),
    (224, 2880, 6, 6, 40),
]


@PATHS
@pytest.mark.parametrize("H,I,E,k,T", SMALL_SHAPES)
def test_ffn_small_shapes(dev, H, I, E, k, T, path):
    wl = S.small_workload(H, I, E, k, T, wid=300 + H % 97 + I % 89)
    layer = _layer(wl, dev)
    rng = np.random.default_rng(H * 7 + I)
    ids, w = _random_routing(rng, T, k, E)
    x_bits = S.activations(wl, 0, 0)
    y = _run_ffn(layer, x_bits, ids, w, dev, path)
    ref = _ref(path, x_bits, ids, w, S.expert_source(wl), E, H, I)
    err, cos = check_ffn(y, ref, f"path {path} H{H} I{I} E{E} k{k} T{T}")
    log(f"path {path} H{H} I{I} E{E} k{k} T{T}: normwise {err:.2e} cosine {cos:.7f}")


def _restrict_codes(byte_row, scale_byte):
    """Limit the 32 codes of one block so that code * 2^(e-127) stays below 2^128, the bf16
    range: |code| <= 1.5 for e = 254, <= 3 for e = 253 (the codes' magnitude bits)."""
    lo, hi = byte_row & 0x0F, byte_row >> 4
    def fix(n):
        if scale_byte == 254:
            return n & 0xB                       # magnitude 0, 0.5, 1, 1.5
        if scale_byte == 253:
            return np.where((n & 0x6) == 0x6, n ^ 0x2, n)  # 4 -> 2, 6 -> 3
        return n
    return (fix(lo) | (fix(hi) << 4)).astype(np.uint8)


def _extreme_scale_experts(H, I):
    """Five experts with extreme ue8m0 bytes (codes uniform, other scale bytes 120..130):
     0: a quarter of the blocks of every matrix at bytes 0, 1 or 2 (bf16 subnormal weights);
     1: K-block 3 of every gate and up row at 252, 253 or 254 (codes kept below 2^128);
        the inputs' K-block 3 is scaled by 2^-112, so these blocks weigh like the others;
     2: I-block 2 of every down row at 252, 253 or 254; gate and up rows 64..95 at byte 67,
        so the h entries they meet are about 2^-110;
     3: gate row 5, K-block 1 at byte 255 (NaN): h[5] is NaN, so every output is NaN;
     4: down row 7, K-block 0 at byte 255: output row 7 is NaN, the rest finite."""
    wl = S.small_workload(H, I, 5, 2, 14, wid=950)
    rng = np.random.default_rng(950)
    experts = []
    for e in range(5):
        codes, scales = S.expert_blob(wl, 0, e)
        (gc, gs), (uc, us), (dc, ds) = O.split_expert(codes, scales, H, I)  # views
        if e == 0:
            for c, s in ((gc, gs), (uc, us), (dc, ds)):
                sel = rng.random(s.shape) < 0.25
                s[sel] = rng.integers(0, 3, size=int(sel.sum()), dtype=np.uint8)
        elif e == 1:
            for c, s in ((gc, gs), (uc, us)):
                for r in range(s.shape[0]):
                    s[r, 3] = rng.integers(252, 255)
                    c[r, 48:64] = _restrict_codes(c[r, 48:64], int(s[r, 3]))
        elif e == 2:
            for r in range(ds.shape[0]):
                ds[r, 2] = rng.integers(252, 255)
                dc[r, 32:48] = _restrict_codes(dc[r, 32:48], int(ds[r, 2]))
            gs[64:96, :] = 67
            us[64:96, :] = 67
        elif e == 3:
            gs[5, 1] = 255
        else:
            ds[7, 0] = 255
        w = np.concatenate([O.dequant_fp4(c, s).ravel() for c, s in ((gc, gs), (uc, us), (dc, ds))])
        assert np.nanmax(np.abs(w)) < 2.0 ** 128
        experts.append((codes, scales))
    return wl, experts


def _check_ffn_nan_aware(y_bits, ref, label):
    """NaN positions equal to the oracle's; the finite part of each token within the bar."""
    y = O.bf16_to_f64(y_bits)
    for t in range(y.shape[0]):
        nan_y, nan_r = np.isnan(y[t]), np.isnan(ref[t])
        assert np.array_equal(nan_y, nan_r), f"{label} token {t}: NaN positions differ " \
            f"({int(nan_y.sum())} vs {int(nan_r.sum())})"
        fin = ~nan_r
        if fin.any():
            check_ffn(O.f64_to_bf16_bits(y[t][fin])[None, :], ref[t][fin][None, :], f"{label} token {t}")


@PATHS
def test_ffn_extreme_scale_bytes(dev, path):
    """FFN parity with scale bytes 0, 1, 2, 252, 253, 254 and 255 in the weights, on every
    path: tiny blocks change nothing visible, huge blocks (balanced by tiny inputs) carry
    their exact power of two, and a NaN block poisons exactly the outputs it reaches."""
    C, D = _mods()
    H, I = 256, 128
    wl, experts = _extreme_scale_experts(H, I)
    src = lambda e: experts[e]  # noqa: E731
    packed = D.upload_experts(src, 5, H, I, dev)
    layer = D.MoeFp4Layer(packed, 5, H, I, 2)
    x = O.bf16_to_f64(S.activations(wl, 0, 0))
    x[:, 96:128] *= 2.0 ** -112
    x_bits = O.f64_to_bf16_bits(x)
    ids = np.array([[0, -1], [0, 1], [1, -1], [1, 2], [2, -1], [2, 0], [3, -1], [3, 0],
                    [4, -1], [4, 1], [0, 2], [1, 0], [2, 1], [0, 0]], np.int32)
    w = (np.random.default_rng(951).random(ids.shape) + 0.05).astype(np.float32)
    keep = np.arange(14) if path != GROUPED_FP8 else np.array([0, 1, 2, 3, 4, 5, 10, 11, 12, 13])
    y = _run_ffn(layer, x_bits, ids, w, dev, path)
    ref = _ref(path, x_bits[keep], ids[keep], w[keep], src, 5, H, I)
    _check_ffn_nan_aware(y[keep], ref, f"extreme scales, path {path}")
    if path != GROUPED_FP8:
        assert np.all(np.isnan(O.bf16_to_f64(y[6]))) and np.isnan(O.bf16_to_f64(y[8][7]))
    log(f"extreme scale bytes, path {path}: NaN positions equal, finite parts within the bar")


@pytest.fixture(scope="module")
def decode_layer(dev):
    wl = S.WORKLOADS["layer_decode_h4096_i2880_e384"]
    log("uploading 384 experts (7.2 GB)")
    return wl, _layer(wl, dev)


@pytest.mark.timeout(900)
def test_layer_decode_full_size_route_and_ffn(dev, decode_layer):
    """One 384-expert layer at full size, batch 1, 100 tokens one call at a time, as the
    bench runs them (moe_fp4_moe_forward: the one-launch route, then the decode FFN kernels):
    ids bit-exact and weights against the oracle's routing of each token, outputs within
    the bar of the oracle's FFN."""
    _, D = _mods()
    wl, layer = decode_layer
    n_tok = 100
    wr_bits = S.router_weights(wl, 0)
    x_all = np.concatenate([S.activations(wl, 0, s) for s in range(n_tok)])
    xd = D.upload_bf16(x_all, dev)
    ys, idss, ws = [], [], []
    for s in range(n_tok):
        y, ids, w = layer.forward_fused(xd[s:s + 1])
        ys.append(y.clone()), idss.append(ids.clone()), ws.append(w.clone())
    torch.cuda.synchronize()
    ids_g = torch.cat(idss).cpu().numpy()
    w_g = torch.cat(ws).cpu().numpy()
    y_g = D.bf16_bits(torch.cat(ys))
    ids_ref, w_ref, _ = O.route(x_all, wr_bits, wl.k)
    check_route(ids_g, w_g, ids_ref, w_ref, "decode 100 tokens")
    ref = oracle_ffn_parallel(x_all, ids_ref, w_ref, S.expert_source(wl), wl.n_experts,
                              wl.hidden, wl.inter)
    err, cos = check_ffn(y_g, ref, "decode 100 tokens")
    log(f"decode, 100 tokens ({len(np.unique(ids_ref))} distinct experts): worst normwise "
        f"{err:.2e}, worst cosine {cos:.7f}")


def test_moe_forward_matches_route_then_ffn(dev, decode_layer):
    """The one-call layer gives bit-identical ids, weights and outputs to moe_fp4_route
    followed by moe_fp4_expert_ffn, for batch 1, a batch of 5 tokens (decode path) and 40
    tokens (grouped path); and its ids match the oracle."""
    _, D = _mods()
    wl, layer = decode_layer
    wr_bits = S.router_weights(wl, 0)
    for T, step in ((1, 100), (1, 101), (5, 102), (40, 103)):  # 40: grouped path
        x_bits = S.activations(wl, 0, step, tokens=T)
        x = D.upload_bf16(x_bits, dev)
        y1, ids1, w1 = layer.forward(x)
        y2, ids2, w2 = layer.forward_fused(x)
        torch.cuda.synchronize()
        assert torch.equal(ids1, ids2) and torch.equal(w1, w2), f"T={T}"
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"T={T}"
        ids_ref, w_ref, _ = O.route(x_bits, wr_bits, wl.k)
        check_route(ids2.cpu().numpy(), w2.cpu().numpy(), ids_ref, w_ref, f"fused T={T}")


def test_layer_batched64_zipf_full_size(dev, decode_layer):
    """64 tokens per step through the 384-expert layer, Zipf(1.1)-skewed logits."""
    _, D = _mods()
    wl_l, layer = decode_layer
    wl = S.WORKLOADS["batched64_zipf"]
    lg = S.router_logits(wl, 0, 0)
    ids, w = layer.route_logits(torch.from_numpy(lg).to(dev))
    ids_ref, w_ref = O.topk_softmax(lg.astype(np.float64), 6)
    torch.cuda.synchronize()
    check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, "zipf64")
    x_bits = S.activations(wl, 0, 0)
    # the layer holds the decode workload's experts
    ref = O.expert_ffn(x_bits, ids_ref, w_ref, S.expert_source(wl_l), 384, 4096, 2880)
    for path in (DECODE, GROUPED):
        y = layer.ffn(D.upload_bf16(x_bits, dev), ids, w, path=path)
        torch.cuda.synchronize()
        err, cos = check_ffn(D.bf16_bits(y), ref, f"zipf64 path {path}")
        log(f"batched64 zipf path {path}: {len(np.unique(ids_ref))} distinct experts, "
            f"normwise {err:.2e} cosine {cos:.7f}")
    # the single-term FP8 path against its own oracle numerics, on a sample of tokens
    sample = np.sort(np.random.default_rng(64).choice(64, size=8, replace=False))
    ref8 = O.expert_ffn_mx(x_bits[sample], ids_ref[sample], w_ref[sample], S.expert_source(wl_l),
                           384, 4096, 2880, "e4m3", 1)
    y = layer.ffn(D.upload_bf16(x_bits, dev), ids, w, path=GROUPED_FP8)
    torch.cuda.synchronize()
    yb = D.bf16_bits(y)
    err, cos = check_ffn(yb[sample], ref8, "zipf64 grouped_fp8")
    err_x = max(O.normwise_rel_err(O.bf16_to_f64(yb[sample][i]), ref[sample][i]) for i in range(8))
    log(f"batched64 zipf grouped_fp8, sample of 8: normwise {err:.2e} cosine {cos:.7f} against the "
        f"one-term MX oracle; {err_x:.2e} from the exact result")


@pytest.mark.parametrize("name", ["mtp4_correlated", "streams8_uniform"])
def test_layer_multi_token_full_size(dev, decode_layer, name):
    """The multi-token decode shapes through the 384-expert layer as the bench runs them
    (automatic path choice: the small-M kernels), every token against the oracle, and the
    decode kernels on the same routing."""
    C, D = _mods()
    wl_l, layer = decode_layer
    wl = S.WORKLOADS[name]
    lg = S.router_logits(wl, 0, 0)
    ids, w = layer.route_logits(torch.from_numpy(lg).to(dev))
    ids_ref, w_ref = O.topk_softmax(lg.astype(np.float64), 6)
    torch.cuda.synchronize()
    check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, name)
    x_bits = S.activations(wl, 0, 0)
    ref = O.expert_ffn(x_bits, ids_ref, w_ref, S.expert_source(wl_l), 384, 4096, 2880)
    C.moe_fp4_timing_reset()
    C.moe_fp4_timing_enable(True)
    y = layer.ffn(D.upload_bf16(x_bits, dev), ids, w)
    torch.cuda.synchronize()
    C.moe_fp4_timing_enable(False)
    launched = {n for kind, n in enumerate(C.KERNEL_NAMES) if C.moe_fp4_timing_read(kind)[0]}
    C.moe_fp4_timing_reset()
    assert "small_m_gate_up" in launched and "gate_up" not in launched, launched
    err, cos = check_ffn(D.bf16_bits(y), ref, f"{name} small-M")
    y_d = layer.ffn(D.upload_bf16(x_bits, dev), ids, w, path=DECODE)
    torch.cuda.synchronize()
    check_ffn(D.bf16_bits(y_d), ref, f"{name} decode")
    log(f"{name}: {len(np.unique(ids_ref))} distinct experts, small-M normwise {err:.2e} cosine {cos:.7f}")


def _prefill_sampled(dev, layer, wl_l, wl, n_sample, seed, paths):
    _, D = _mods()
    lg = S.router_logits(wl, 0, 0)
    ids, w = layer.route_logits(torch.from_numpy(lg).to(dev))
    x_bits = S.activations(wl, 0, 0)
    T = x_bits.shape[0]
    sample = np.sort(np.random.default_rng(seed).choice(T, size=n_sample, replace=False))
    ids_ref, w_ref = O.topk_softmax(lg[sample].astype(np.float64), 6)
    check_route(ids.cpu().numpy()[sample], w.cpu().numpy()[sample], ids_ref, w_ref, wl.name)
    xd = D.upload_bf16(x_bits, dev)
    ref = oracle_ffn_parallel(x_bits[sample], ids_ref, w_ref, S.expert_source(wl_l), 384, 4096, 2880)
    for path in paths:
        y = layer.ffn(xd, ids, w, path=path)
        torch.cuda.synchronize()
        yb = D.bf16_bits(y)
        assert np.all(np.isfinite(O.bf16_to_f64(yb))), f"{wl.name} path {path}"
        err, cos = check_ffn(yb[sample], ref, f"{wl.name} path {path}")
        log(f"{wl.name} path {path}, sample of {n_sample} ({len(np.unique(ids_ref))} experts): "
            f"normwise {err:.2e} cosine {cos:.7f}")
        del y


@pytest.mark.timeout(900)
def test_layer_prefill8192_sampled(dev, decode_layer):
    """8192 tokens with uniform logits through the full-size layer on the grouped path (the
    automatic choice) and the decode kernels; the oracle checks a seeded sample of 512
    tokens, which between them use nearly all 384 experts."""
    wl_l, layer = decode_layer
    _prefill_sampled(dev, layer, wl_l, S.WORKLOADS["prefill8192_uniform"], 512, 55, (None, DECODE))


@pytest.mark.timeout(900)
def test_layer_prefill32768_sampled(dev, decode_layer):
    """The 32768-token matrix-core-bound shape (512 tokens per expert) on the grouped path,
    as the bench runs it; the oracle checks a seeded sample of 64 tokens, and the one-term
    FP8 mode is held to its own oracle mode on 16 of them."""
    _, D = _mods()
    wl_l, layer = decode_layer
    wl = S.WORKLOADS["prefill32768_uniform"]
    _prefill_sampled(dev, layer, wl_l, wl, 64, 77, (None,))
    lg = S.router_logits(wl, 0, 0)
    ids, w = layer.route_logits(torch.from_numpy(lg).to(dev))
    x_bits = S.activations(wl, 0, 0)
    sample = np.sort(np.random.default_rng(78).choice(x_bits.shape[0], size=16, replace=False))
    ids_ref, w_ref = O.topk_softmax(lg[sample].astype(np.float64), 6)
    y = layer.ffn(D.upload_bf16(x_bits, dev), ids, w, path=GROUPED_FP8)
    torch.cuda.synchronize()
    ref8 = O.expert_ffn_mx(x_bits[sample], ids_ref, w_ref, S.expert_source(wl_l), 384, 4096, 2880,
                           "e4m3", 1)
    err, cos = check_ffn(D.bf16_bits(y)[sample], ref8, "prefill32768 grouped_fp8")
    log(f"prefill32768 grouped_fp8, sample of 16: normwise {err:.2e} cosine {cos:.7f}")


# ------------------------------------------------------------------------------ edge cases

@pytest.fixture(scope="module")
def small_layer(dev):
    wl = S.small_workload(512, 384, 12, 6, 1, wid=400)
    return wl, _layer(wl, dev)


@pytest.mark.parametrize("T", [1, 3, 70])
def test_moe_forward_small_layer(dev, small_layer, T):
    _, D = _mods()
    wl, layer = small_layer
    wr_bits = S.router_weights(wl, 0)
    x_bits = S.activations(wl, 0, 7, tokens=T)
    y, ids, w = layer.forward_fused(D.upload_bf16(x_bits, dev))
    torch.cuda.synchronize()
    ids_ref, w_ref, _ = O.route(x_bits, wr_bits, wl.k)
    check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, f"fused small T={T}")
    ref = O.expert_ffn(x_bits, ids_ref, w_ref, S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter)
    check_ffn(D.bf16_bits(y), ref, f"fused small T={T}")


def test_t0_is_a_no_op(dev, small_layer):
    C, D = _mods()
    wl, layer = small_layer
    y = torch.full((1, wl.hidden), 7, dtype=torch.int16, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    x = torch.zeros((1, wl.hidden), dtype=torch.int16, device=dev)
    ids = torch.zeros((1, 6), dtype=torch.int32, device=dev)
    w = torch.zeros((1, 6), dtype=torch.float32, device=dev)
    C.moe_fp4_expert_ffn(x, ids, w, 0, 6, layer.packed, wl.n_experts, wl.hidden, wl.inter, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7)


@PATHS
def test_invalid_and_duplicate_ids(dev, small_layer, path):
    C, D = _mods()
    wl, layer = small_layer
    E = wl.n_experts
    ids = np.array([[3, -1, 5, E, 1000, 2],
                    [4, 4, 4, 1, 1, 0],
                    [-5, -1, E, E + 1, 99, 2 ** 31 - 1]], np.int32)
    w = np.random.default_rng(9).random((3, 6)).astype(np.float32)
    x_bits = S.activations(wl, 0, 1, tokens=3)
    y = _run_ffn(layer, x_bits, ids, w, dev, path)
    ref = _ref(path, x_bits, ids, w, S.expert_source(wl), E, wl.hidden, wl.inter)
    check_ffn(y[:2], ref[:2], f"invalid/duplicate ids, path {path}")
    assert np.all(O.bf16_to_f64(y[2]) == 0.0)  # no valid id: exactly zero
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    C.moe_fp4_validate_ids(torch.from_numpy(ids).to(dev), 3, 6, E, bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == int(np.sum((ids < 0) | (ids >= E)))


@PATHS
@pytest.mark.parametrize("k", [1, 8])
def test_k_extremes(dev, small_layer, k, path):
    wl, layer = small_layer
    rng = np.random.default_rng(10 + k)
    ids, w = _random_routing(rng, 5, k, wl.n_experts)
    x_bits = S.activations(wl, 0, 2, tokens=5)
    y = _run_ffn(layer, x_bits, ids, w, dev, path)
    ref = _ref(path, x_bits, ids, w, S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter)
    check_ffn(y, ref, f"k={k} path {path}")


@PATHS
def test_slot_permutation_is_bit_identical(dev, small_layer, path):
    wl, layer = small_layer
    rng = np.random.default_rng(11)
    T = 9
    ids, w = _random_routing(rng, T, 6, wl.n_experts)
    ids[0, 1] = ids[0, 0]  # a duplicate id with its own weight
    x_bits = S.activations(wl, 0, 3, tokens=T)
    y0 = _run_ffn(layer, x_bits, ids, w, dev, path)
    for trial in range(3):
        perm = np.stack([rng.permutation(6) for _ in range(T)])
        y1 = _run_ffn(layer, x_bits, np.take_along_axis(ids, perm, 1), np.take_along_axis(w, perm, 1),
                      dev, path)
        assert np.array_equal(y0, y1), f"trial {trial}"
    # and token order: the grouped path's per-expert grouping must not depend on it
    tp = rng.permutation(T)
    y2 = _run_ffn(layer, x_bits[tp], ids[tp], w[tp], dev, path)
    assert np.array_equal(y0[tp], y2)


@pytest.mark.parametrize("path", [None, DECODE, GROUPED, SMALL_M, GROUPED_FP8],
                         ids=["auto", "decode", "grouped", "small_m", "grouped_fp8"])
@pytest.mark.parametrize("T", [1, 17, 64, 65, 300, 1024, 1400])
def test_row_counts_and_repeat_determinism(dev, small_layer, T, path):
    """Same input five times: bit-identical outputs and no NaN/Inf, at token counts on both
    sides of 64."""
    wl, layer = small_layer
    rng = np.random.default_rng(T)
    ids, w = _random_routing(rng, T, 6, wl.n_experts)
    x_bits = S.activations(wl, 0, 4, tokens=T)
    outs = [_run_ffn(layer, x_bits, ids, w, dev, path) for _ in range(5)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.all(np.isfinite(O.bf16_to_f64(outs[0])))
    sample = np.unique(np.linspace(0, T - 1, min(T, 8)).astype(int))
    ref = _ref(path, x_bits[sample], ids[sample], w[sample], S.expert_source(wl), wl.n_experts,
               wl.hidden, wl.inter)
    check_ffn(outs[0][sample], ref, f"T={T} path {path}")


def _routing_with_counts(rng, T, k, E, fixed):
    """Distinct ids per token; expert e of `fixed` (e -> n) takes slot j in tokens 0 .. n - 1,
    the other slots random among the experts not in `fixed`."""
    rest = np.array([e for e in range(E) if e not in fixed])
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        row = [e for e, n in fixed.items() if t < n]
        row += list(rng.permutation(rest)[: k - len(row)])
        ids[t] = row
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
    return ids, w


@pytest.mark.parametrize("path", [GROUPED, GROUPED_FP8], ids=["grouped", "grouped_fp8"])
@pytest.mark.parametrize("case", ["one_expert_everywhere", "group_edges"])
def test_grouped_item_order_every_token(dev, small_layer, path, case):
    """The grouped kernels walk (row block, column tile) items grouped by expert, up to eight
    row blocks per group. Every token is checked against the oracle where an expert spans
    several groups: one expert in every one of 1400 tokens (22 row blocks: groups of 8, 8
    and 6), and experts with exactly 512 and 513 pairs (one full group; a full group and a
    second group of one single-row block)."""
    wl, layer = small_layer
    rng = np.random.default_rng(31 if case == "group_edges" else 32)
    if case == "one_expert_everywhere":
        T = 1400
        ids, w = _routing_with_counts(rng, T, 6, wl.n_experts, {3: T})
    else:
        T = 600
        ids, w = _routing_with_counts(rng, T, 6, wl.n_experts, {0: 513, 1: 512})
    x_bits = S.activations(wl, 0, 9, tokens=T)
    y = _run_ffn(layer, x_bits, ids, w, dev, path)
    ref = _ref(path, x_bits, ids, w, S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter)
    check_ffn(y, ref, f"{case} path {path}")


@pytest.mark.parametrize("E,k,T", [(3, 2, 24), (4, 2, 16), (16, 6, 8)])
def test_small_m_shared_experts(dev, E, k, T):
    """Many pairs per expert: groups larger than the tile's 8 rows split into several groups
    (E 3, T 24: about 16 pairs per expert), and every token choosing the same experts (the
    MTP-like case, one group per expert). Checked against the oracle and the decode path."""
    wl = S.small_workload(320, 160, E, k, T, wid=700 + E)
    layer = _layer(wl, dev)
    rng = np.random.default_rng(E * 100 + T)
    ids, w = _random_routing(rng, T, k, E)
    x_bits = S.activations(wl, 0, 0)
    for label, idv in (("random", ids), ("shared", np.tile(ids[:1], (T, 1)))):
        y_s = _run_ffn(layer, x_bits, idv, w, dev, SMALL_M)
        y_d = _run_ffn(layer, x_bits, idv, w, dev, DECODE)
        ref = O.expert_ffn(x_bits, idv, w, S.expert_source(wl), E, wl.hidden, wl.inter)
        check_ffn(y_s, ref, f"small_m {label} E{E} k{k} T{T}")
        check_ffn(y_d, ref, f"decode {label} E{E} k{k} T{T}")


def test_auto_path_choice(dev, small_layer):
    """The automatic choice runs the decode kernels for one token, the small-M ones from 2
    to 23 tokens and the grouped ones from 24 on (read from the library's per-kernel launch
    counters)."""
    C, D = _mods()
    wl, layer = small_layer
    names = ("gate_up", "small_m_gate_up", "grouped_gate_up")
    for T, expect in ((1, "gate_up"), (2, "small_m_gate_up"), (23, "small_m_gate_up"),
                      (24, "grouped_gate_up")):
        rng = np.random.default_rng(T)
        ids, w = _random_routing(rng, T, 6, wl.n_experts)
        x_bits = S.activations(wl, 0, 5, tokens=T)
        C.moe_fp4_timing_reset()
        C.moe_fp4_timing_enable(True)
        _run_ffn(layer, x_bits, ids, w, dev)
        C.moe_fp4_timing_enable(False)
        launched = {n for kind, n in enumerate(C.KERNEL_NAMES) if C.moe_fp4_timing_read(kind)[0]}
        C.moe_fp4_timing_reset()
        assert expect in launched and not (set(names) - {expect}) & launched, (T, launched)


# ------------------------------------------------------------------------------ layer chain

@pytest.mark.parametrize("H", [4096, 320, 96])
def test_residual_rmsnorm_matches_oracle(dev, H):
    """r += y in fp32 (exactly the fp64 sum rounded to fp32) and x = bf16(r / rms): at most
    one bf16 unit in the last place from the oracle (the rounding of the normalised value
    can differ where the fp64 quotient lies within an ulp of a rounding boundary)."""
    C, D = _mods()
    rng = np.random.default_rng(H)
    T = 5
    x0 = O.f64_to_bf16_bits(rng.standard_normal((T, H)))
    y = O.f64_to_bf16_bits(rng.standard_normal((T, H)) * 3.0)
    r = torch.empty((T, H), dtype=torch.float32, device=dev)
    C.moe_fp4_residual_init(D.upload_bf16(x0, dev), r, T, H)
    xo = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    C.moe_fp4_residual_rmsnorm(r, D.upload_bf16(y, dev), xo, T, H, 1e-6)
    torch.cuda.synchronize()
    r_ref, x_ref = O.residual_rmsnorm(O.bf16_to_f64(x0), O.bf16_to_f64(y))
    assert np.array_equal(r.cpu().numpy(), r_ref.astype(np.float32))
    xg = O.bf16_to_f64(D.bf16_bits(xo))
    xr = O.bf16_to_f64(x_ref)
    ulp = np.abs(xr) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(xg - xr) <= ulp), np.max(np.abs(xg - xr) / ulp)
    assert np.mean(xg == xr) > 0.99


@pytest.mark.parametrize("H,E,k,T", [(4096, 384, 6, 1), (320, 24, 4, 1), (96, 8, 2, 1),
                                     (16384, 16, 6, 1), (4096, 384, 6, 3)])
def test_route_residual_matches_norm_then_route(dev, H, E, k, T):
    """moe_fp4_route_residual (one launch at T = 1) gives bit-identical residual, normalised
    input, ids and weights to moe_fp4_residual_rmsnorm followed by moe_fp4_route."""
    C, D = _mods()
    rng = np.random.default_rng(H + E + T)
    base = S.small_workload(H, 64, E, k, T, wid=600 + H % 97)
    wr = D.upload_bf16(S.router_weights(base, 0), dev)
    layer = D.MoeFp4Layer(torch.empty(16, dtype=torch.uint8, device=dev), E, H, 64, k, wr)
    for rep in range(3):  # repeated calls reuse the workspace's synchronisation words
        r0 = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(dev)
        y = D.upload_bf16(O.f64_to_bf16_bits(rng.standard_normal((T, H)) * 2.0), dev)
        r_fused = torch.empty_like(r0)
        x_fused = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ids1, w1 = layer.route_residual(r0, y, r_fused, x_fused, 1e-6)
        r_ref = r0.clone()
        x_ref = torch.empty_like(x_fused)
        C.moe_fp4_residual_rmsnorm(r_ref, y, x_ref, T, H, 1e-6)
        ids2, w2 = layer.route(x_ref)
        torch.cuda.synchronize()
        assert torch.equal(r_fused, r_ref), (H, E, T, rep)
        assert torch.equal(x_fused.view(torch.int16), x_ref.view(torch.int16)), (H, E, T, rep)
        assert torch.equal(ids1, ids2) and torch.equal(w1, w2), (H, E, T, rep)
        ids_o, w_o, _ = O.route(D.bf16_bits(x_ref), S.router_weights(base, 0), k)
        check_route(ids1.cpu().numpy(), w1.cpu().numpy(), ids_o, w_o, f"route_residual H{H} T{T}")


def test_layer_stack_teacher_forced(dev):
    """Four chained layers at batch 1: every layer's routing (bit-exact), FFN (tolerance)
    and residual + RMSNorm (within one bf16 ulp) checked against the oracle on the GPU's own
    input to that layer."""
    C, D = _mods()
    base = S.small_workload(512, 384, 16, 4, 1, wid=500)
    layers = [_layer(base, dev, layer=l) for l in range(4)]
    H = base.hidden
    x_bits = S.activations(base, 0, 0)
    x = D.upload_bf16(x_bits, dev)
    r = torch.empty((1, H), dtype=torch.float32, device=dev)
    C.moe_fp4_residual_init(x, r, 1, H)
    for tok in range(3):
        for l, layer in enumerate(layers):
            x_in = D.bf16_bits(x)
            r_in = r.cpu().numpy().astype(np.float64)
            y, ids, w = layer.forward_fused(x)
            xn = torch.empty_like(x)
            C.moe_fp4_residual_rmsnorm(r, y, xn, 1, H, 1e-6)
            torch.cuda.synchronize()
            ids_ref, w_ref, _ = O.route(x_in, S.router_weights(base, l), base.k)
            check_route(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, f"token {tok} layer {l}")
            ref = O.expert_ffn(x_in, ids_ref, w_ref, S.expert_source(base, l), base.n_experts, H,
                               base.inter)
            yb = D.bf16_bits(y)
            check_ffn(yb, ref, f"token {tok} layer {l}")
            _, x_ref = O.residual_rmsnorm(r_in, O.bf16_to_f64(yb))
            xg, xr = O.bf16_to_f64(D.bf16_bits(xn)), O.bf16_to_f64(x_ref)
            assert np.all(np.abs(xg - xr) <= np.abs(xr) * 2.0 ** -7 + 1e-30), (tok, l)
            x = xn
        x = D.upload_bf16(S.activations(base, 0, tok + 1), dev)  # next token: fresh input
        C.moe_fp4_residual_init(x, r, 1, H)
