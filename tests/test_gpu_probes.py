"""GPU checks of the two measurement probes behind the measured peaks: the streaming read
reads the word at every probed position of its buffer, the ragged tail included, and the
matrix-core loop runs to completion for both operand formats."""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TRIGGER = 0x9E3779B9  # the word whose XOR over the buffer makes the probe write its sink


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import moe_fp4 as C
    C.lib()
    return C


def _as_u32(v: int) -> int:
    return v - (1 << 32) if v >= (1 << 31) else v


@pytest.mark.parametrize("words16", [1, 3, 4096 * 8 + 5, (64 << 20) // 16 + 3])
def test_stream_read_covers_every_word(C, words16):
    """Each lane XORs the words it reads and writes the sink only when its XOR equals the
    trigger word; with the trigger planted alone at one position, the sink is written iff
    that position is read. Positions: first, last (the ragged tail), middle, and the last
    word of the unrolled part."""
    dev = torch.device("cuda:0")
    buf = torch.zeros(words16 * 4, dtype=torch.int32, device=dev)
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    per_round = min(2048, -(-words16 // (256 * 8))) * 256 * 8
    unrolled_end = (words16 // per_round) * per_round
    positions = sorted({0, words16 - 1, words16 // 2, max(unrolled_end - 1, 0)})
    for pos in positions:
        buf.zero_()
        buf[4 * pos + (pos % 4)] = _as_u32(TRIGGER)
        sink.fill_(7)
        C.moe_fp4_debug_stream_read(buf, buf.numel() * 4, sink)
        torch.cuda.synchronize()
        assert int(sink[0]) == _as_u32(TRIGGER), f"{words16} words, position {pos}"
    buf.zero_()
    sink.fill_(7)
    C.moe_fp4_debug_stream_read(buf, buf.numel() * 4, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 7


@pytest.mark.parametrize("fmt", [4, 0])
def test_mfma_loop_runs(C, fmt):
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda:0")
    C.moe_fp4_timing_reset()
    C.moe_fp4_timing_enable(True)
    C.moe_fp4_debug_mfma_loop(fmt, 256, 16, sink)
    torch.cuda.synchronize()
    C.moe_fp4_timing_enable(False)
    n, ms = C.moe_fp4_timing_read(C.KERNEL_NAMES.index("probe_mfma"))
    C.moe_fp4_timing_reset()
    assert n == 1 and ms > 0
    assert int(sink[0]) == 7


def test_prefetch_experts_reads_only(C):
    """moe_fp4_prefetch_experts only reads: the packed weights, the FFN's results on them and
    the sink are unchanged, for every matrix selection, with invalid ids skipped."""
    import numpy as np

    from fp4_expert_ffn_amd import device as D
    from synth import moe_inputs as S

    dev = torch.device("cuda:0")
    wl = S.small_workload(512, 384, 12, 6, 3, wid=990)
    packed = D.upload_experts(S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter, dev)
    before = packed.clone()
    layer = D.MoeFp4Layer(packed, wl.n_experts, wl.hidden, wl.inter, wl.k)
    rng = np.random.default_rng(990)
    ids = torch.from_numpy(np.stack([rng.permutation(12)[:6] for _ in range(3)]).astype(np.int32)).to(dev)
    w = torch.from_numpy(rng.random((3, 6)).astype(np.float32)).to(dev)
    x = D.upload_bf16(S.activations(wl, 0, 0), dev)
    y0 = layer.ffn(x, ids, w).clone()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    pf_ids = torch.tensor([3, -1, 11, 12, 0], dtype=torch.int32, device=dev)
    for mats in range(1, 8):
        C.moe_fp4_prefetch_experts(pf_ids, 5, packed, 12, wl.hidden, wl.inter, mats, sink)
    y1 = layer.ffn(x, ids, w)
    torch.cuda.synchronize()
    assert torch.equal(packed, before)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.all(sink == 0)
