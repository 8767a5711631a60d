"""The no-allocation entry point (moe_fp4_moe_forward_noalloc, workspace in a static device
array of the library) against moe_fp4_moe_forward on a caller-owned workspace: the same
kernels on the same workspace layout, so the results must be bit-identical. Two calls in a
row on the shared array, the second with a smaller input (and another path), then a call
too large for the array, which must be refused with nothing enqueued."""

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import moe_inputs as S
from tests.gpu_helpers import check_ffn, check_route, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_noalloc_forward_matches_workspace_forward():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C

    C.lib()
    dev = torch.device("cuda:0")
    wl = S.small_workload(512, 384, 12, 6, 1, wid=980)
    packed = D.upload_experts(S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter, dev)
    wr_bits = S.router_weights(wl, 0)
    wr = D.upload_bf16(wr_bits, dev)
    layer = D.MoeFp4Layer(packed, wl.n_experts, wl.hidden, wl.inter, wl.k, wr)
    H, E, k, I = wl.hidden, wl.n_experts, wl.k, wl.inter
    # 40 tokens (grouped path), then 1 (the one-launch route and the decode kernels), then 5
    # (small-M), then 1 again: each call reuses the array the previous one left
    for step, T in enumerate((40, 1, 5, 1)):
        x_bits = S.activations(wl, 0, 50 + step, tokens=T)
        x = D.upload_bf16(x_bits, dev)
        y_ref, ids_ref, w_ref = layer.forward_fused(x)
        ids = torch.full((T, k), -7, dtype=torch.int32, device=dev)
        w = torch.full((T, k), -7.0, dtype=torch.float32, device=dev)
        y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=dev)
        C.moe_fp4_moe_forward_noalloc(x, wr, T, H, E, k, packed, I, ids, w, y)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref) and torch.equal(w, w_ref), (step, T)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (step, T)
        io, wo, _ = O.route(x_bits, wr_bits, k)
        check_route(ids.cpu().numpy(), w.cpu().numpy(), io, wo, f"noalloc T={T}")
        ref = O.expert_ffn(x_bits, io, wo, S.expert_source(wl), E, H, I)
        check_ffn(D.bf16_bits(y), ref, f"noalloc T={T}")
    # a problem larger than the static array: refused before anything is enqueued
    big = S.small_workload(4096, 2880, 384, 6, 1, wid=981)
    T = 200
    assert C.moe_fp4_moe_forward_workspace_bytes(T, 6, 384, 4096, 2880) > C.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, 4096), dtype=torch.bfloat16, device=dev)
    wr_big = torch.zeros((384, 4096), dtype=torch.bfloat16, device=dev)
    ids = torch.full((T, 6), -7, dtype=torch.int32, device=dev)
    w = torch.zeros((T, 6), dtype=torch.float32, device=dev)
    y = torch.zeros((T, 4096), dtype=torch.bfloat16, device=dev)
    with pytest.raises(C.MoeFp4Error) as err:
        C.moe_fp4_moe_forward_noalloc(x, wr_big, T, 4096, 384, 6, packed, 2880, ids, w, y)
    assert err.value.status == C.ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.all(ids == -7)
    del big
    log("noalloc forward: bit-identical to the workspace forward at T = 40, 1, 5, 1; "
        "T = 200 at full size refused")
