"""Full-size parity of the 16-layer batch-1 decode stack (16 MoE layers of 384 experts,
hidden 4096, intermediate 2880, top-6; about 116 GB of packed FP4 experts resident in HBM),
run exactly as the bench runs it: layer 0 through moe_fp4_moe_forward, every later layer
through moe_fp4_route_residual (residual + RMSNorm fused into the router kernel) and
moe_fp4_expert_ffn, then the last residual + RMSNorm.

Teacher-forced against the oracle: every layer of tokens 0, 1, 28, 29, 500 and 999 is
checked on the GPU's own input to that layer (ids bit-exact, weights within 2^-22, the FFN
within the normwise / cosine bar, the residual exactly and the normalised input within one
bf16 ulp), so a rounding-level difference in one layer cannot legitimately flip a route
later. The experts are drawn on the device by the workload's counter-based generator; the
oracle receives each expert it needs as the canonical blob, regenerated with the same
generator and copied to the host.
"""

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import moe_inputs as S
from tests.gpu_helpers import check_ffn, check_route, log, oracle_ffn_parallel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOKENS = (0, 1, 28, 29, 500, 999)
EPS = 1e-6


@pytest.mark.timeout(1200)
def test_stack16_teacher_forced_full_size():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C

    C.lib()
    dev = torch.device("cuda:0")
    wl = S.WORKLOADS["stack16_decode"]
    H, I, E, k, L = wl.hidden, wl.inter, wl.n_experts, wl.k, wl.layers
    stride = C.moe_fp4_packed_expert_stride(H, I)
    log(f"generating and packing {L} x {E} experts on the device")
    layers = []
    for l in range(L):
        packed = torch.empty(stride * E, dtype=torch.uint8, device=dev)
        for e0 in range(0, E, S.STACK_CHUNK):
            e1 = min(E, e0 + S.STACK_CHUNK)
            codes, scales = S.device_expert_blobs(wl, l, e0, e1, dev)
            C.moe_fp4_pack(codes, scales, e1 - e0, H, I, packed.data_ptr() + e0 * stride,
                           (e1 - e0) * stride)
            del codes, scales
        layers.append(D.MoeFp4Layer(packed, E, H, I, k, D.upload_bf16(S.router_weights(wl, l), dev)))
    torch.cuda.synchronize()
    ws = layers[0]._forward_workspace(1)
    for lay in layers:
        lay._fws = ws
    log("stack resident; running the teacher-forced tokens")

    # GPU pass: per token and layer, the layer's input (x, residual before its update),
    # routing and output, exactly in the bench's call sequence
    rec = {}
    r = torch.empty((1, H), dtype=torch.float32, device=dev)
    r2 = torch.empty_like(r)
    xa = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    xb = torch.empty_like(xa)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    for t in TOKENS:
        x = D.upload_bf16(S.activations(wl, 0, t), dev)
        C.moe_fp4_residual_init(x, r, 1, H)
        rc, rn = r, r2
        for l, lay in enumerate(layers):
            r_prev = rc.cpu().numpy().astype(np.float64)
            y_prev = D.bf16_bits(y)
            ids = torch.empty((1, k), dtype=torch.int32, device=dev)
            w = torch.empty((1, k), dtype=torch.float32, device=dev)
            if l == 0:
                lay.forward_fused(x, ids, w, y)
                xin, r_now = x, rc
            else:
                xn = xa if l % 2 == 0 else xb
                lay.route_residual(rc, y, rn, xn, EPS, ids, w)
                lay.ffn(xn, ids, w, y)
                xin, r_now = xn, rn
                rc, rn = rn, rc
            torch.cuda.synchronize()
            rec[(t, l)] = dict(x=D.bf16_bits(xin), r_prev=r_prev, y_prev=y_prev,
                               r=r_now.cpu().numpy(), ids=ids.cpu().numpy(), w=w.cpu().numpy(),
                               y=D.bf16_bits(y))

    # oracle, layer by layer (the experts a layer's tokens chose, regenerated on the device)
    worst_err, worst_cos = 0.0, 1.0
    for l in range(L):
        x_l = np.concatenate([rec[(t, l)]["x"] for t in TOKENS])
        ids_ref, w_ref, _ = O.route(x_l, S.router_weights(wl, l), k)
        for i, t in enumerate(TOKENS):
            g = rec[(t, l)]
            check_route(g["ids"], g["w"], ids_ref[i:i + 1], w_ref[i:i + 1], f"token {t} layer {l}")
            if l > 0:  # the fused residual + RMSNorm that produced this layer's input
                r_ref, x_ref = O.residual_rmsnorm(g["r_prev"], O.bf16_to_f64(g["y_prev"]), EPS)
                assert np.array_equal(g["r"], r_ref.astype(np.float32)), (t, l)
                xg, xr = O.bf16_to_f64(g["x"]), O.bf16_to_f64(x_ref)
                assert np.all(np.abs(xg - xr) <= np.abs(xr) * 2.0 ** -7 + 1e-30), (t, l)
        blobs = {}
        need = sorted(set(int(e) for e in ids_ref.ravel()))
        for e0 in sorted(set(e // S.STACK_CHUNK * S.STACK_CHUNK for e in need)):
            codes, scales = S.device_expert_blobs(wl, l, e0, min(E, e0 + S.STACK_CHUNK), dev)
            for e in need:
                if e0 <= e < e0 + S.STACK_CHUNK:
                    blobs[e] = (codes[e - e0].cpu().numpy(), scales[e - e0].cpu().numpy())
            del codes, scales
        ref = oracle_ffn_parallel(x_l, ids_ref, w_ref, lambda e: blobs[e], E, H, I)
        y_l = np.concatenate([rec[(t, l)]["y"] for t in TOKENS])
        err, cos = check_ffn(y_l, ref, f"layer {l}")
        worst_err, worst_cos = max(worst_err, err), min(worst_cos, cos)
        del blobs
        if l % 4 == 3:
            log(f"layers 0..{l}: ids bit-exact, norm within 1 ulp, worst normwise {worst_err:.2e} "
                f"cosine {worst_cos:.7f}")
    del layers, ws
    torch.cuda.empty_cache()
