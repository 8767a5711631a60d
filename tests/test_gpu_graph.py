"""Graph replay of whole layer calls, the way the bench times them. Every replay must give the
eager results bit for bit, with eager calls on the same workspace between the replays: the
batch-1 route carries synchronisation words from call to call in its workspace, and no
kernel may depend on a value frozen at capture time. One token runs the decode kernels, four
the small-M kernels, 64 the grouped GEMM path."""

import numpy as np
import pytest

from synth import moe_inputs as S

from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C
    C.lib()
    dev = torch.device("cuda:0")
    wl = S.small_workload(512, 256, 16, 4, 64, wid=910)
    packed = D.upload_experts(S.expert_source(wl), wl.n_experts, wl.hidden, wl.inter, dev)
    wr = D.upload_bf16(S.router_weights(wl, 0), dev)
    return D, D.MoeFp4Layer(packed, wl.n_experts, wl.hidden, wl.inter, wl.k, wr), wl


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().copy()


@pytest.mark.parametrize("T", [1, 4, 64])
def test_graph_replays_match_eager(layer, T):
    D, L, wl = layer
    dev = L.device
    n = 3  # layer calls per graph, each on its own tokens
    xs = [D.upload_bf16(S.activations(wl, 0, 10 + i, tokens=T), dev) for i in range(n)]
    eager = []
    for x in xs:
        y, ids, w = L.forward_fused(x)
        torch.cuda.synchronize()
        eager.append((_bits(y), ids.cpu().numpy().copy(), w.cpu().numpy().copy()))

    ids_g = [torch.empty((T, L.k), dtype=torch.int32, device=dev) for _ in range(n)]
    w_g = [torch.empty((T, L.k), dtype=torch.float32, device=dev) for _ in range(n)]
    y_g = [torch.empty((T, L.hidden), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    for i in range(n):  # workspaces exist before the capture
        L.forward_fused(xs[i], ids_g[i], w_g[i], y_g[i])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(n):
            L.forward_fused(xs[i], ids_g[i], w_g[i], y_g[i])
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: clobber the outputs, and one more eager layer call on the
        # same workspace (it advances the batch-1 route's epoch)
        for i in range(n):
            y_g[i].zero_()
            ids_g[i].fill_(-7)
            w_g[i].fill_(-1.0)
        L.forward_fused(xs[(rep + 1) % n])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(n):
            y_e, ids_e, w_e = eager[i]
            assert np.array_equal(ids_g[i].cpu().numpy(), ids_e), f"T={T} replay {rep} call {i}: ids"
            assert np.array_equal(w_g[i].cpu().numpy().view(np.uint32), w_e.view(np.uint32)), \
                f"T={T} replay {rep} call {i}: weights"
            assert np.array_equal(_bits(y_g[i]), y_e), f"T={T} replay {rep} call {i}: y"
    log(f"graph T={T}: 3 replays x {n} layer calls bit-identical to eager")


def test_graph_replays_layer_stack(layer):
    """Three layers at batch 1 as the 16-layer decode workload chains them: the first routes
    its input, the later ones route straight from the residual stream (residual add, RMSNorm
    and route in one launch), all on one route workspace."""
    D, L, wl = layer
    from fp4_expert_ffn_amd import moe_fp4 as C
    dev = L.device
    H, k, n = L.hidden, L.k, 3
    x0 = D.upload_bf16(S.activations(wl, 0, 40, tokens=1), dev)
    r = [torch.empty((1, H), dtype=torch.float32, device=dev) for _ in range(n)]
    xl = [x0] + [torch.empty((1, H), dtype=torch.bfloat16, device=dev) for _ in range(n - 1)]
    y = [torch.empty((1, H), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    ids = [torch.empty((1, k), dtype=torch.int32, device=dev) for _ in range(n)]
    w = [torch.empty((1, k), dtype=torch.float32, device=dev) for _ in range(n)]

    def stack():
        C.moe_fp4_residual_init(x0, r[0], 1, H)
        L.route(x0, ids[0], w[0])
        L.ffn(x0, ids[0], w[0], y[0])
        for l in range(1, n):
            L.route_residual(r[l - 1], y[l - 1], r[l], xl[l], ids=ids[l], w=w[l])
            L.ffn(xl[l], ids[l], w[l], y[l])

    stack()
    torch.cuda.synchronize()
    ref = [(_bits(y[l]), ids[l].cpu().numpy().copy(), _bits(xl[l])) for l in range(n)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        stack()
    torch.cuda.synchronize()
    for rep in range(3):
        for l in range(n):
            y[l].zero_()
            ids[l].fill_(-7)
        L.route(x0)  # an eager call on the same route workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(n):
            assert np.array_equal(ids[l].cpu().numpy(), ref[l][1]), f"replay {rep} layer {l}: ids"
            assert np.array_equal(_bits(xl[l]), ref[l][2]), f"replay {rep} layer {l}: x"
            assert np.array_equal(_bits(y[l]), ref[l][0]), f"replay {rep} layer {l}: y"
    log("graph: 3-layer residual stack, 3 replays bit-identical to eager")


def test_graph_replays_fp8_shared_expert():
    """The FP8 shared expert's two launches, captured and replayed."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_expert_ffn_amd import moe_fp4 as C
    C.lib()
    dev = torch.device("cuda:0")
    H, I, T = 512, 384, 2

    def pack(rows, cols, seed):
        codes, scales = S.fp8_matrix(rows, cols, seed=seed)
        c = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
        sc = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).to(dev)
        nb = C.moe_fp4_fp8_packed_bytes(rows, cols)
        p = torch.empty(nb, dtype=torch.uint8, device=dev)
        C.moe_fp4_fp8_pack(c, sc, rows, cols, p, nb)
        return p

    pg, pu, pd = pack(I, H, 21), pack(I, H, 22), pack(H, I, 23)
    x = torch.randn((T, H), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    wsb = C.moe_fp4_shared_expert_workspace_bytes(T, I)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    C.moe_fp4_shared_expert(x, T, pg, pu, pd, H, I, y, ws, wsb)
    torch.cuda.synchronize()
    ref = _bits(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        C.moe_fp4_shared_expert(x, T, pg, pu, pd, H, I, y, ws, wsb)
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), ref), f"replay {rep}"
