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
