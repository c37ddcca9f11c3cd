"""Route + forward captured in a HIP graph (through torch.cuda.CUDAGraph on the library's stream
argument): every replay, with the program's own eager work and synchronisations between replays,
gives the eager call's index lists and output bit for bit.  The library enqueues kernels only
(no memset, copy or host wait outside its debug check), which is what makes a step capturable."""

import pytest
import torch

import block_sparse_linear_02_amd as sla
import gen
from tests import cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sla.lib()
    wl = gen.workload("video_l", H=2, N=3600, grid=(1, 45, 80), topk=6).with_(name="graph", wid=11)
    c = cases.make_case(wl, gap=False)
    d = torch.device("cuda:0")
    return wl, {n: c[n].to(d).contiguous() for n in ("Q", "K", "V", "alpha", "Wq", "Wk")}


@pytest.mark.parametrize("mode", ["mask_product", "fused"])
def test_graph_replays_match_eager(case, mode):
    wl, g = case
    Q, K, V, alpha, Wq, Wk = (g[n] for n in ("Q", "K", "V", "alpha", "Wq", "Wk"))
    B, H, N, d = Q.shape
    nb, k = wl.n_blocks, wl.topk
    variant = {"fused": 0, "mask_product": 3}[mode]
    ws_r = torch.empty(sla.route_workspace_bytes(Q, k), dtype=torch.uint8, device=Q.device)
    ws_f = torch.empty(sla.forward_workspace_bytes(Q, k, variant), dtype=torch.uint8, device=Q.device)
    idx = torch.empty((B, H, nb, k), dtype=torch.int32, device=Q.device)
    O = torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device)

    def step():
        sla.route(Q, K, Wq, Wk, k, workspace=ws_r, idx_out=idx)
        sla.forward(Q, K, V, idx, alpha, linear_mode=mode, workspace=ws_f, out=O)

    step()
    torch.cuda.synchronize()
    idx_e, O_e = idx.clone(), O.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream, as torch asks before a capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    other_alpha = torch.rand_like(alpha)
    for r in range(4):
        idx.fill_(-1)
        O.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_e), f"replay {r}: idx differs"
        assert torch.equal(O, O_e), f"replay {r}: O differs"
        # eager work between replays, on other outputs
        sla.forward(Q, K, V, idx_e, other_alpha, linear_mode=mode)
        torch.cuda.synchronize()
