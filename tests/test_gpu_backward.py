"""GPU parity of the backward (training path) through the C ABI against the CPU float64 oracle
(oracle/train.py).

Bar: every gradient (dQ, dK, dV, dalpha) within relative L2 1e-2 of the oracle's (relative to
the larger of the reference's norm and a tenth of dV's, since dQ and dK can vanish exactly).
The bound comes from the arithmetic: the kernels round dO_s = alpha dO, G = (1 - alpha) dO / den, P and dS to bf16
before their MFMAs (each a relative 2^-9 per value) on top of the forward's own bf16 rounding of
P and of the linear states, so a gradient carries a few times 2^-9 of relative error; 1e-2 leaves
a margin of about two over the measured values.  The recomputed forward returned with the
gradients equals the forward entry point's output bit for bit.  Small cases on every element;
the full-size workload on one whole head (dK and dV need every query block of the head).
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_linear_02_amd as sla
import gen
import oracle

pytestmark = pytest.mark.gpu

TOL_REL = 1e-2


def say(msg):
    print(f"[gpu-bwd] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sla.lib()


def draw(wl, seed=0):
    c = gen.draw(wl, seed)
    rng = np.random.default_rng(seed + 77)
    c["dO"] = torch.from_numpy(rng.standard_normal(c["Q"].shape).astype(np.float32)).to(torch.bfloat16)
    return c


def run(c, idx_np, heads=None, want_O=False):
    wl = c["workload"]
    d = torch.device("cuda:0")
    g = {k: c[k].to(d) for k in ("Q", "K", "V", "alpha", "dO")}
    idx = torch.from_numpy(np.ascontiguousarray(idx_np)).to(d)
    res = sla.backward(g["Q"], g["K"], g["V"], idx, g["alpha"], g["dO"], want_O=want_O)
    torch.cuda.synchronize()
    got = [x.cpu().double().numpy() for x in res[:4]]
    heads = range(wl.B * wl.H) if heads is None else heads
    worst = {}
    for bh in heads:
        b, h = divmod(bh, wl.H)
        ref = oracle.backward_head(c["Q"][b, h], c["K"][b, h], c["V"][b, h], idx_np[b, h], c["alpha"][b, h],
                                   c["dO"][b, h], 64)
        # relative to the larger of the reference and a tenth of dV's norm: dQ and dK vanish
        # identically in degenerate cases (a single token: a one-key softmax has no gradient)
        floor = 0.1 * np.linalg.norm(ref[2])
        for name, gv, rv in zip(("dQ", "dK", "dV", "dalpha"), got, ref):
            gg = gv[b, h]
            assert np.all(np.isfinite(gg)), f"{name}: non-finite"
            err = float(np.linalg.norm(gg - rv) / max(np.linalg.norm(rv), floor, 1e-300))
            worst[name] = max(worst.get(name, 0.0), err)
    say(f"{wl.name}: " + ", ".join(f"{k} rel-L2 {v:.2e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= TOL_REL, f"{k}: relative L2 error {v}"
    return res


def small(k=6, **kw):
    return gen.workload("video_l").with_(name=f"bwd_ragged_k{k}", H=2, N=3600, grid=(1, 45, 80), topk=k, **kw)


def route_idx(c, k):
    return oracle.route(c["Q"], c["K"], c["Wq"].double(), c["Wk"].double(), k, 64)["idx"]


@pytest.mark.parametrize("k", [6, 0, 1, 57])
def test_backward_small(k):
    """57 query and key blocks with a 16-token tail: k = 6, nothing kept (linear branch only),
    one block kept, and every block kept (sparse branch only)."""
    c = draw(small(k))
    run(c, route_idx(c, k))


def test_backward_returns_the_forward():
    c = draw(small(6))
    idx_np = route_idx(c, 6)
    res = run(c, idx_np, want_O=True)
    d = torch.device("cuda:0")
    O = sla.forward(*(c[k].to(d) for k in ("Q", "K", "V")), torch.from_numpy(idx_np).to(d), c["alpha"].to(d),
                    linear_mode="mask_product")
    torch.cuda.synchronize()
    assert torch.equal(res[4], O)


EDGE = [
    gen.workload("tiny").with_(name="bwd_n1", B=1, H=1, N=1, d=128, dtype="bf16", topk=1, wid=8),
    gen.workload("tiny").with_(name="bwd_n65_k0", B=1, H=2, N=65, d=128, dtype="bf16", topk=0, wid=8),
    gen.workload("tiny").with_(name="bwd_n65_k1", B=1, H=2, N=65, d=128, dtype="bf16", topk=1, wid=8),
    gen.workload("tiny").with_(name="bwd_n200_k2", B=2, H=3, N=200, d=128, dtype="bf16", topk=2, wid=8),
    gen.workload("tiny").with_(name="bwd_n4097_k33", B=1, H=1, N=4097, d=128, dtype="bf16", topk=33, wid=8),
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_backward_edge_shapes(wl):
    """One token, a one-token tail block, odd n_b with batch > 1, 65 blocks with half kept."""
    c = draw(wl)
    run(c, route_idx(c, wl.topk))


def test_backward_random_alpha_extremes():
    """alpha exactly 0 and 1 on some rows (one branch carries all the gradient there)."""
    c = draw(small(6))
    a = c["alpha"].clone()
    a[:, :, ::7] = 0.0
    a[:, :, 3::7] = 1.0
    c["alpha"] = a
    run(c, route_idx(c, 6))


def test_backward_video_s_head():
    """video_s (N=32768, H=12, k=51): the whole of head 5 against the oracle."""
    c = draw(gen.workload("video_s"))
    run(c, route_idx(c, 51), heads=[5])
