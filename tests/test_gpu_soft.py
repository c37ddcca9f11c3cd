"""GPU parity of the SoftTop-k training path (include/sla_soft.h) against the CPU float64 oracle
(oracle/soft.py): the soft router, the soft-mask forward, its gradients with respect to the
mask, alpha and the router projections, and stage-1 steps.

Bars.  The mask: the GPU forms the scores in fp32 from fp32 block means and bisects tau in fp32,
so M sits within about 1e-6 / T of the oracle's; max-abs 1e-4 at T >= 0.05.  The forward: the
bf16 bars of the hard forward (max-abs 1e-2, relative L2 5e-3).  The gradients come from bf16
operands (dO_s, G, the states h_j and dA_i, each rounded once: about 2^-9 relative) summed in
fp32: relative L2 2e-2 for dM and the projection gradients, 5e-3 for dalpha (a product of fp32
rows).  A plausible mistake (a sign, a transposed operand, a dropped term) moves these by O(1).
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_linear_02_amd as sla
import gen
import oracle
from tests import cases

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-soft] {msg}", flush=True)
    sys.stdout.flush()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sla.lib()


_CACHE = {}


def small(H=2, N=1800, k=5):
    """Clustered video-shaped inputs: 1800 tokens (a 1 x 45 x 40 latent slice), 29 blocks with a
    8-token last block."""
    key = (H, N, k)
    if key not in _CACHE:
        wl = gen.workload("video_l", H=H, N=N, grid=(1, 45, 40), topk=k).with_(name=f"soft_{H}_{N}_{k}", wid=9)
        _CACHE[key] = cases.make_case(wl, gap=False)
    return _CACHE[key]


def dev(c):
    d = torch.device("cuda:0")
    return {n: c[n].to(d) for n in ("Q", "K", "V", "alpha", "Wq", "Wk")}


@pytest.mark.parametrize("k,T", [(5, 0.5), (5, 0.05), (0, 0.5), (29, 0.5), (1, 0.2)])
def test_soft_route(k, T):
    c = small()
    g = dev(c)
    say(f"soft route k={k} T={T}")
    M = sla.soft_route(g["Q"], g["K"], g["Wq"], g["Wk"], k, T)
    torch.cuda.synchronize()
    ref = oracle.soft_route(c["Q"], c["K"], c["Wq"].double(), c["Wk"].double(), k, T, 64)["M"]
    got = M.cpu().double().numpy()
    err = float(np.abs(got - ref).max())
    say(f"  max|dM| {err:.3e}, row sums {got.sum(-1).min():.4f} .. {got.sum(-1).max():.4f}")
    assert err <= 1e-4
    np.testing.assert_allclose(got.sum(-1), k, rtol=0, atol=2e-3)


def test_soft_forward_matches_oracle():
    c = small()
    g = dev(c)
    M = sla.soft_route(g["Q"], g["K"], g["Wq"], g["Wk"], 5, 0.3)
    say("soft forward")
    O = sla.soft_forward(g["Q"], g["K"], g["V"], M, g["alpha"])
    torch.cuda.synchronize()
    ref, _, _ = oracle.forward_soft(c["Q"], c["K"], c["V"], M.cpu().double().numpy(), c["alpha"], 64)
    got = O.cpu().double().numpy()
    err, rel = float(np.abs(got - ref).max()), rel_l2(got, ref)
    say(f"  max|dO| {err:.3e} rel-L2 {rel:.3e}")
    assert np.all(np.isfinite(got)) and err <= 1e-2 and rel <= 5e-3


def test_soft_forward_binary_mask_is_hard_forward():
    """A 0/1 mask through the soft forward gives the hard forward of the kept sets it encodes (the
    oracle's, at the hard forward's bars: the soft kernel walks every key block, so its running
    maximum, and with it the bf16 rounding of P, can differ from the hard kernel's)."""
    c = small()
    g = dev(c)
    k = 5
    idx, mask, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], k, want_mask=True)
    say("soft forward on a binary mask")
    Os = sla.soft_forward(g["Q"], g["K"], g["V"], mask.to(torch.float32), g["alpha"])
    torch.cuda.synchronize()
    ref, _, _ = oracle.forward(c["Q"], c["K"], c["V"], idx.cpu().numpy(), c["alpha"], 64)
    got = Os.cpu().double().numpy()
    err, rel = float(np.abs(got - ref).max()), rel_l2(got, ref)
    say(f"  against the oracle's hard forward: max|dO| {err:.3e} rel-L2 {rel:.3e}")
    assert err <= 1e-2 and rel <= 5e-3


def test_soft_backward_matches_oracle():
    c = small()
    g = dev(c)
    k, T = 5, 0.3
    M = sla.soft_route(g["Q"], g["K"], g["Wq"], g["Wk"], k, T)
    gen_ = torch.Generator().manual_seed(11)
    dO = torch.randn(c["Q"].shape, generator=gen_).to(torch.bfloat16)
    say("soft backward")
    dWq, dWk, da, dM = sla.soft_backward(g["Q"], g["K"], g["V"], g["Wq"], g["Wk"], T, M, g["alpha"],
                                         dO.to(g["Q"].device), k)
    torch.cuda.synchronize()
    Mn = M.cpu().double().numpy()
    dM_ref, da_ref = oracle.backward_soft(c["Q"], c["K"], c["V"], Mn, c["alpha"], dO, 64)
    r = oracle.soft_route(c["Q"], c["K"], c["Wq"].double(), c["Wk"].double(), k, T, 64)
    ds = oracle.soft_topk_backward(Mn, dM_ref, T, k)
    dWq_ref, dWk_ref = oracle.router_backward(r["qbar"], r["kbar"], r["qt"], r["kt"], ds)
    res = {"dM": rel_l2(dM.cpu().numpy(), dM_ref), "dalpha": rel_l2(da.cpu().numpy(), da_ref),
           "dWq": rel_l2(dWq.cpu().numpy(), dWq_ref), "dWk": rel_l2(dWk.cpu().numpy(), dWk_ref)}
    say(f"  rel-L2 {res}")
    assert res["dM"] <= 2e-2 and res["dWq"] <= 2e-2 and res["dWk"] <= 2e-2 and res["dalpha"] <= 5e-3


def test_stage1_steps():
    """One step against the oracle's loss and update, then ten more: the loss goes down."""
    c = small()
    g = dev(c)
    k, T, lr, lra = 5, 0.3, 10.0, 1000.0
    H, N = c["Q"].shape[1], c["Q"].shape[2]
    nb = -(-N // 64)
    # O_full on the GPU: every block kept, alpha = 1
    idx_all = torch.arange(nb, dtype=torch.int32, device=g["Q"].device).expand(1, H, nb, nb).contiguous()
    O_full = sla.forward(g["Q"], g["K"], g["V"], idx_all, torch.ones_like(g["alpha"]), linear_mode="mask_product")
    Wq, Wk, alpha = g["Wq"].clone(), g["Wk"].clone(), g["alpha"].clone()
    say("stage-1 step 0")
    loss0 = sla.stage1_step(g["Q"], g["K"], g["V"], O_full, Wq, Wk, alpha, k, T, lr, lra)
    torch.cuda.synchronize()
    Ofn = O_full.cpu().double().numpy()
    ref = oracle.stage1_grads(c["Q"], c["K"], c["V"], c["Wq"].double(), c["Wk"].double(), c["alpha"], k, T, Ofn, 64)
    l0 = float(loss0.item())
    say(f"  loss {l0:.6e} oracle {ref['loss']:.6e}")
    assert abs(l0 - ref["loss"]) <= 5e-3 * ref["loss"]
    dWq_gpu = (g["Wq"] - Wq).cpu().double().numpy() / lr
    dWk_gpu = (g["Wk"] - Wk).cpu().double().numpy() / lr
    rq, rk = rel_l2(dWq_gpu, ref["dWq"]), rel_l2(dWk_gpu, ref["dWk"])
    a_ref = np.clip(c["alpha"].double().numpy() - lra * ref["dalpha"], 0.0, 1.0)
    ra = rel_l2(alpha.cpu().double().numpy() - c["alpha"].double().numpy(), a_ref - c["alpha"].double().numpy())
    say(f"  update rel-L2: dWq {rq:.3e} dWk {rk:.3e} alpha step {ra:.3e}")
    assert rq <= 2e-2 and rk <= 2e-2 and ra <= 2e-2
    losses = [l0]
    for _ in range(10):
        losses.append(float(sla.stage1_step(g["Q"], g["K"], g["V"], O_full, Wq, Wk, alpha, k, T, lr, lra).item()))
    say(f"  losses {['%.4e' % x for x in losses]}")
    assert losses[-1] < losses[0]
