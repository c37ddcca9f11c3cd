"""GPU parity of the PISA path (statistics, covariance-aware routing, forward) through the C ABI,
against the CPU float64 oracle (oracle/pisa.py).

Bars:
* statistics: centroids (bf16 hi + lo) within 2e-5 relative of the oracle's, value sums within
  bf16 rounding, Hbar and M_j within 1e-4 (bf16 inputs, exact products, fp32 sums) or 1e-2
  (fp32 inputs: bf16 MFMA operands) in L2, relative to the larger of the reference and the size
  of the summed terms sum |k||v| (either can be exactly 0, e.g. for a single token);
* routing: the ranked scores within 1e-4 (1 + |s|) of the oracle's; the kept set is exactly the
  HardTop-k of the kernel's own fp32 scores (ties to the lower index, ascending), i.e. the
  integer decision is taken in the kernel's precision and compared bit for bit; against the
  oracle's float64 ranking the kept set is identical on every row whose k-th/(k+1)-th score gap
  exceeds twice the largest measured score error, and on the other rows a valid top-k within
  that margin;
* forward: O within max-abs 1e-2 and relative L2 5e-3 of the oracle evaluated with the same
  kept set.
Small cases are compared on every element; the full-size workloads (the ones the benchmark
times) on every router row and statistic of sampled heads and on sampled query blocks.
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_linear_02_amd as sla
import gen
import oracle

pytestmark = pytest.mark.gpu

TOL_MAX = 1e-2
TOL_REL = 5e-3
SCORE_TOL = 1e-4


def say(msg):
    print(f"[gpu-pisa] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sla.lib()


_CACHE = {}


def case(wl):
    if wl.name not in _CACHE:
        say(f"generating {wl}")
        c = gen.draw(wl, seed=0)
        d = torch.device("cuda:0")
        c["g"] = {k: c[k].to(d) for k in ("Q", "K", "V")}
        _CACHE.clear()  # one case at a time keeps host and device memory bounded
        _CACHE[wl.name] = c
    return _CACHE[wl.name]


def small_ragged(H=2, k=6, **kw):
    return gen.workload("pisa_video_s").with_(name=f"pisa_ragged_k{k}", H=H, N=3600, grid=(1, 45, 80),
                                              topk=k, **kw)  # 57 blocks, a 16-token tail


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def check_close(got, ref, rel_tol=TOL_REL, max_tol=TOL_MAX, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    rel = rel_l2(got, ref) if got.size else 0.0
    say(f"{what}: max|d| {err:.3e}  rel-L2 {rel:.3e}")
    if max_tol is not None:
        assert err <= max_tol, f"{what}: max abs error {err}"
    assert rel <= rel_tol, f"{what}: relative L2 error {rel}"


def f64(t):
    return t.detach().cpu().to(torch.float32).double().numpy()


def check_stats(c, st, heads, what):
    """Statistics of the listed heads (flattened b * H + h) against the oracle."""
    wl = c["workload"]
    tol = 1e-4 if wl.dtype == "bf16" else 1e-2
    kbar = f64(st.kbar_hi) + f64(st.kbar_lo)
    vsum, hbar, M = f64(st.vsum), f64(st.hbar), f64(st.M)
    hbar_t = f64(st.hbar_t)
    lnM = f64(st.lnM)
    for bh in heads:
        b, h = divmod(bh, wl.H)
        ref = oracle.pisa_block_stats(c["K"][b, h], c["V"][b, h], 64)
        Mr = oracle.pisa_cov_norms(ref["H"], ref["Hbar"])
        cs = 1.0 + np.abs(ref["centroid"]).max()
        err = np.abs(kbar[b, h] - ref["centroid"]).max()
        assert err <= 2e-5 * cs, f"{what} head {bh}: centroid error {err}"
        verr = np.abs(vsum[b, h] - ref["vsum"]) - (2.0 ** -8) * np.abs(ref["vsum"])
        assert verr.max() <= 1e-4 * (1.0 + np.abs(ref["vsum"]).max()), f"{what} head {bh}: value sums"
        # errors relative to the size of the summed terms |k||v| (Hbar and M can be 0 exactly,
        # e.g. a single token, while the GPU's sums carry rounding of that size)
        Kh, Vh = f64(c["K"][b, h]), f64(c["V"][b, h])
        nb = ref["H"].shape[0]
        blk_abs = np.array([np.linalg.norm(np.abs(Kh[j * 64 : (j + 1) * 64]).T @ np.abs(Vh[j * 64 : (j + 1) * 64]))
                            for j in range(nb)])
        rh = float(np.linalg.norm(hbar[b, h] - ref["Hbar"]) / max(np.linalg.norm(ref["Hbar"]), blk_abs.mean()))
        rm = float(np.linalg.norm(M[b, h] - Mr) / max(np.linalg.norm(Mr), np.linalg.norm(blk_abs) / np.sqrt(nb)))
        say(f"{what} head {bh}: centroid {err:.2e}, Hbar rel {rh:.2e}, M rel {rm:.2e}")
        assert rh <= tol, f"{what} head {bh}: Hbar rel-L2 {rh}"
        assert rm <= tol, f"{what} head {bh}: M rel-L2 {rm}"
        # Hbar^T is the bf16 rounding of the transpose of the fp32 Hbar
        assert np.abs(hbar_t[b, h] - hbar[b, h].T).max() <= 2.0 ** -8 * np.abs(hbar[b, h]).max() + 1e-30
        fin = M[b, h] > 0
        assert np.all(np.isneginf(lnM[b, h][~fin]))
        np.testing.assert_allclose(lnM[b, h][fin], np.log(M[b, h][fin]), rtol=0, atol=1e-5)


def check_route(c, st, k, covariance, heads, what):
    """Route every row of the listed heads; returns the GPU idx (numpy, all heads)."""
    wl = c["workload"]
    g = c["g"]
    idx, mask, scores = sla.pisa_route(g["Q"], st, k, covariance=covariance, want_mask=True, want_scores=True)
    torch.cuda.synchronize()
    idx_np, mask_np, sc = idx.cpu().numpy(), mask.cpu().numpy(), scores.cpu().double().numpy()
    nb = wl.n_blocks
    assert idx_np.shape == (wl.B, wl.H, nb, k)
    worst, band = 0.0, 0
    for bh in heads:
        b, h = divmod(bh, wl.H)
        r = oracle.pisa_route(c["Q"][b, h], c["K"][b, h], c["V"][b, h], k, 64, covariance=covariance)
        ref = r["select"]
        got = sc[b, h]
        assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
        fin = np.isfinite(ref)
        diff = np.abs(got[fin] - ref[fin])
        worst = max(worst, float(diff.max()) if diff.size else 0.0)
        assert np.all(diff <= SCORE_TOL * (1.0 + np.abs(ref[fin]))), f"{what}: score error {diff.max()}"
        # the kept set is the HardTop-k of the kernel's own scores, bit for bit
        own, own_mask = oracle.hard_topk(got, k)
        assert np.array_equal(idx_np[b, h], own), f"{what}: idx is not the top-k of the kernel's scores"
        assert np.array_equal(mask_np[b, h], own_mask), f"{what}: mask differs from idx"
        # against the float64 ranking: a top-k of scores within e of the oracle's is a top-k of
        # the oracle's within 2e, so the kept set must be identical wherever the k-th/(k+1)-th
        # gap exceeds 2e (e = this head's largest score error) and a valid top-k within 2e
        # elsewhere
        if 0 < k < nb:
            srt = -np.sort(-np.where(np.isneginf(ref), -1e300, ref), axis=1)
            kth, nxt = srt[:, k - 1], srt[:, k]
            e = float(diff.max()) if diff.size else 0.0
            eps = np.full(nb, 2.0 * e * (1.0 + 1e-6) + 1e-12)
            clear = (kth - nxt) > eps
            band += int((~clear).sum())
            assert np.array_equal(idx_np[b, h][clear], r["idx"][clear]), f"{what}: idx differs on a clear row"
            rr = np.where(np.isneginf(ref), -1e300, ref)
            for i in np.flatnonzero(~clear):
                keep = np.zeros(nb, dtype=bool)
                keep[idx_np[b, h, i]] = True
                assert rr[i, keep].min() >= rr[i, ~keep].max() - eps[i], f"{what}: row {i} is no top-k"
        else:
            assert np.array_equal(idx_np[b, h], r["idx"])
    say(f"{what}: scores max|d| {worst:.2e}; {band} rows within the tolerance band")
    return idx, idx_np


def check_forward(c, st, idx, idx_np, heads, blocks, what):
    wl = c["workload"]
    g = c["g"]
    O = sla.pisa_forward(g["Q"], g["K"], g["V"], st, idx)
    torch.cuda.synchronize()
    got_O = O.cpu().double().numpy()
    assert np.all(np.isfinite(got_O)), f"{what}: non-finite output"
    gots, refs = [], []
    for bh in heads:
        b, h = divmod(bh, wl.H)
        o = oracle.pisa_forward_head(c["Q"][b, h], c["K"][b, h], c["V"][b, h], idx_np[b, h], 64,
                                     q_blocks=blocks)
        for i, oi in zip(blocks if blocks is not None else range(wl.n_blocks), o):
            refs.append(oi)
            gots.append(got_O[b, h, i * 64 : i * 64 + len(oi)])
    check_close(np.concatenate(gots), np.concatenate(refs), what=what)
    return got_O


def run_case(wl, covariance=True, heads=None, blocks=None, what=None):
    c = case(wl)
    g = c["g"]
    what = what or wl.name
    heads = list(range(wl.B * wl.H)) if heads is None else heads
    say(f"stats {what}")
    st = sla.pisa_stats(g["K"], g["V"])
    torch.cuda.synchronize()
    check_stats(c, st, heads, what)
    say(f"route {what} covariance={covariance}")
    idx, idx_np = check_route(c, st, wl.topk, covariance, heads, what)
    say(f"forward {what}")
    return c, st, idx, check_forward(c, st, idx, idx_np, heads, blocks, what)


# ---------------------------------------------------------------------------------- small


SMALL = [
    gen.workload("tiny").with_(name="pisa_tiny"),
    small_ragged(),
    small_ragged(k=9).with_(d=64, name="pisa_ragged_d64"),
    small_ragged(k=3).with_(dtype="fp32", name="pisa_ragged_fp32"),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("covariance", [True, False])
def test_pisa_small_every_element(wl, covariance):
    run_case(wl, covariance=covariance)


@pytest.mark.parametrize("k", [0, 1, 57])
def test_pisa_degenerate_k(k):
    """k = 0: every block approximated; k = n_b: exact softmax attention (the scan is skipped)."""
    c, _, _, got = run_case(small_ragged(k=k))
    if k == 57:
        q = c["Q"].double()
        ref = torch.nn.functional.scaled_dot_product_attention(q, c["K"].double(), c["V"].double()).numpy()
        check_close(got, ref, what="k = n_b against dense attention")


def test_pisa_deterministic():
    wl = small_ragged()
    c = case(wl)
    g = c["g"]
    outs = []
    for _ in range(2):
        st = sla.pisa_stats(g["K"], g["V"])
        idx, _, _ = sla.pisa_route(g["Q"], st, wl.topk)
        views = [getattr(st, n).clone() for n in sla.PisaStats._NAMES]  # not the alignment padding
        outs.append((views, idx.clone(), sla.pisa_forward(g["Q"], g["K"], g["V"], st, idx)))
    torch.cuda.synchronize()
    for a, b in zip(outs[0][0], outs[1][0]):
        assert torch.equal(a, b)
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])


def test_pisa_forward_with_foreign_index_lists():
    """The forward takes any ascending kept lists, e.g. the SLA2 router's."""
    wl = small_ragged(k=5)
    c = case(wl)
    g = c["g"]
    rng = np.random.default_rng(7)
    nb = wl.n_blocks
    idx_np = np.stack([[np.sort(rng.choice(nb, 5, replace=False)) for _ in range(nb)] for _ in range(wl.H)])[None]
    idx_np = idx_np.astype(np.int32)
    st = sla.pisa_stats(g["K"], g["V"])
    idx = torch.from_numpy(idx_np).to(g["Q"].device)
    check_forward(c, st, idx, idx_np, list(range(wl.H)), None, "random kept lists")


# ---------------------------------------------------------------------------------- edge shapes


def edge(name, B, H, N, d, dtype, k):
    return gen.workload("tiny").with_(name=f"pisa_edge_{name}", B=B, H=H, N=N, d=d, dtype=dtype, topk=k, wid=7)


EDGE = [
    edge("n1_d64_f32_k0", 1, 1, 1, 64, "fp32", 0),  # one token: M = 0, ln M = -inf
    edge("n1_d128_bf16_k1", 1, 2, 1, 128, "bf16", 1),
    edge("n65_d128_bf16_k0", 1, 2, 65, 128, "bf16", 0),  # a 1-token tail block
    edge("n65_d128_bf16_k1", 1, 2, 65, 128, "bf16", 1),
    edge("n65_d128_f32_k1", 1, 2, 65, 128, "fp32", 1),
    edge("n200_d128_bf16_k2", 2, 3, 200, 128, "bf16", 2),  # batch > 1, odd n_b, 8-token tail
    edge("n4097_d128_bf16_k33", 1, 1, 4097, 128, "bf16", 33),  # 65 blocks: two centroid tiles
    edge("n4097_d64_f32_k64", 1, 1, 4097, 64, "fp32", 64),  # only the 1-token tail approximated
    edge("n8191_d128_bf16_k7", 1, 2, 8191, 128, "bf16", 7),  # 128 blocks, 63-token tail
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_pisa_edge_shapes(wl):
    run_case(wl)


def test_pisa_most_blocks():
    """2048 key blocks (the largest supported n_b): the last word of the kept bitmaps and the
    32nd centroid tile."""
    wl = gen.workload("pisa_video_s").with_(name="pisa_2048", H=1, N=2048 * 64 - 5, grid=(32, 64, 64), topk=16)
    wl = wl.with_(grid=(1, 1, wl.N), kind="iid", dtype="bf16")
    run_case(wl, heads=[0], blocks=[0, 1, 1023, 2046, 2047])


# ---------------------------------------------------------------------------------- full size


def test_pisa_video_s_full_size():
    run_case(gen.workload("pisa_video_s"), heads=[0, 6, 11], blocks=[0, 1, 255, 511],
             what="pisa_video_s N=32768 H=12 k=64")


def test_pisa_video_l_full_size():
    run_case(gen.workload("pisa_video_l"), heads=[0, 39], blocks=[0, 590, 1181],
             what="pisa_video_l N=75600 H=40 k=148")
    _CACHE.clear()
