"""GPU parity: the HIP library (through its C ABI) against the CPU float64 oracle.

Bars: router indices and mask bit-exact; O within max-abs 1e-2 and relative L2 5e-3 (bf16 or
fp32 inputs, fp32 accumulation), relative L2 3e-2 for the fp8 and int8 sparse branches; e4m3 and
int8 codes and scales byte-exact.  Small cases are compared element by element over every output; the
full-size workloads (the ones the benchmark times) over every router row and over sampled query
blocks of sampled heads (always including the first and the last, possibly short, block).
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_linear_02_amd as sla
import gen
import oracle
from tests import cases
from tests import lowbit_slack

pytestmark = pytest.mark.gpu

TOL_MAX = 1e-2
TOL_REL = 5e-3
TOL_REL_FP8 = 3e-2


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sla.lib()  # fail loudly if the library is missing


def dev(c):
    d = torch.device("cuda:0")
    return {k: c[k].to(d) for k in ("Q", "K", "V", "alpha", "Wq", "Wk")}


def oracle_route(c, k):
    return oracle.route(c["Q"], c["K"], c["Wq"].double(), c["Wk"].double(), k, 64)


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


_CACHE = {}


def case(key, wl, ks=None):
    if key not in _CACHE:
        say(f"generating {key} {wl}")
        _CACHE[key] = cases.make_case(wl, ks=ks, log=say)
    return _CACHE[key]


def small_ragged(H=2, k=6, **kw):
    return gen.workload("video_l", H=H, N=3600, grid=(1, 45, 80), topk=k, **kw)  # 57 blocks


# ---------------------------------------------------------------------------------- router


@pytest.mark.parametrize(
    "name,wl",
    [
        ("tiny", gen.workload("tiny")),
        ("ragged_bf16", small_ragged()),
        ("ragged_d64", small_ragged(k=9).with_(d=64, name="ragged_d64")),
        ("ragged_fp32", small_ragged(k=3).with_(dtype="fp32", name="ragged_fp32")),
    ],
)
def test_route_bitexact_small(name, wl):
    c = case(name, wl)
    g = dev(c)
    say(f"route {name}")
    idx, mask, probs = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk, want_mask=True, want_scores=True)
    r = oracle_route(c, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), r["idx"])
    assert np.array_equal(mask.cpu().numpy(), r["mask"])
    np.testing.assert_allclose(probs.cpu().numpy(), r["probs"], rtol=0, atol=2e-5)


@pytest.mark.parametrize("k", [0, 1, 57])
def test_route_degenerate_k(k):
    wl = small_ragged(k=k)
    c = case(f"ragged_k{k}", wl)
    g = dev(c)
    say(f"route k={k}")
    idx, mask, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], k, want_mask=True)
    r = oracle_route(c, k)
    assert idx.shape == (1, 2, 57, k)
    assert np.array_equal(idx.cpu().numpy(), r["idx"])
    assert np.array_equal(mask.cpu().numpy(), r["mask"])


def test_route_exact_ties_keep_lowest_index():
    d = torch.device("cuda:0")
    Q = torch.ones((1, 1, 1000, 128), dtype=torch.bfloat16, device=d)
    W = torch.eye(128, dtype=torch.float32, device=d)
    say("route ties")
    idx, _, _ = sla.route(Q, Q, W, W, 5)
    assert idx.cpu().numpy().tolist() == [[[[0, 1, 2, 3, 4]] * 16]]


@pytest.mark.parametrize("k", [150, 250])
def test_route_wide_ties_fall_back_to_the_full_search(k):
    """600 key blocks whose scores take two values (every third block high): more than 128 keys
    share the k-th largest score's top bits, so the select keeps its bitwise search over every
    key rather than over the compacted band; the lowest indices win every tie."""
    d = torch.device("cuda:0")
    nb = 600
    Q = torch.ones((1, 1, nb * 64, 128), dtype=torch.bfloat16, device=d)
    scale = torch.where(torch.arange(nb) % 3 == 0, 1.0, 0.5).repeat_interleave(64)
    K = (torch.ones((1, 1, nb * 64, 128)) * scale[None, None, :, None]).to(torch.bfloat16).to(d)
    W = torch.eye(128, dtype=torch.float32, device=d)
    say(f"route wide ties k={k}")
    idx, mask, _ = sla.route(Q, K, W, W, k, want_mask=True)
    high = [j for j in range(nb) if j % 3 == 0]
    low = [j for j in range(nb) if j % 3 != 0]
    want = sorted(high[:k] + low[:max(0, k - len(high))])
    got = idx.cpu().numpy()
    assert got.shape == (1, 1, nb, k)
    assert (got == np.array(want)[None, None, None, :]).all()
    r = oracle.route(Q.cpu(), K.cpu(), W.cpu().double(), W.cpu().double(), k, 64)
    assert np.array_equal(got, r["idx"])
    assert np.array_equal(mask.cpu().numpy(), r["mask"])


# ---------------------------------------------------------------------------------- forward


def run_forward(c, idx_np, **kw):
    g = dev(c)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np)).to(g["Q"].device)
    alpha = kw.pop("alpha", g["alpha"])
    O = sla.forward(g["Q"], g["K"], g["V"], idx, alpha, **kw)
    torch.cuda.synchronize()
    return O.cpu().double().numpy()


@pytest.mark.parametrize(
    "name,wl",
    [
        ("tiny", gen.workload("tiny")),
        ("ragged_bf16", small_ragged()),
        ("ragged_d64", small_ragged(k=9).with_(d=64, name="ragged_d64")),
        ("ragged_fp32", small_ragged(k=3).with_(dtype="fp32", name="ragged_fp32")),
    ],
)
def test_forward_small_every_element(name, wl):
    c = case(name, wl)
    r = oracle_route(c, wl.topk)
    say(f"forward {name}")
    got = run_forward(c, r["idx"])
    ref, _, _ = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, what=f"forward {name}")


def test_forward_branches_isolated():
    """alpha = 1 gives the sparse branch alone, alpha = 0 the linear branch alone."""
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    r = oracle_route(c, wl.topk)
    _, Os, Ol = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    d = torch.device("cuda:0")
    one = torch.ones_like(c["alpha"]).to(d)
    say("forward alpha=1")
    check_close(run_forward(c, r["idx"], alpha=one), Os, what="sparse branch (alpha=1)")
    say("forward alpha=0")
    check_close(run_forward(c, r["idx"], alpha=torch.zeros_like(one)), Ol, what="linear branch (alpha=0)")


@pytest.mark.parametrize("k", [0, 1, 57])
def test_forward_degenerate_k(k):
    """k = 0: no sparse branch; k = n_b: full softmax attention and no linear branch."""
    wl = small_ragged(k=k)
    c = case(f"ragged_k{k}", wl)
    r = oracle_route(c, k)
    say(f"forward k={k}")
    got = run_forward(c, r["idx"])
    ref, _, Ol = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, what=f"forward k={k}")
    if k == 57:
        assert np.all(Ol == 0)


@pytest.mark.parametrize(
    "name,wl",
    [
        ("tiny", gen.workload("tiny")),
        ("ragged_bf16", small_ragged()),
        ("ragged_d64", small_ragged(k=9).with_(d=64, name="ragged_d64")),
        ("ragged_fp32", small_ragged(k=3).with_(dtype="fp32", name="ragged_fp32")),
        ("ragged_k0", small_ragged(k=0)),
        ("ragged_k1", small_ragged(k=1)),
        ("ragged_k57", small_ragged(k=57)),
    ],
)
def test_forward_mask_product_mode(name, wl):
    """The mask-product linear mode (all T_i from one mask x states product) against the oracle,
    on every element, and against the fused mode."""
    c = case(name, wl)
    r = oracle_route(c, wl.topk)
    say(f"forward mask_product {name}")
    got = run_forward(c, r["idx"], linear_mode="mask_product")
    ref, _, _ = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, what=f"forward mask_product {name}")
    fused = run_forward(c, r["idx"])
    check_close(got, fused, rel_tol=2e-3, max_tol=5e-3, what=f"mask_product vs fused {name}")


def test_mask_product_linear_branch_alone():
    """alpha = 0: the linear branch alone, built from the mask x states product."""
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    r = oracle_route(c, wl.topk)
    _, _, Ol = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    zero = torch.zeros_like(c["alpha"]).to(torch.device("cuda:0"))
    say("forward mask_product alpha=0")
    check_close(run_forward(c, r["idx"], alpha=zero, linear_mode="mask_product"), Ol,
                what="mask_product linear branch (alpha=0)")


def test_forward_literal_linear_mode():
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    r = oracle_route(c, wl.topk)
    say("forward literal")
    got = run_forward(c, r["idx"], linear_mode="literal")
    ref, _, _ = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, what="forward literal")
    fused = run_forward(c, r["idx"])
    check_close(got, fused, rel_tol=1e-3, max_tol=1e-3, what="literal vs fused")


@pytest.mark.parametrize("mode", ["mask_product", "fused"])
def test_router_on_second_stream(mode):
    """sla_route on a second stream with the forward waiting on its event (idx_ready) only
    before idx is read: the same output, bit for bit, as route then forward on one stream; three
    steps in a row, each router waiting for the previous step's forward."""
    c = case("ragged_bf16", small_ragged())
    g = dev(c)
    k = c["workload"].topk
    idx_ref, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], k)
    O_ref = sla.forward(g["Q"], g["K"], g["V"], idx_ref, g["alpha"], linear_mode=mode)
    idx = torch.empty_like(idx_ref)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    outs = []
    for _ in range(3):
        side.wait_stream(main)
        with torch.cuda.stream(side):
            sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], k, idx_out=idx)
            ready.record()
        outs.append(sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode=mode, idx_ready=ready))
    torch.cuda.synchronize()
    say(f"router on a second stream ({mode}): 3 steps")
    assert torch.equal(idx, idx_ref)
    for O in outs:
        assert torch.equal(O, O_ref)


def test_forward_deterministic():
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    g = dev(c)
    say("determinism")
    outs = []
    for _ in range(2):
        idx, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk)
        outs.append((idx.cpu(), sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"]).cpu(),
                     sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], fp8=True).cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------------- fp8


def test_quantize_e4m3_bytes_exact():
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    g = dev(c)
    for name in ("Q", "K", "V"):
        say(f"quantize {name}")
        codes, scales = sla.quantize_e4m3(g[name])
        codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
        for b in range(wl.B):
            for h in range(wl.H):
                rc, rs, _ = oracle.quantize_blocks(c[name][b, h], 64)
                assert np.array_equal(scales[b, h], rs)
                assert np.array_equal(codes[b, h], rc)


def test_fp8_forward_small():
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    r = oracle_route(c, wl.topk)
    say("forward fp8 small")
    got = run_forward(c, r["idx"], fp8=True)
    ref, _, _ = oracle.forward_fp8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, rel_tol=TOL_REL_FP8, max_tol=None, what="forward fp8 small")


@pytest.mark.parametrize("k", [0, 1, 57])
def test_fp8_forward_degenerate_k(k):
    """The quantised sparse branch with nothing kept, one block kept, and every block kept."""
    wl = small_ragged(k=k)
    c = case(f"ragged_k{k}", wl)
    r = oracle_route(c, k)
    say(f"forward fp8 k={k}")
    got = run_forward(c, r["idx"], fp8=True)
    ref, _, _ = oracle.forward_fp8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, rel_tol=TOL_REL_FP8, max_tol=None, what=f"forward fp8 k={k}")


@pytest.mark.parametrize("lowbit,mode", [("fp8", "mask_product"), ("fp8", "fused"), ("int8", "mask_product")])
def test_lowbit_kv_codes_from_the_state_kernel(lowbit, mode, monkeypatch):
    """The K and V codes the state kernel writes on its way through K and V give the same output,
    bit for bit, as codes from the stand-alone quantiser (SLA_SEPARATE_QUANT=1), on a ragged
    sequence (last block 16 tokens) with two heads."""
    wl = small_ragged(k=6)
    c = case("ragged_bf16", wl)
    r = oracle_route(c, 6)
    kw = {"fp8": lowbit == "fp8", "int8": lowbit == "int8", "linear_mode": mode}
    say(f"forward {lowbit} {mode}: codes from the state kernel, then from their own launches")
    monkeypatch.delenv("SLA_SEPARATE_QUANT", raising=False)
    fused = run_forward(c, r["idx"], **kw)
    monkeypatch.setenv("SLA_SEPARATE_QUANT", "1")
    apart = run_forward(c, r["idx"], **kw)
    assert np.array_equal(fused, apart), f"{lowbit} {mode}: max |diff| {np.abs(fused - apart).max()}"


@pytest.mark.parametrize("k", [6, 0, 1, 57])
def test_fp8_forward_mask_product(k):
    """The quantised sparse branch on two query blocks per workgroup (mask-product linear mode)
    against the oracle, on every element, for k = 6 and the degenerate counts."""
    wl = small_ragged(k=k)
    c = case("ragged_bf16" if k == 6 else f"ragged_k{k}", wl)
    r = oracle_route(c, k)
    say(f"forward fp8 mask_product k={k}")
    got = run_forward(c, r["idx"], fp8=True, linear_mode="mask_product")
    ref, _, _ = oracle.forward_fp8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, rel_tol=TOL_REL_FP8, max_tol=None, what=f"forward fp8 mask_product k={k}")
    fused = run_forward(c, r["idx"], fp8=True)
    check_close(got, fused, rel_tol=1e-2, max_tol=None, what=f"fp8 mask_product vs fused k={k}")


def test_quantize_int8_bytes_exact():
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    g = dev(c)
    for name in ("Q", "K", "V"):
        say(f"quantize int8 {name}")
        codes, scales = sla.quantize_int8(g[name])
        codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
        for b in range(wl.B):
            for h in range(wl.H):
                rc, rs, _ = oracle.quantize_blocks_int8(c[name][b, h], 64)
                assert np.array_equal(scales[b, h], rs)
                assert np.array_equal(codes[b, h], rc)


@pytest.mark.parametrize("k", [6, 0, 1, 57])
def test_int8_forward(k):
    """The INT8 sparse branch (two query blocks per workgroup, mask-product linear mode) against
    the int8 oracle on every element, for k = 6 and the degenerate counts; alpha = 1 isolates
    the quantised branch."""
    wl = small_ragged(k=k)
    c = case("ragged_bf16" if k == 6 else f"ragged_k{k}", wl)
    r = oracle_route(c, k)
    say(f"forward int8 k={k}")
    got = run_forward(c, r["idx"], int8=True, linear_mode="mask_product")
    ref, Os, _ = oracle.forward_int8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, rel_tol=TOL_REL_FP8, max_tol=None, what=f"forward int8 k={k}")
    if 0 < k:
        one = torch.ones_like(c["alpha"]).to("cuda:0")
        check_close(run_forward(c, r["idx"], alpha=one, int8=True, linear_mode="mask_product"), Os,
                    rel_tol=TOL_REL_FP8, max_tol=None, what=f"int8 sparse branch alone k={k}")


@pytest.mark.parametrize("k", [6, 30])
def test_lowbit_p_reading_conformance(k):
    """alpha = 1: the fp8 (fused and mask-product kernels) and int8 sparse branches alone against
    the oracle's O_s, element by element within the flip-aware bound of tests/lowbit_slack.py:
    one code step for P entries whose code the kernels' fp32 rounding (and, for e4m3, the fp8
    product's accumulation) may decide either way, plus a small relative tolerance of each row's
    magnitude.  Another reading of the P step (a per-row or per-query-block
    scale, a dequantised denominator) breaks it on thousands of elements, which the 3e-2
    acceptance bar cannot see."""
    wl = small_ragged(k=k)
    c = case(f"ragged_k{k}", wl)
    r = oracle_route(c, k)
    one = torch.ones_like(c["alpha"]).to(torch.device("cuda:0"))
    starts, ends, _ = oracle.block_ranges(wl.N, 64)
    qb = list(range(wl.n_blocks))
    runs = [("fp8", "fused"), ("fp8", "mask_product"), ("int8", "mask_product")]
    gots = {run: run_forward(c, r["idx"], alpha=one, linear_mode=run[1], **{run[0]: True}) for run in runs}
    for fmt in ("fp8", "int8"):
        head = oracle.forward_fp8_head if fmt == "fp8" else oracle.forward_int8_head
        quant = oracle.quantize_blocks if fmt == "fp8" else oracle.quantize_blocks_int8
        for h in range(wl.H):
            trace = []
            _, Os, _ = head(c["Q"][0, h], c["K"][0, h], c["V"][0, h], r["idx"][0, h], np.ones(wl.N), 64, trace=trace)
            Qd, Kd, Vd = (quant(c[n][0, h], 64)[2] for n in ("Q", "K", "V"))
            sl = lowbit_slack.slack_rows(trace, Vd, starts, ends, qb, fmt, Qd, Kd)
            slack = np.concatenate([s_ for s_, _ in sl])
            tol = np.concatenate([t_ for _, t_ in sl])
            ref = np.concatenate(Os)
            for run in [x for x in runs if x[0] == fmt]:
                got = gots[run][0, h]
                res = lowbit_slack.check_within_slack(got, ref, slack, tol)
                say(f"{fmt} P reading k={k} {run[1]} head {h}: rel-L2 {rel_l2(got, ref):.3e} {res}")
                assert res["violations"] == 0, (fmt, run, h, res)


def test_fp8_forward_branches_isolated():
    """alpha = 1: the quantised sparse branch alone; alpha = 0: the linear branch, unquantised."""
    wl = small_ragged()
    c = case("ragged_bf16", wl)
    r = oracle_route(c, wl.topk)
    _, Os, Ol = oracle.forward_fp8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    one = torch.ones_like(c["alpha"]).to(torch.device("cuda:0"))
    say("forward fp8 alpha=1")
    check_close(run_forward(c, r["idx"], alpha=one, fp8=True), Os, rel_tol=TOL_REL_FP8, max_tol=None,
                what="fp8 sparse branch (alpha=1)")
    say("forward fp8 alpha=0")
    check_close(run_forward(c, r["idx"], alpha=torch.zeros_like(one), fp8=True), Ol,
                what="linear branch beside fp8 (alpha=0)")


# ---------------------------------------------------------------------------------- branch dropping


def drop_alpha(alpha, seed=5):
    """alpha [B, H, N] with per-head patterns: head 0 all 1 (linear weight 0), head 1 all 0,
    head 2 in [0.97, 1] with one token exactly at 1 - 1/32, head 3 in [0, 0.02], the rest as
    drawn."""
    a = alpha.clone()
    g = torch.Generator().manual_seed(seed)
    a[:, 0] = 1.0
    a[:, 1] = 0.0
    a[:, 2] = 0.97 + 0.03 * torch.rand(a[:, 2].shape, generator=g)
    a[:, 2, 7] = 1.0 - 0.03125
    a[:, 3] = 0.02 * torch.rand(a[:, 3].shape, generator=g)
    return a


@pytest.mark.parametrize("tau", [0.0, 0.03125])
def test_branch_drop(tau):
    """Mask-product forward with branch dropping against the oracle's forward_dropped; with
    tau = 0 the output equals the undropped run bit for bit."""
    wl = small_ragged(H=5)
    c = case("ragged_h5", wl)
    r = oracle_route(c, wl.topk)
    alpha = drop_alpha(c["alpha"])
    ref, dl, ds = oracle.forward_dropped(c["Q"], c["K"], c["V"], r["idx"], alpha, tau, 64)
    say(f"branch drop tau={tau}: linear {dl.tolist()}, sparse {ds.tolist()}")
    a_dev = alpha.to("cuda:0")
    got = run_forward(c, r["idx"], alpha=a_dev, linear_mode="mask_product", drop_tau=tau)
    check_close(got, ref, what=f"branch drop tau={tau}")
    if tau == 0.0:
        plain = run_forward(c, r["idx"], alpha=a_dev, linear_mode="mask_product")
        assert np.array_equal(got, plain), "tau = 0 must not change the output"


def test_branch_drop_full_size():
    c = case("video_s", gen.workload("video_s"))
    g = dev(c)
    r = oracle_route(c, 51)
    alpha = drop_alpha(c["alpha"])
    tau = 0.03125
    idx = torch.from_numpy(r["idx"]).to(g["Q"].device)
    say("branch drop video_s")
    O = sla.forward(g["Q"], g["K"], g["V"], idx, alpha.to(g["Q"].device), linear_mode="mask_product",
                    drop_tau=tau)
    torch.cuda.synchronize()
    got = O.cpu().double().numpy()
    dl, ds = oracle.branch_drops(alpha, tau)
    gots, refs = [], []
    for h in (0, 1, 2, 3, 9):
        _, os_, ol = oracle.forward_head(c["Q"][0, h], c["K"][0, h], c["V"][0, h], r["idx"][0, h],
                                         alpha[0, h], 64, q_blocks=[0, 300, 511])
        for i, a_s, a_l in zip([0, 300, 511], os_, ol):
            a = alpha[0, h, i * 64 : i * 64 + len(a_s)].double().numpy()[:, None]
            refs.append((0.0 if ds[0, h] else a * a_s) + (0.0 if dl[0, h] else (1 - a) * a_l))
            gots.append(got[0, h, i * 64 : i * 64 + len(a_s)])
    check_close(np.concatenate(gots), np.concatenate(refs), what="branch drop video_s")


# ---------------------------------------------------------------------------------- full size


def oracle_blocks(c, idx_np, heads, blocks, fp8=False, alpha=None):
    """Oracle output rows of the given query blocks of the given (flattened b*H + h) heads,
    concatenated in that order; blocks=None means every query block."""
    wl = c["workload"]
    alpha = c["alpha"] if alpha is None else alpha
    refs = []
    for bh in heads:
        b, h = divmod(bh, wl.H)
        args = (c["Q"][b, h], c["K"][b, h], c["V"][b, h], idx_np[b, h], alpha[b, h], 64)
        qb = list(range(wl.n_blocks)) if blocks is None else blocks
        o, _, _ = (oracle.forward_fp8_head if fp8 else oracle.forward_head)(*args, q_blocks=qb)
        refs.extend(o)
    return np.concatenate(refs)


def gpu_blocks(c, got_O, heads, blocks):
    """The GPU rows matching oracle_blocks(c, ..., heads, blocks)."""
    wl = c["workload"]
    gots = []
    for bh in heads:
        b, h = divmod(bh, wl.H)
        if blocks is None:
            gots.append(got_O[b, h])
        else:
            gots.extend(got_O[b, h, i * 64 : min((i + 1) * 64, wl.N)] for i in blocks)
    return np.concatenate(gots)


def sampled_compare(c, idx_np, got_O, heads, blocks, fp8=False, what=""):
    ref = oracle_blocks(c, idx_np, heads, blocks, fp8=fp8)
    got = gpu_blocks(c, got_O, heads, blocks)
    if fp8:
        check_close(got, ref, rel_tol=TOL_REL_FP8, max_tol=None, what=what)
    else:
        check_close(got, ref, what=what)


def full_size(c, heads, blocks, fp8=False, what="", linear_mode="fused"):
    wl = c["workload"]
    g = dev(c)
    say(f"route {what}")
    idx, mask, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk, want_mask=True)
    r = oracle_route(c, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), f"{what}: router indices differ"
    assert np.array_equal(mask.cpu().numpy(), r["mask"]), f"{what}: router mask differs"
    say(f"forward {what}")
    O = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], fp8=fp8, linear_mode=linear_mode)
    torch.cuda.synchronize()
    got = O.cpu().double().numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    sampled_compare(c, r["idx"], got, heads, blocks, fp8=fp8, what=what)


def test_video_s_full_size():
    c = case("video_s", gen.workload("video_s"))
    full_size(c, heads=[0, 5, 11], blocks=[0, 1, 200, 511], what="video_s N=32768 H=12 k=51")


def test_video_s_full_size_mask_product():
    c = case("video_s", gen.workload("video_s"))
    full_size(c, heads=[0, 7], blocks=[0, 300, 511], what="video_s mask_product", linear_mode="mask_product")


@pytest.mark.parametrize("mode", ["fused", "mask_product"])
def test_video_l_full_size(mode):
    c = case("video_l", gen.workload("video_l"))
    full_size(c, heads=[0, 39], blocks=[0, 600, 1181], what=f"video_l N=75600 H=40 k=60 {mode}",
              linear_mode=mode)


def test_video_s_whole_output_mask_product():
    """The benchmarked launch (router, then the mask-product forward) at N=32768 H=12 k=51 against
    the oracle on every output element: every query block of every head."""
    c = case("video_s", gen.workload("video_s"))
    wl = c["workload"]
    g = dev(c)
    say("video_s whole output: route + mask_product forward")
    idx, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk)
    r = oracle_route(c, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), "video_s: router indices differ"
    O = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode="mask_product")
    torch.cuda.synchronize()
    got = O.cpu().double().numpy()
    say("video_s whole output: oracle (12 heads)")
    ref, _, _ = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    check_close(got, ref, what="video_s whole output mask_product")


def test_video_l_whole_head_mask_product():
    """N=75600 (1182 key blocks, a 16-token last block) in the benchmarked mask-product mode:
    every query block of two heads against the oracle."""
    c = case("video_l", gen.workload("video_l"))
    wl = c["workload"]
    g = dev(c)
    say("video_l whole heads: route + mask_product forward")
    idx, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk)
    r = oracle_route(c, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), "video_l: router indices differ"
    O = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode="mask_product")
    torch.cuda.synchronize()
    got = O.cpu().double().numpy()
    say("video_l whole heads: oracle (heads 7, 38)")
    ref = oracle_blocks(c, r["idx"], [7, 38], None)
    check_close(gpu_blocks(c, got, [7, 38], None), ref, what="video_l whole heads mask_product")


def test_mask_product_odd_blocks_lone_last_window():
    """n_b = 1025 (N = 65590, a 54-token last block): the last matching window of query blocks
    holds one block alone, which runs in a workgroup by itself; every query block of the one
    head against the oracle."""
    wl = gen.workload("video_l", H=1, N=65590, grid=(1, 70, 937), topk=24)
    c = case("odd_1025", wl)
    g = dev(c)
    say("odd n_b 1025: route + mask_product forward")
    idx, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk)
    r = oracle_route(c, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), "odd n_b 1025: router indices differ"
    O = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode="mask_product")
    torch.cuda.synchronize()
    got = O.cpu().double().numpy()
    say("odd n_b 1025: oracle (1 head)")
    ref = oracle_blocks(c, r["idx"], [0], None)
    check_close(gpu_blocks(c, got, [0], None), ref, what="odd n_b 1025 mask_product")


def test_video_l_fp8_full_size():
    c = case("video_l", gen.workload("video_l"))
    full_size(c, heads=[0, 21], blocks=[0, 1181], fp8=True, what="video_l fp8")


def test_video_l_fp8_full_size_mask_product():
    c = case("video_l", gen.workload("video_l"))
    full_size(c, heads=[3, 30], blocks=[0, 591, 1181], fp8=True, what="video_l fp8 mask_product",
              linear_mode="mask_product")


def test_video_l_int8_full_size():
    c = case("video_l", gen.workload("video_l"))
    wl = c["workload"]
    g = dev(c)
    r = oracle_route(c, wl.topk)
    idx = torch.from_numpy(r["idx"]).to(g["Q"].device)
    say("forward video_l int8")
    O = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], int8=True, linear_mode="mask_product")
    torch.cuda.synchronize()
    got = O.cpu().double().numpy()
    gots, refs = [], []
    for bh in (5, 33):
        b, h = divmod(bh, wl.H)
        o, _, _ = oracle.forward_int8_head(c["Q"][b, h], c["K"][b, h], c["V"][b, h], r["idx"][b, h],
                                           c["alpha"][b, h], 64, q_blocks=[0, 700, 1181])
        for i, oi in zip([0, 700, 1181], o):
            refs.append(oi)
            gots.append(got[b, h, i * 64 : i * 64 + len(oi)])
    check_close(np.concatenate(gots), np.concatenate(refs), rel_tol=TOL_REL_FP8, max_tol=None,
                what="video_l int8")


@pytest.mark.parametrize("k", [102, 51, 26, 15])
@pytest.mark.parametrize("scale", [0.5, 1.0, 2.0])
def test_sparsity_sweep(scale, k):
    """keep {20,10,5,3}% of 512 key blocks at cluster scale {0.5,1,2}, B=2, H=12, N=32768;
    alpha fixed at 0.5 and random sigmoid(N(0,1)) (the same Q, K, V for both); the fused and the
    mask-product linear modes."""
    wl = gen.workload("video_s").with_(B=2, topk=k, cluster_scale=scale, name=f"sweep_s{scale:g}_k{k}", wid=4)
    c = case(wl.name, wl)
    g = dev(c)
    r = oracle_route(c, k)
    say(f"sweep s={scale} k={k} route")
    idx, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], k)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), f"sweep s={scale} k={k}: indices differ"
    for a in ("half", "random"):
        alpha = torch.full_like(g["alpha"], 0.5) if a == "half" else g["alpha"]
        ref = oracle_blocks(c, r["idx"], [0, 23], [0, 511], alpha=alpha.cpu())
        for mode in ("fused", "mask_product"):
            say(f"sweep s={scale} k={k} alpha={a} forward {mode}")
            O = sla.forward(g["Q"], g["K"], g["V"], idx, alpha, linear_mode=mode)
            torch.cuda.synchronize()
            check_close(gpu_blocks(c, O.cpu().double().numpy(), [0, 23], [0, 511]), ref,
                        what=f"sweep s={scale} k={k} alpha={a} {mode}")
    _CACHE.pop(wl.name, None)  # keep host memory bounded


# ---------------------------------------------------------------------------------- edge shapes


def edge(name, B, H, N, d, dtype, k):
    return gen.workload("tiny").with_(name=f"edge_{name}", B=B, H=H, N=N, d=d, dtype=dtype, topk=k, wid=6)


EDGE = [
    edge("n1_d64_f32_k0", 1, 1, 1, 64, "fp32", 0),  # one token, nothing kept
    edge("n1_d64_f32_k1", 1, 2, 1, 64, "fp32", 1),  # one token, its only block kept
    edge("n1_d128_bf16_k1", 1, 1, 1, 128, "bf16", 1),
    edge("n1_d128_bf16_k0", 2, 1, 1, 128, "bf16", 0),
    edge("n64_d64_bf16_k1", 1, 3, 64, 64, "bf16", 1),  # exactly one full block
    edge("n65_d128_bf16_k0", 1, 2, 65, 128, "bf16", 0),  # a 1-token tail block
    edge("n65_d128_bf16_k1", 1, 2, 65, 128, "bf16", 1),
    edge("n65_d128_f32_k2", 1, 2, 65, 128, "fp32", 2),
    edge("n127_d64_f32_k1", 2, 1, 127, 64, "fp32", 1),
    edge("n200_d128_bf16_k2", 2, 3, 200, 128, "bf16", 2),  # batch > 1, 8-token tail
    edge("n4097_d128_bf16_k33", 1, 1, 4097, 128, "bf16", 33),  # 65 blocks, half kept, 1-token tail
    edge("n4097_d64_f32_k65", 1, 1, 4097, 64, "fp32", 65),  # every block kept
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_edge_shapes(wl):
    """Tiny and ragged shapes (one token, a one-token tail, one full block, batch > 1, k = 0,
    1, half and all): router bit-exact, and every linear mode plus the fp8 sparse branch (bf16,
    d = 128) on every element against the oracle."""
    c = case(wl.name, wl)
    g = dev(c)
    r = oracle_route(c, wl.topk)
    say(f"edge route {wl.name}")
    idx, mask, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], wl.topk, want_mask=True)
    assert idx.shape == (wl.B, wl.H, wl.n_blocks, wl.topk)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), f"{wl.name}: router indices differ"
    assert np.array_equal(mask.cpu().numpy(), r["mask"]), f"{wl.name}: router mask differs"
    ref, _, _ = oracle.forward(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
    for mode in ("fused", "literal", "mask_product"):
        say(f"edge forward {wl.name} {mode}")
        check_close(run_forward(c, r["idx"], linear_mode=mode), ref, what=f"{wl.name} {mode}")
    if wl.dtype == "bf16" and wl.d == 128:
        ref8, _, _ = oracle.forward_fp8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
        for mode in ("fused", "mask_product"):
            say(f"edge forward {wl.name} fp8 {mode}")
            check_close(run_forward(c, r["idx"], fp8=True, linear_mode=mode), ref8, rel_tol=TOL_REL_FP8,
                        max_tol=None, what=f"{wl.name} fp8 {mode}")
        ref_i8, _, _ = oracle.forward_int8(c["Q"], c["K"], c["V"], r["idx"], c["alpha"], 64)
        say(f"edge forward {wl.name} int8")
        check_close(run_forward(c, r["idx"], int8=True, linear_mode="mask_product"), ref_i8,
                    rel_tol=TOL_REL_FP8, max_tol=None, what=f"{wl.name} int8")
    _CACHE.pop(wl.name, None)


# key-slot counts per lane of the router's top-k: 2, 4, 16, 20, 32 and 32 again at the largest
# supported n_b (2048); clustered latent grids whose token counts leave a short last block
ROUTE_GRIDS = [((2, 50, 63), 128), ((4, 50, 63), 64), ((16, 45, 88), 128), ((20, 50, 79), 64),
               ((24, 50, 79), 128), ((26, 63, 80), 128)]


@pytest.mark.parametrize("grid,d", ROUTE_GRIDS, ids=[f"grid{'x'.join(map(str, g))}_d{d}" for g, d in ROUTE_GRIDS])
def test_route_many_blocks(grid, d):
    """Every key-slot instantiation of the top-k, up to the largest supported n_b: indices and
    mask bit-exact; at n_b = 2048 also the forward (fused and mask-product) on sampled blocks."""
    N = grid[0] * grid[1] * grid[2]
    nb = -(-N // 64)
    k = max(1, nb // 10)
    wl = gen.workload("video_s").with_(name=f"route_nb{nb}", H=1, N=N, d=d, grid=grid, topk=k, wid=7)
    c = case(wl.name, wl)
    g = dev(c)
    say(f"route nb={nb} d={d} k={k}")
    idx, mask, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], k, want_mask=True)
    r = oracle_route(c, k)
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), f"nb={nb}: router indices differ"
    assert np.array_equal(mask.cpu().numpy(), r["mask"]), f"nb={nb}: router mask differs"
    if nb == 2048:
        for mode in ("fused", "mask_product"):
            say(f"forward nb=2048 {mode}")
            O = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode=mode)
            torch.cuda.synchronize()
            sampled_compare(c, r["idx"], O.cpu().double().numpy(), heads=[0], blocks=[0, 1023, 2047],
                            what=f"nb=2048 {mode}")
    _CACHE.pop(wl.name, None)


def test_route_rejects_too_many_blocks():
    """n_b above the largest supported count is an error, not a silent truncation."""
    nb = 2049
    d = torch.device("cuda:0")
    Q = torch.zeros((1, 1, 64 * nb, 64), dtype=torch.bfloat16, device=d)
    W = torch.eye(64, dtype=torch.float32, device=d)
    with pytest.raises(Exception):
        sla.route(Q, Q, W, W, 4)
