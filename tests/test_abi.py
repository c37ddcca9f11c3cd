"""The C ABI on the host (no GPU needed): the library loads, exports every function that
include/*.h declares, sizes workspaces, and rejects bad arguments with the documented status
before enqueuing anything."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

import block_sparse_linear_02_amd as sla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first


@pytest.fixture(scope="module")
def L():
    # SLA_TEST_LIB: another build of the library to run these checks against (the host-only
    # AddressSanitizer build, tests/test_asan_host.py)
    other = os.environ.get("SLA_TEST_LIB")
    if other:
        return sla.configure(ctypes.CDLL(other))
    if not os.path.exists(sla.lib_path()):
        from block_sparse_linear_02_amd import build

        build.build()
    return sla.lib()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(sla_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) >= 16, names
    assert "sla_pisa_forward" in names and "sla_route" in names
    out = subprocess.run(["nm", "-D", "--defined-only", sla.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sla_\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        assert hasattr(L, n)


def P(B=1, H=2, N=4096, d=128, block=64, topk=8, dtype=sla.SLA_BF16):
    return sla.Problem(B, H, N, d, block, topk, dtype)


def test_workspace_sizes(L):
    r = lambda p: L.sla_route_workspace_bytes(ctypes.byref(p))  # noqa: E731
    f = lambda p, v: L.sla_forward_workspace_bytes(ctypes.byref(p), v)  # noqa: E731
    assert r(P()) > 0 and f(P(), 0) > 0
    assert r(P(N=8192)) > r(P()) and r(P(H=4)) > r(P())
    for v in (0, 1, 2, 3, 4):
        assert f(P(N=8192), v) > f(P(), v) and f(P(H=4), v) > f(P(), v)
    assert f(P(), 2) > f(P(), 0) and f(P(), 1) > f(P(), 0) and f(P(), 3) > f(P(), 0)
    assert f(P(), 4) > f(P(), 3) and f(P(), 4) > f(P(), 1)
    # invalid or unsupported problems size to 0
    assert r(P(B=0)) == 0 and r(P(block=32)) == 0 and r(P(d=96)) == 0 and r(P(topk=65)) == 0
    assert f(P(), 5) == f(P(), 4)  # int8 codes take the space of the fp8 ones
    assert f(P(), 6) == 0 and f(P(), -1) == 0
    assert L.sla_route_workspace_bytes(None) == 0


@pytest.mark.parametrize(
    "prob,status",
    [
        (P(B=0), sla.SLA_ERR_INVALID),
        (P(H=-1), sla.SLA_ERR_INVALID),
        (P(N=0), sla.SLA_ERR_INVALID),
        (P(topk=-1), sla.SLA_ERR_INVALID),
        (P(topk=65), sla.SLA_ERR_INVALID),  # n_b = 64
        (P(block=32), sla.SLA_ERR_UNSUPPORTED),
        (P(d=96), sla.SLA_ERR_UNSUPPORTED),
        (P(dtype=7), sla.SLA_ERR_UNSUPPORTED),
        (P(N=64 * 2049, topk=1), sla.SLA_ERR_UNSUPPORTED),  # more key blocks than the router holds
        (P(B=1 << 20, H=1 << 12, N=1 << 17, topk=1), sla.SLA_ERR_INVALID),  # too many (b, h, block)
    ],
)
def test_problem_checks(L, prob, status):
    ws = 1 << 40
    assert L.sla_route(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == status
    assert L.sla_forward(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == status


def test_pointer_and_workspace_checks(L):
    p = P()
    ws_r = L.sla_route_workspace_bytes(ctypes.byref(p))
    ws_f = L.sla_forward_workspace_bytes(ctypes.byref(p), 0)
    assert L.sla_route(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws_r, None) == sla.SLA_ERR_INVALID
    assert L.sla_route(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws_r, None) == sla.SLA_ERR_INVALID
    assert L.sla_route(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, ws_r, None) == sla.SLA_ERR_INVALID
    assert L.sla_route(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, ws_r, None) == sla.SLA_ERR_INVALID
    assert L.sla_route(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws_r - 1, None) == sla.SLA_ERR_WORKSPACE
    assert L.sla_forward(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, ws_f, None) == sla.SLA_ERR_INVALID
    assert L.sla_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws_f, None) == sla.SLA_ERR_INVALID
    assert L.sla_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_f, None) == sla.SLA_ERR_INVALID
    assert L.sla_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws_f, None) == sla.SLA_ERR_INVALID
    assert L.sla_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_f - 1, None) == sla.SLA_ERR_WORKSPACE
    # idx may be NULL only when nothing is kept
    p0 = P(topk=0)
    assert L.sla_forward(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws_f, None) == sla.SLA_ERR_INVALID
    ws0 = L.sla_forward_workspace_bytes(ctypes.byref(p0), 0)
    assert L.sla_forward(ctypes.byref(p0), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws0 - 1, None) == sla.SLA_ERR_WORKSPACE


def test_fp8_and_mode_checks(L):
    p = P()
    ws = 1 << 40
    opts_lit = sla.ForwardOpts(sla.LINEAR_MODES["literal"], None, None)
    opts_mp = sla.ForwardOpts(sla.LINEAR_MODES["mask_product"], None, None)
    opts_bad = sla.ForwardOpts(7, None, None)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert L.sla_forward_fp8(ctypes.byref(P(d=64)), *args) == sla.SLA_ERR_UNSUPPORTED
    assert L.sla_forward_fp8(ctypes.byref(P(dtype=sla.SLA_F32)), *args) == sla.SLA_ERR_UNSUPPORTED
    assert L.sla_forward_fp8_ex(ctypes.byref(p), *args, ctypes.byref(opts_lit)) == sla.SLA_ERR_INVALID
    # fp8 with the mask-product mode is accepted: with a one-byte workspace it stops at the size
    # check, before anything is enqueued
    small = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)
    assert L.sla_forward_fp8_ex(ctypes.byref(p), *small, ctypes.byref(opts_mp)) == sla.SLA_ERR_WORKSPACE
    assert L.sla_forward_ex(ctypes.byref(p), *args, ctypes.byref(opts_bad)) == sla.SLA_ERR_INVALID
    assert L.sla_quantize_e4m3(ctypes.byref(P(d=64)), FAKE, FAKE, FAKE, None) == sla.SLA_ERR_UNSUPPORTED
    assert L.sla_quantize_e4m3(ctypes.byref(p), None, FAKE, FAKE, None) == sla.SLA_ERR_INVALID


def test_int8_checks(L):
    p = P()
    ws = 1 << 40
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert L.sla_forward_int8(ctypes.byref(P(d=64)), *args) == sla.SLA_ERR_UNSUPPORTED
    assert L.sla_forward_int8(ctypes.byref(P(dtype=sla.SLA_F32)), *args) == sla.SLA_ERR_UNSUPPORTED
    for mode in ("fused", "literal"):
        o = sla.ForwardOpts(sla.LINEAR_MODES[mode], None, None)
        assert L.sla_forward_int8_ex(ctypes.byref(p), *args, ctypes.byref(o)) in (
            sla.SLA_ERR_UNSUPPORTED, sla.SLA_ERR_INVALID)
    o = sla.ForwardOpts(sla.LINEAR_MODES["mask_product"], None, None, None, None, 1, 0.0)
    assert L.sla_forward_int8_ex(ctypes.byref(p), *args, ctypes.byref(o)) == sla.SLA_ERR_UNSUPPORTED
    small = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)
    assert L.sla_forward_int8(ctypes.byref(p), *small) == sla.SLA_ERR_WORKSPACE
    assert L.sla_quantize_int8(ctypes.byref(P(d=64)), FAKE, FAKE, FAKE, None) == sla.SLA_ERR_UNSUPPORTED
    assert L.sla_quantize_int8(ctypes.byref(p), FAKE, None, FAKE, None) == sla.SLA_ERR_INVALID


def test_branch_drop_checks(L):
    p = P()
    ws = 1 << 40
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    mp, fused = sla.LINEAR_MODES["mask_product"], sla.LINEAR_MODES["fused"]
    for tau in (-0.01, 0.5, float("nan")):
        o = sla.ForwardOpts(mp, None, None, None, None, 1, tau)
        assert L.sla_forward_ex(ctypes.byref(p), *args, ctypes.byref(o)) == sla.SLA_ERR_INVALID
    o = sla.ForwardOpts(fused, None, None, None, None, 1, 0.0)
    assert L.sla_forward_ex(ctypes.byref(p), *args, ctypes.byref(o)) == sla.SLA_ERR_UNSUPPORTED
    o = sla.ForwardOpts(mp, None, None, None, None, 1, 0.0)
    assert L.sla_forward_fp8_ex(ctypes.byref(p), *args, ctypes.byref(o)) == sla.SLA_ERR_UNSUPPORTED
    # accepted settings stop at the workspace check here (one byte), before anything is enqueued
    small = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)
    o = sla.ForwardOpts(mp, None, None, None, None, 1, 0.25)
    assert L.sla_forward_ex(ctypes.byref(p), *small, ctypes.byref(o)) == sla.SLA_ERR_WORKSPACE


def test_backward_checks(L):
    p = P()
    wb = L.sla_backward_workspace_bytes(ctypes.byref(p))
    assert wb > 0 and L.sla_backward_workspace_bytes(ctypes.byref(P(H=4))) > wb
    assert L.sla_backward_workspace_bytes(ctypes.byref(P(d=96))) == 0
    f = L.sla_backward
    args = [FAKE] * 10 + [None, FAKE, wb, None]  # Q K V idx alpha dO dQ dK dV dalpha O ws bytes stream
    assert f(ctypes.byref(P(d=64)), *args) == sla.SLA_ERR_UNSUPPORTED
    assert f(ctypes.byref(P(dtype=sla.SLA_F32)), *args) == sla.SLA_ERR_UNSUPPORTED
    for i in range(10):
        bad = list(args)
        bad[i] = None
        assert f(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, i
    short = list(args)
    short[12] = wb - 1
    assert f(ctypes.byref(p), *short) == sla.SLA_ERR_WORKSPACE


def test_validate_checks(L):
    """sla_validate_idx: the host-side checks run before the device check; topk = 0 checks
    nothing (no device call)."""
    f = L.sla_validate_idx
    assert f(ctypes.byref(P()), None, None) == sla.SLA_ERR_INVALID
    assert f(ctypes.byref(P(topk=65)), FAKE, None) == sla.SLA_ERR_INVALID  # topk > n_b
    assert f(ctypes.byref(P(d=96)), FAKE, None) == sla.SLA_ERR_UNSUPPORTED
    assert f(ctypes.byref(P(topk=0)), None, None) == sla.SLA_OK


def test_soft_checks(L):
    """SoftTop-k entry points: bf16 with d = 128 only, null pointers and a temperature that is not
    a positive finite number rejected, a short workspace rejected, all before anything is
    enqueued."""
    p = P()
    ws = L.sla_soft_workspace_bytes(ctypes.byref(p))
    assert ws > 0 and L.sla_soft_workspace_bytes(ctypes.byref(P(H=4))) > ws
    assert L.sla_soft_workspace_bytes(ctypes.byref(P(d=64))) == 0
    assert L.sla_soft_workspace_bytes(ctypes.byref(P(dtype=sla.SLA_F32))) == 0
    route = L.sla_soft_route
    r_args = [FAKE, FAKE, FAKE, FAKE, 0.5, FAKE, FAKE, ws, None]  # Q K Wq Wk T M ws bytes stream
    assert route(ctypes.byref(P(d=64)), *r_args) == sla.SLA_ERR_UNSUPPORTED
    for i in (0, 1, 2, 3, 5, 6):
        bad = list(r_args)
        bad[i] = None
        assert route(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, i
    for t in (0.0, -1.0, float("inf"), float("nan")):
        bad = list(r_args)
        bad[4] = t
        assert route(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, t
    short = list(r_args)
    short[7] = ws - 1
    assert route(ctypes.byref(p), *short) == sla.SLA_ERR_WORKSPACE
    fwd = L.sla_soft_forward
    f_args = [FAKE] * 7 + [ws, None]  # Q K V M alpha O ws bytes stream
    for i in range(7):
        bad = list(f_args)
        bad[i] = None
        assert fwd(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, i
    short = list(f_args)
    short[7] = ws - 1
    assert fwd(ctypes.byref(p), *short) == sla.SLA_ERR_WORKSPACE
    bwd = L.sla_soft_backward
    # Q K V Wq Wk T M alpha dO dWq dWk dalpha dM O ws bytes stream
    b_args = [FAKE] * 5 + [0.5] + [FAKE] * 6 + [None, None, FAKE, ws, None]
    for i in (0, 1, 2, 3, 4, 6, 7, 8, 9, 10, 11, 14):
        bad = list(b_args)
        bad[i] = None
        assert bwd(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, i
    bad = list(b_args)
    bad[5] = 0.0
    assert bwd(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID
    short = list(b_args)
    short[15] = ws - 1
    assert bwd(ctypes.byref(p), *short) == sla.SLA_ERR_WORKSPACE
    step = L.sla_stage1_step
    # Q K V O_full Wq Wk alpha T lr lra loss ws bytes stream
    s_args = [FAKE] * 7 + [0.5, 1.0, 1.0, FAKE, FAKE, ws, None]
    for i in (0, 1, 2, 3, 4, 5, 6, 10, 11):
        bad = list(s_args)
        bad[i] = None
        assert step(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, i
    short = list(s_args)
    short[12] = ws - 1
    assert step(ctypes.byref(p), *short) == sla.SLA_ERR_WORKSPACE


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4):
        assert L.sla_status_string(st).decode()
    assert L.sla_status_string(42) == b"unknown status"
    assert L.sla_last_hip_error() == 0


def test_binding_refuses_cpu_tensors(L):
    x = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sla.route(x, x, torch.eye(128), torch.eye(128), 1)
    with pytest.raises(ValueError):
        sla.forward(x, x, x, torch.zeros((1, 1, 1, 1), dtype=torch.int32), torch.zeros((1, 1, 64)))


def test_pisa_sizes_and_offsets(L):
    sb = lambda p: L.sla_pisa_stats_bytes(ctypes.byref(p))  # noqa: E731
    wb = lambda p: L.sla_pisa_workspace_bytes(ctypes.byref(p))  # noqa: E731
    p = P()
    assert sb(p) > 0 and wb(p) > 0
    assert sb(P(N=8192)) > sb(p) and sb(P(H=4)) > sb(p) and wb(P(H=4)) > wb(p)
    assert sb(P(B=0)) == 0 and wb(P(d=96)) == 0 and sb(P(block=32)) == 0
    offs = (ctypes.c_size_t * 7)()
    assert L.sla_pisa_stats_offsets(ctypes.byref(p), offs) == sla.SLA_OK
    B, H, N, d = 1, 2, 4096, 128
    nb = N // 64
    sizes = [B * H * nb * d * 2] * 3 + [B * H * d * d * 2, B * H * d * d * 4, B * H * nb * 4, B * H * nb * 4]
    for i in range(7):
        assert offs[i] % 256 == 0
        if i:
            assert offs[i] >= offs[i - 1] + sizes[i - 1]
    assert offs[6] + sizes[6] <= sb(p)
    assert L.sla_pisa_stats_offsets(ctypes.byref(P(d=96)), offs) == sla.SLA_ERR_UNSUPPORTED
    assert L.sla_pisa_stats_offsets(ctypes.byref(p), None) == sla.SLA_ERR_INVALID


def test_pisa_argument_checks(L):
    p = P()
    sb = L.sla_pisa_stats_bytes(ctypes.byref(p))
    wb = L.sla_pisa_workspace_bytes(ctypes.byref(p))
    # every call below fails a check before anything is enqueued
    assert L.sla_pisa_stats(ctypes.byref(p), FAKE, None, FAKE, sb, FAKE, wb, None) == sla.SLA_ERR_INVALID
    assert L.sla_pisa_stats(ctypes.byref(p), FAKE, FAKE, FAKE, sb - 1, FAKE, wb, None) == sla.SLA_ERR_WORKSPACE
    assert L.sla_pisa_stats(ctypes.byref(p), FAKE, FAKE, FAKE, sb, FAKE, wb - 1, None) == sla.SLA_ERR_WORKSPACE
    assert L.sla_pisa_stats(ctypes.byref(P(d=96)), FAKE, FAKE, FAKE, sb, FAKE, wb, None) == sla.SLA_ERR_UNSUPPORTED
    r = L.sla_pisa_route
    assert r(ctypes.byref(p), FAKE, FAKE, sb, 2, FAKE, None, None, FAKE, wb, None) == sla.SLA_ERR_INVALID
    assert r(ctypes.byref(p), FAKE, FAKE, sb, 1, None, None, None, FAKE, wb, None) == sla.SLA_ERR_INVALID
    assert r(ctypes.byref(p), FAKE, FAKE, sb - 1, 1, FAKE, None, None, FAKE, wb, None) == sla.SLA_ERR_WORKSPACE
    assert r(ctypes.byref(p), FAKE, FAKE, sb, 0, FAKE, None, None, FAKE, wb - 1, None) == sla.SLA_ERR_WORKSPACE
    assert r(ctypes.byref(P(topk=65)), FAKE, FAKE, sb, 1, FAKE, None, None, FAKE, wb, None) == sla.SLA_ERR_INVALID
    f = L.sla_pisa_forward
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, sb, None, FAKE, None) == sla.SLA_ERR_INVALID
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, None, sb, FAKE, FAKE, None) == sla.SLA_ERR_INVALID
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, sb, FAKE, None, None) == sla.SLA_ERR_INVALID
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, sb - 1, FAKE, FAKE, None) == sla.SLA_ERR_WORKSPACE
    assert f(ctypes.byref(P(block=32)), FAKE, FAKE, FAKE, FAKE, sb, FAKE, FAKE, None) == sla.SLA_ERR_UNSUPPORTED


def test_pisa_binding_refuses_cpu_tensors(L):
    x = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sla.pisa_stats(x, x)


def test_svoo_checks(L):
    """SVOO co-clustering and row permutations: every call below is refused on the host, before
    anything is enqueued."""
    p = P()
    wb = L.sla_svoo_workspace_bytes(ctypes.byref(p))
    assert wb > 0 and L.sla_svoo_workspace_bytes(ctypes.byref(P(H=4))) > wb
    for bad in (P(d=64), P(d=96), P(dtype=sla.SLA_F32)):
        assert L.sla_svoo_workspace_bytes(ctypes.byref(bad)) == 0
    c = L.sla_svoo_cluster
    args = [FAKE, FAKE, 3, None, None, FAKE, FAKE, FAKE, wb, None]  # Q K iters qa ka pq pk ws bytes stream
    assert c(ctypes.byref(P(d=64)), *args) == sla.SLA_ERR_UNSUPPORTED
    assert c(ctypes.byref(P(dtype=sla.SLA_F32)), *args) == sla.SLA_ERR_UNSUPPORTED
    for i in (0, 1, 5, 6, 7):  # Q, K, perm_q, perm_k, workspace
        bad = list(args)
        bad[i] = None
        assert c(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, i
    for iters in (0, -1, 65):
        bad = list(args)
        bad[2] = iters
        assert c(ctypes.byref(p), *bad) == sla.SLA_ERR_INVALID, iters
    short = list(args)
    short[8] = wb - 1
    assert c(ctypes.byref(p), *short) == sla.SLA_ERR_WORKSPACE
    for fn in (L.sla_svoo_gather, L.sla_svoo_scatter):
        for rb in (0, 3, 6, 4100, -4):
            assert fn(ctypes.byref(p), FAKE, rb, FAKE, FAKE, None) == sla.SLA_ERR_INVALID, rb
        assert fn(ctypes.byref(p), None, 256, FAKE, FAKE, None) == sla.SLA_ERR_INVALID
        assert fn(ctypes.byref(p), FAKE, 256, None, FAKE, None) == sla.SLA_ERR_INVALID
        assert fn(ctypes.byref(p), FAKE, 256, FAKE, None, None) == sla.SLA_ERR_INVALID
        assert fn(ctypes.byref(P(N=0)), FAKE, 256, FAKE, FAKE, None) == sla.SLA_ERR_INVALID
        assert fn(ctypes.byref(P(B=2, H=40000)), FAKE, 256, FAKE, FAKE, None) == sla.SLA_ERR_UNSUPPORTED


def test_svoo_binding_refuses_cpu_tensors(L):
    x = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    perm = torch.zeros((1, 1, 64), dtype=torch.int32)
    with pytest.raises(ValueError):
        sla.svoo_cluster(x, x)
    with pytest.raises(ValueError):
        sla.svoo_gather(x, perm)
    with pytest.raises(ValueError):
        sla.svoo_scatter(x, perm)


def test_out_rows_checks(L):
    """out_rows is refused outside the bf16 mask-product forward, on the host."""
    p = P()
    o = sla.ForwardOpts(sla.LINEAR_MODES["fused"], None, None, None, None, 0, 0.0, None, FAKE)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert L.sla_forward_ex(ctypes.byref(p), *args, ctypes.byref(o)) == sla.SLA_ERR_UNSUPPORTED
    o = sla.ForwardOpts(sla.LINEAR_MODES["mask_product"], None, None, None, None, 0, 0.0, None, FAKE)
    assert L.sla_forward_fp8_ex(ctypes.byref(p), *args, ctypes.byref(o)) == sla.SLA_ERR_UNSUPPORTED
    # accepted: stops at the workspace check (one byte), before anything is enqueued
    small = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)
    assert L.sla_forward_ex(ctypes.byref(p), *small, ctypes.byref(o)) == sla.SLA_ERR_WORKSPACE
