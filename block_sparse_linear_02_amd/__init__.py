"""Python binding of libsla, the MI355X (gfx950) SLA2 sparse-linear attention forward.

Argument marshalling only: every step of the forward runs in the HIP kernels of libsla.so
(C ABI in include/sla.h).  torch supplies device memory (tensors, workspaces) and the HIP
stream (torch.cuda.current_stream()).  There is no CPU fallback: without the built library or
a GPU every call raises.

    idx, mask, scores = route(Q, K, proj_q, proj_k, topk, want_mask=False, want_scores=False)
    O = forward(Q, K, V, idx, alpha)                     # bf16 (or fp32-input) sparse branch
    O = forward(Q, K, V, idx, alpha, fp8=True)           # e4m3 sparse branch
    O = forward(Q, K, V, idx, alpha, int8=True, linear_mode="mask_product")  # int8 sparse branch
    O = forward(Q, K, V, idx, alpha, linear_mode="literal")

PISA exact-or-approximate attention (C ABI in include/sla_pisa.h):

    st = pisa_stats(K, V)                                # centroids, value sums, Hbar, M_j
    idx, mask, scores = pisa_route(Q, st, topk, covariance=True)
    O = pisa_forward(Q, K, V, st, idx)

SoftTop-k training path (C ABI in include/sla_soft.h; bf16, d = 128):

    M = soft_route(Q, K, proj_q, proj_k, topk, temperature)    # soft mask [B, H, n_b, n_b]
    O = soft_forward(Q, K, V, M, alpha)
    dWq, dWk, dalpha, dM = soft_backward(Q, K, V, proj_q, proj_k, temperature, M, alpha, dO)
    loss = stage1_step(Q, K, V, O_full, proj_q, proj_k, alpha, topk, temperature, lr, lr_alpha)

SVOO co-clustered blocks (C ABI in include/sla_svoo.h):

    perm_q, perm_k, q_assign, k_assign = svoo_cluster(Q, K, iters=3)
    O = svoo_forward(Q, K, V, proj_q, proj_k, alpha, topk, perm_q, perm_k)

Shapes: Q, K, V [B, H, N, d] (bf16 or fp32, d in {64, 128}), proj_q / proj_k [d, d] fp32,
alpha [B, H, N] fp32, idx [B, H, ceil(N/64), topk] int32 ascending, O [B, H, N, d] fp32.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SLAError",
    "lib",
    "lib_path",
    "route",
    "route_noalloc",
    "forward",
    "quantize_e4m3",
    "quantize_int8",
    "backward",
    "route_workspace_bytes",
    "forward_workspace_bytes",
    "PisaStats",
    "pisa_stats",
    "pisa_route",
    "pisa_forward",
    "pisa_workspace_bytes",
    "soft_workspace_bytes",
    "soft_route",
    "soft_forward",
    "soft_backward",
    "stage1_step",
    "BLOCK",
]

BLOCK = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsla.so")
_LIB = None

SLA_OK, SLA_ERR_INVALID, SLA_ERR_UNSUPPORTED, SLA_ERR_WORKSPACE, SLA_ERR_HIP = 0, -1, -2, -3, -4
SLA_F32, SLA_BF16 = 0, 1
LINEAR_MODES = {"fused": 0, "literal": 1, "mask_product": 2}


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "N", "d", "block", "topk", "dtype")]


class ForwardOpts(ctypes.Structure):
    _fields_ = [
        ("linear_mode", ctypes.c_int32),
        ("sparse_begin", ctypes.c_void_p),
        ("sparse_end", ctypes.c_void_p),
        ("states_begin", ctypes.c_void_p),
        ("states_end", ctypes.c_void_p),
        ("branch_drop", ctypes.c_int32),
        ("drop_tau", ctypes.c_float),
        ("idx_ready", ctypes.c_void_p),
        ("out_rows", ctypes.c_void_p),
    ]


class SLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().sla_status_string(status).decode()
        if status == SLA_ERR_HIP:
            msg += f" (hipError {lib().sla_last_hip_error()})"
        super().__init__(f"{what}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def configure(L: ctypes.CDLL) -> ctypes.CDLL:
    """Argument and result types of every libsla entry point on a loaded copy of the library."""
    P = ctypes.POINTER(Problem)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.sla_route_workspace_bytes.argtypes = [P]
    L.sla_route_workspace_bytes.restype = sz
    L.sla_forward_workspace_bytes.argtypes = [P, i32]
    L.sla_forward_workspace_bytes.restype = sz
    L.sla_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sla_route.restype = i32
    L.sla_route_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.sla_route_noalloc.restype = i32
    L.sla_validate_idx.argtypes = [P, vp, vp]
    L.sla_validate_idx.restype = i32
    fwd = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    for name in ("sla_forward", "sla_forward_fp8"):
        getattr(L, name).argtypes = fwd
        getattr(L, name).restype = i32
    for name in ("sla_forward_int8",):
        getattr(L, name).argtypes = fwd
        getattr(L, name).restype = i32
    for name in ("sla_forward_ex", "sla_forward_fp8_ex", "sla_forward_int8_ex"):
        getattr(L, name).argtypes = fwd + [ctypes.POINTER(ForwardOpts)]
        getattr(L, name).restype = i32
    for name in ("sla_quantize_e4m3", "sla_quantize_int8"):
        getattr(L, name).argtypes = [P, vp, vp, vp, vp]
        getattr(L, name).restype = i32
    L.sla_backward_workspace_bytes.argtypes = [P]
    L.sla_backward_workspace_bytes.restype = sz
    L.sla_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sla_backward.restype = i32
    L.sla_pisa_stats_bytes.argtypes = [P]
    L.sla_pisa_stats_bytes.restype = sz
    L.sla_pisa_workspace_bytes.argtypes = [P]
    L.sla_pisa_workspace_bytes.restype = sz
    L.sla_pisa_stats_offsets.argtypes = [P, ctypes.POINTER(sz)]
    L.sla_pisa_stats_offsets.restype = i32
    L.sla_pisa_stats.argtypes = [P, vp, vp, vp, sz, vp, sz, vp]
    L.sla_pisa_stats.restype = i32
    L.sla_pisa_route.argtypes = [P, vp, vp, sz, i32, vp, vp, vp, vp, sz, vp]
    L.sla_pisa_route.restype = i32
    L.sla_pisa_forward.argtypes = [P, vp, vp, vp, vp, sz, vp, vp, vp]
    L.sla_pisa_forward.restype = i32
    L.sla_svoo_workspace_bytes.argtypes = [P]
    L.sla_svoo_workspace_bytes.restype = sz
    L.sla_svoo_cluster.argtypes = [P, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.sla_svoo_cluster.restype = i32
    for name in ("sla_svoo_gather", "sla_svoo_scatter"):
        getattr(L, name).argtypes = [P, vp, i32, vp, vp, vp]
        getattr(L, name).restype = i32
    f32 = ctypes.c_float
    L.sla_soft_workspace_bytes.argtypes = [P]
    L.sla_soft_workspace_bytes.restype = sz
    L.sla_soft_route.argtypes = [P, vp, vp, vp, vp, f32, vp, vp, sz, vp]
    L.sla_soft_route.restype = i32
    L.sla_soft_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sla_soft_forward.restype = i32
    L.sla_soft_backward.argtypes = [P, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sla_soft_backward.restype = i32
    L.sla_stage1_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, sz, vp]
    L.sla_stage1_step.restype = i32
    L.sla_status_string.argtypes = [i32]
    L.sla_status_string.restype = ctypes.c_char_p
    L.sla_last_hip_error.argtypes = []
    L.sla_last_hip_error.restype = i32
    return L


def lib() -> ctypes.CDLL:
    """The loaded libsla.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m block_sparse_linear_02_amd.build`"
            )
        _LIB = configure(ctypes.CDLL(_LIB_PATH))
    return _LIB


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_qkv(*ts):
    B, H, N, d = ts[0].shape
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("inputs must be GPU tensors")
        if t.shape != (B, H, N, d) or t.dtype != ts[0].dtype:
            raise ValueError("Q, K, V must share shape [B, H, N, d] and dtype")
    if ts[0].dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("Q, K, V must be bf16 or fp32")


def make_problem(B, H, N, d, topk, dtype) -> Problem:
    dt = SLA_BF16 if dtype == torch.bfloat16 else SLA_F32
    return Problem(B, H, N, d, BLOCK, topk, dt)


def _problem(Q, topk) -> Problem:
    B, H, N, d = Q.shape
    return make_problem(B, H, N, d, topk, Q.dtype)


def route_workspace_bytes(Q, topk: int) -> int:
    return lib().sla_route_workspace_bytes(ctypes.byref(_problem(Q, topk)))


def forward_workspace_bytes(Q, topk: int, variant: int = 0) -> int:
    return lib().sla_forward_workspace_bytes(ctypes.byref(_problem(Q, topk)), variant)


def validate_idx(Q, idx) -> bool:
    """Debug check of idx [B, H, n_b, topk] int32 for inputs shaped like Q (sla_validate_idx):
    True when every entry lies in [0, n_b) and each row is strictly ascending.  Synchronises
    the current stream."""
    B, H, N, d = Q.shape
    nb = -(-N // BLOCK)
    if idx.dtype != torch.int32 or idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, nb):
        raise ValueError("idx must be int32 [B, H, n_b, topk]")
    idx = idx.contiguous()
    st = lib().sla_validate_idx(ctypes.byref(_problem(Q, idx.shape[3])), _ptr(idx), _stream())
    if st == SLA_ERR_INVALID:
        return False
    if st != SLA_OK:
        raise SLAError(st, "sla_validate_idx")
    return True


def route(Q, K, proj_q, proj_k, topk: int, want_mask: bool = False, want_scores: bool = False,
          workspace=None, idx_out=None):
    """Router: block mean-pool, projection, block scores, HardTop-k.  Returns (idx, mask,
    scores); mask / scores are None unless requested."""
    _check_qkv(Q, K)
    Q, K = Q.contiguous(), K.contiguous()
    proj_q = proj_q.contiguous().to(torch.float32)
    proj_k = proj_k.contiguous().to(torch.float32)
    B, H, N, d = Q.shape
    nb = -(-N // BLOCK)
    p = _problem(Q, topk)
    dev = Q.device
    idx = idx_out if idx_out is not None else torch.empty((B, H, nb, topk), dtype=torch.int32, device=dev)
    mask = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=dev) if want_mask else None
    scores = torch.empty((B, H, nb, nb), dtype=torch.float32, device=dev) if want_scores else None
    need = lib().sla_route_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().sla_route(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(proj_q), _ptr(proj_k), _ptr(idx),
                         _ptr(mask), _ptr(scores), _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_route")
    return idx, mask, scores


def route_noalloc(Q, K, proj_q, proj_k, idx, mask=None, scores=None):
    """The router on the library's static per-GPU scratch (sla_route_noalloc): no workspace, and
    the caller passes every output (idx [B, H, n_b, topk] int32; mask, scores optional), so the
    call allocates nothing.  Q, K, proj_q and proj_k must already be contiguous, with proj_q and
    proj_k in float32.  Calls that overlap on one GPU share the scratch and race."""
    _check_qkv(Q, K)
    for t in (Q, K, proj_q, proj_k, idx):
        if not t.is_contiguous():
            raise ValueError("route_noalloc takes contiguous tensors")
    if proj_q.dtype != torch.float32 or proj_k.dtype != torch.float32 or idx.dtype != torch.int32:
        raise ValueError("route_noalloc takes float32 projections and an int32 idx")
    p = _problem(Q, idx.shape[-1])
    st = lib().sla_route_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(proj_q), _ptr(proj_k),
                                 _ptr(idx), _ptr(mask), _ptr(scores), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_route_noalloc")
    return idx, mask, scores


def forward(Q, K, V, idx, alpha, fp8: bool = False, linear_mode: str = "fused", workspace=None,
            out=None, events=None, state_events=None, drop_tau=None, int8: bool = False,
            idx_ready=None, out_rows=None):
    """O = alpha * O_s + (1 - alpha) * O_l.  `events` = (begin, end) torch.cuda.Event pair
    recorded around the sparse kernel, `state_events` likewise around the linear-state kernels
    (the events must already exist, e.g. recorded once).  drop_tau (0 <= tau < 0.5, bf16
    mask-product mode): per (b, h), drop the linear branch when max(1 - alpha) <= tau and the
    sparse branch when max(alpha) <= tau, decided on the GPU.  idx_ready (a recorded
    torch.cuda.Event): the linear states are built at once and the stream waits for the event
    only before idx is read, so a router on another stream overlaps them.  out_rows ([B, H, N]
    int32 permutation, bf16 mask-product mode): output row r is written to row out_rows[r]."""
    _check_qkv(Q, K, V)
    Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
    B, H, N, d = Q.shape
    topk = idx.shape[-1]
    idx = idx.contiguous().to(torch.int32)
    alpha = alpha.contiguous().to(torch.float32)
    p = _problem(Q, topk)
    mode = LINEAR_MODES[linear_mode]
    if fp8 and int8:
        raise ValueError("fp8 and int8 exclude each other")
    variant = 5 if int8 else ((4 if mode == 2 else 1) if fp8 else {0: 0, 1: 2, 2: 3}[mode])
    need = lib().sla_forward_workspace_bytes(ctypes.byref(p), variant)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    O = out if out is not None else torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device)
    opts = ForwardOpts(mode, None, None, None, None, 0 if drop_tau is None else 1,
                       0.0 if drop_tau is None else float(drop_tau))
    if events is not None:
        opts.sparse_begin = ctypes.c_void_p(events[0].cuda_event)
        opts.sparse_end = ctypes.c_void_p(events[1].cuda_event)
    if state_events is not None:
        opts.states_begin = ctypes.c_void_p(state_events[0].cuda_event)
        opts.states_end = ctypes.c_void_p(state_events[1].cuda_event)
    if idx_ready is not None:
        opts.idx_ready = ctypes.c_void_p(idx_ready.cuda_event)
    if out_rows is not None:
        out_rows = out_rows.contiguous().to(torch.int32)
        if tuple(out_rows.shape) != (B, H, N) or out_rows.device != Q.device:
            raise ValueError("out_rows must be [B, H, N] on the inputs' device")
        opts.out_rows = _ptr(out_rows)
    fn = lib().sla_forward_int8_ex if int8 else (lib().sla_forward_fp8_ex if fp8 else lib().sla_forward_ex)
    st = fn(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(alpha), _ptr(O), _ptr(ws),
            ws.numel(), _stream(), ctypes.byref(opts))
    if st != SLA_OK:
        raise SLAError(st, "sla_forward_int8" if int8 else ("sla_forward_fp8" if fp8 else "sla_forward"))
    return O


def backward(Q, K, V, idx, alpha, dO, workspace=None, want_O=False, out=None):
    """Gradients (dQ, dK, dV, dalpha) of O = alpha O_s + (1 - alpha) O_l for the kept sets idx
    (bf16, d = 128); the forward is recomputed on the GPU.  Returns (dQ, dK, dV, dalpha[, O])."""
    _check_qkv(Q, K, V, dO)
    Q, K, V, dO = Q.contiguous(), K.contiguous(), V.contiguous(), dO.contiguous()
    B, H, N, d = Q.shape
    topk = idx.shape[-1]
    idx = idx.contiguous().to(torch.int32)
    alpha = alpha.contiguous().to(torch.float32)
    p = _problem(Q, topk)
    need = lib().sla_backward_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    if out is None:
        out = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device) for _ in range(3)) + (
            torch.empty((B, H, N), dtype=torch.float32, device=Q.device),)
    dQ, dK, dV, da = out
    O = torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device) if want_O else None
    st = lib().sla_backward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(alpha), _ptr(dO),
                            _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(da), _ptr(O), _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_backward")
    return (dQ, dK, dV, da, O) if want_O else (dQ, dK, dV, da)


def soft_workspace_bytes(Q, topk: int) -> int:
    return lib().sla_soft_workspace_bytes(ctypes.byref(_problem(Q, topk)))


def _soft_ws(p, dev, workspace):
    need = lib().sla_soft_workspace_bytes(ctypes.byref(p))
    if need == 0:
        raise SLAError(SLA_ERR_UNSUPPORTED, "sla_soft_workspace_bytes")
    return workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)


def soft_route(Q, K, proj_q, proj_k, topk: int, temperature: float, workspace=None, out=None):
    """SoftTop-k router (training): the soft mask M [B, H, n_b, n_b] fp32 with row sums topk."""
    _check_qkv(Q, K)
    Q, K = Q.contiguous(), K.contiguous()
    proj_q = proj_q.contiguous().to(torch.float32)
    proj_k = proj_k.contiguous().to(torch.float32)
    B, H, N, d = Q.shape
    nb = -(-N // BLOCK)
    p = _problem(Q, topk)
    ws = _soft_ws(p, Q.device, workspace)
    M = out if out is not None else torch.empty((B, H, nb, nb), dtype=torch.float32, device=Q.device)
    st = lib().sla_soft_route(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(proj_q), _ptr(proj_k), float(temperature),
                              _ptr(M), _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_soft_route")
    return M


def soft_forward(Q, K, V, M, alpha, workspace=None, out=None):
    """Soft-mask forward: O = alpha O_s + (1 - alpha) O_l, key block j of query block i weighted
    by M[i][j] in the sparse branch and 1 - M[i][j] in the linear one."""
    _check_qkv(Q, K, V)
    Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
    M = M.contiguous().to(torch.float32)
    alpha = alpha.contiguous().to(torch.float32)
    B, H, N, d = Q.shape
    p = _problem(Q, 0)
    ws = _soft_ws(p, Q.device, workspace)
    O = out if out is not None else torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device)
    st = lib().sla_soft_forward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(M), _ptr(alpha), _ptr(O),
                                _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_soft_forward")
    return O


def soft_backward(Q, K, V, proj_q, proj_k, temperature: float, M, alpha, dO, topk: int,
                  want_dM: bool = True, workspace=None):
    """Gradients of <dO, O> for the soft forward with M = soft_route(..., topk, temperature):
    returns (dproj_q, dproj_k, dalpha, dM or None)."""
    _check_qkv(Q, K, V, dO)
    Q, K, V, dO = Q.contiguous(), K.contiguous(), V.contiguous(), dO.contiguous()
    proj_q = proj_q.contiguous().to(torch.float32)
    proj_k = proj_k.contiguous().to(torch.float32)
    M = M.contiguous().to(torch.float32)
    alpha = alpha.contiguous().to(torch.float32)
    B, H, N, d = Q.shape
    nb = -(-N // BLOCK)
    p = _problem(Q, topk)
    ws = _soft_ws(p, Q.device, workspace)
    dev = Q.device
    dWq = torch.empty((d, d), dtype=torch.float32, device=dev)
    dWk = torch.empty((d, d), dtype=torch.float32, device=dev)
    da = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dM = torch.empty((B, H, nb, nb), dtype=torch.float32, device=dev) if want_dM else None
    st = lib().sla_soft_backward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(proj_q), _ptr(proj_k),
                                 float(temperature), _ptr(M), _ptr(alpha), _ptr(dO), _ptr(dWq), _ptr(dWk),
                                 _ptr(da), _ptr(dM), None, _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_soft_backward")
    return dWq, dWk, da, dM


def stage1_step(Q, K, V, O_full, proj_q, proj_k, alpha, topk: int, temperature: float,
                lr_proj: float, lr_alpha: float, workspace=None, loss=None):
    """One stage-1 step in place on proj_q, proj_k, alpha (fp32 contiguous GPU tensors); returns
    the step's loss (before the update) as a one-element GPU tensor."""
    _check_qkv(Q, K, V)
    for t in (proj_q, proj_k, alpha, O_full):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != Q.device:
            raise ValueError("proj_q, proj_k, alpha, O_full must be contiguous fp32 tensors on the inputs' device")
    Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
    p = _problem(Q, topk)
    ws = _soft_ws(p, Q.device, workspace)
    loss = loss if loss is not None else torch.empty(1, dtype=torch.float32, device=Q.device)
    st = lib().sla_stage1_step(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(O_full), _ptr(proj_q),
                               _ptr(proj_k), _ptr(alpha), float(temperature), float(lr_proj), float(lr_alpha),
                               _ptr(loss), _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_stage1_step")
    return loss


def quantize_int8(X):
    """Per-(b, h, 64-token block) absmax int8 codes of X (bf16, d = 128) and their scales."""
    _check_qkv(X)
    X = X.contiguous()
    B, H, N, d = X.shape
    nb = -(-N // BLOCK)
    codes = torch.empty((B, H, N, d), dtype=torch.int8, device=X.device)
    scales = torch.empty((B, H, nb), dtype=torch.float32, device=X.device)
    p = _problem(X, 0)
    st = lib().sla_quantize_int8(ctypes.byref(p), _ptr(X), _ptr(codes), _ptr(scales), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_quantize_int8")
    return codes, scales


def quantize_e4m3(X):
    """Per-(b, h, 64-token block) absmax e4m3 codes of X (bf16, d = 128) and their scales."""
    _check_qkv(X)
    X = X.contiguous()
    B, H, N, d = X.shape
    nb = -(-N // BLOCK)
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=X.device)
    scales = torch.empty((B, H, nb), dtype=torch.float32, device=X.device)
    p = _problem(X, 0)
    st = lib().sla_quantize_e4m3(ctypes.byref(p), _ptr(X), _ptr(codes), _ptr(scales), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_quantize_e4m3")
    return codes, scales


class PisaStats:
    """The PISA statistics buffer of one K, V (written by pisa_stats) with typed views:
    kbar_hi, kbar_lo, vsum [B, H, n_b, d] bf16; hbar_t [B, H, d, d] bf16 (Hbar transposed);
    hbar [B, H, d, d] fp32; M, lnM [B, H, n_b] fp32."""

    _NAMES = ("kbar_hi", "kbar_lo", "vsum", "hbar_t", "hbar", "M", "lnM")

    def __init__(self, buf, shape, offsets):
        self.buf = buf
        self.shape = shape  # (B, H, N, d)
        B, H, N, d = shape
        nb = -(-N // BLOCK)
        shapes = [(B, H, nb, d)] * 3 + [(B, H, d, d)] * 2 + [(B, H, nb)] * 2
        dtypes = [torch.bfloat16] * 4 + [torch.float32] * 3
        for name, off, shp, dt in zip(self._NAMES, offsets, shapes, dtypes):
            n = 1
            for x in shp:
                n *= x
            nbytes = n * torch.empty((), dtype=dt).element_size()
            setattr(self, name, buf[off : off + nbytes].view(dt).view(shp))


def pisa_workspace_bytes(Q, topk: int = 0) -> int:
    """Scratch bytes of pisa_stats and pisa_route for inputs shaped like Q."""
    return lib().sla_pisa_workspace_bytes(ctypes.byref(_problem(Q, topk)))


def pisa_stats(K, V, workspace=None, out=None) -> PisaStats:
    """PISA statistics pass over K, V [B, H, N, d]: centroids, value sums, Hbar, M_j, ln M_j."""
    _check_qkv(K, V)
    K, V = K.contiguous(), V.contiguous()
    p = _problem(K, 0)
    L = lib()
    nbytes = L.sla_pisa_stats_bytes(ctypes.byref(p))
    offs = (ctypes.c_size_t * 7)()
    st = L.sla_pisa_stats_offsets(ctypes.byref(p), offs)
    if st != SLA_OK:
        raise SLAError(st, "sla_pisa_stats_offsets")
    buf = out if out is not None else torch.empty(max(nbytes, 1), dtype=torch.uint8, device=K.device)
    need = L.sla_pisa_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=K.device)
    st = L.sla_pisa_stats(ctypes.byref(p), _ptr(K), _ptr(V), _ptr(buf), buf.numel(), _ptr(ws),
                          ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_pisa_stats")
    return PisaStats(buf, tuple(K.shape), list(offs))


def pisa_route(Q, stats: PisaStats, topk: int, covariance: bool = True, want_mask: bool = False,
               want_scores: bool = False, workspace=None, idx_out=None):
    """Covariance-aware HardTop-k of PISA.  Returns (idx, mask, scores); scores are the ranked
    selection scores (qbar . kbar / sqrt(d) [+ ln M_j]); mask / scores None unless requested."""
    _check_qkv(Q)
    Q = Q.contiguous()
    if tuple(Q.shape) != stats.shape:
        raise ValueError("Q must have the shape of the K, V the statistics were taken from")
    B, H, N, d = Q.shape
    nb = -(-N // BLOCK)
    p = _problem(Q, topk)
    dev = Q.device
    idx = idx_out if idx_out is not None else torch.empty((B, H, nb, topk), dtype=torch.int32, device=dev)
    mask = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=dev) if want_mask else None
    scores = torch.empty((B, H, nb, nb), dtype=torch.float32, device=dev) if want_scores else None
    need = lib().sla_pisa_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().sla_pisa_route(ctypes.byref(p), _ptr(Q), _ptr(stats.buf), stats.buf.numel(),
                              1 if covariance else 0, _ptr(idx), _ptr(mask), _ptr(scores), _ptr(ws),
                              ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_pisa_route")
    return idx, mask, scores


def pisa_forward(Q, K, V, stats: PisaStats, idx, out=None):
    """PISA forward: exact attention over the kept blocks, zero-order block terms plus the
    global first-order Hbar correction over the rest.  Returns O [B, H, N, d] fp32."""
    _check_qkv(Q, K, V)
    Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
    if tuple(Q.shape) != stats.shape:
        raise ValueError("Q, K, V must have the shape the statistics were taken from")
    B, H, N, d = Q.shape
    topk = idx.shape[-1]
    idx = idx.contiguous().to(torch.int32)
    p = _problem(Q, topk)
    O = out if out is not None else torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device)
    st = lib().sla_pisa_forward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(stats.buf),
                                stats.buf.numel(), _ptr(idx), _ptr(O), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_pisa_forward")
    return O


def svoo_workspace_bytes(Q) -> int:
    return lib().sla_svoo_workspace_bytes(ctypes.byref(_problem(Q, 0)))


def svoo_cluster(Q, K, iters: int = 3, workspace=None, out=None):
    """SVOO co-clustering of queries and keys (bf16, d = 128): returns (perm_q, perm_k, q_assign,
    k_assign), all [B, H, N] int32; perm maps a position of the cluster-sorted sequence to the
    original token."""
    _check_qkv(Q, K)
    Q, K = Q.contiguous(), K.contiguous()
    B, H, N, d = Q.shape
    p = _problem(Q, 0)
    need = lib().sla_svoo_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    if out is None:
        out = tuple(torch.empty((B, H, N), dtype=torch.int32, device=Q.device) for _ in range(4))
    pq, pk, qa, ka = out
    st = lib().sla_svoo_cluster(ctypes.byref(p), _ptr(Q), _ptr(K), int(iters), _ptr(qa), _ptr(ka), _ptr(pq),
                                _ptr(pk), _ptr(ws), ws.numel(), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_svoo_cluster")
    return pq, pk, qa, ka


def _permute(X, perm, out, scatter):
    if X.device.type != "cuda" or X.dim() < 3:
        raise ValueError("X must be a GPU tensor [B, H, N, ...]")
    X = X.contiguous()
    B, H, N = X.shape[:3]
    perm = perm.contiguous().to(torch.int32)
    if tuple(perm.shape) != (B, H, N):
        raise ValueError("perm must be [B, H, N]")
    row_bytes = X.element_size() * (X.numel() // max(B * H * N, 1))
    Y = out if out is not None else torch.empty_like(X)
    p = make_problem(B, H, N, 128, 0, torch.bfloat16)
    fn = lib().sla_svoo_scatter if scatter else lib().sla_svoo_gather
    st = fn(ctypes.byref(p), _ptr(X), int(row_bytes), _ptr(perm), _ptr(Y), _stream())
    if st != SLA_OK:
        raise SLAError(st, "sla_svoo_scatter" if scatter else "sla_svoo_gather")
    return Y


def svoo_gather(X, perm, out=None):
    """Y[b, h, p] = X[b, h, perm[b, h, p]] for the rows of X [B, H, N, ...]."""
    return _permute(X, perm, out, 0)


def svoo_scatter(X, perm, out=None):
    """Y[b, h, perm[b, h, p]] = X[b, h, p] for the rows of X [B, H, N, ...]."""
    return _permute(X, perm, out, 1)


def svoo_forward(Q, K, V, proj_q, proj_k, alpha, topk: int, perm_q, perm_k, linear_mode: str = "mask_product",
                 out=None):
    """The SLA2 path on co-clustered blocks: Q and alpha gathered by perm_q, K and V by perm_k,
    route and forward on the permuted sequence, output rows scattered back.  Returns (O in the
    original query order, idx of the permuted blocks)."""
    Qp, Kp, Vp = svoo_gather(Q, perm_q), svoo_gather(K, perm_k), svoo_gather(V, perm_k)
    ap = svoo_gather(alpha.contiguous().to(torch.float32), perm_q)
    idx, _, _ = route(Qp, Kp, proj_q, proj_k, topk)
    if linear_mode == "mask_product" and Q.dtype == torch.bfloat16:
        # the forward's epilogue writes each row straight to its original position
        return forward(Qp, Kp, Vp, idx, ap, linear_mode=linear_mode, out=out, out_rows=perm_q), idx
    Op = forward(Qp, Kp, Vp, idx, ap, linear_mode=linear_mode)
    return svoo_scatter(Op, perm_q, out=out), idx
