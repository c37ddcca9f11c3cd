"""INT8 (QAT-forward) sparse branch of the SLA2 forward, in float64 around an exact int8 codec.

TEST INFRASTRUCTURE ONLY (see the package docstring).

SLA2 (Italian summary) section 2.C and (Arabic summary) section 2.jim: low-bit attention, INT8 or
FP8, in the sparse branch only; the forward pass quantises Q, K, P and V.  The e4m3 variant is in
fp8.py; this is the INT8 one, with the same granularity readings:

  * codes: symmetric signed 8-bit integers in [-127, 127] (-128 unused, so the grid is
    symmetric), round to nearest, ties to even, saturating;
  * Q, K, V: one scale per (batch, head, 64-token block) over all channels.  With a = max|x|
    over the block's valid rows, inv = fp32(127 / a), s = fp32(a / 127),
    code = int8(fp32(x * inv)); an all-zero block gets s = 1 and codes 0;
  * P: P^ = exp(S - m) with the exact row maximum m over all kept keys; one scale per (query
    block x KV block) tile, sP = max(tile) / 127, codes int8(P^ / sP) in [0, 127];
  * S = (Q8 K8^T) sQ sK / sqrt(d) and O_s = sum_j (P8 V8_j) sP sV_j / sum P^: the integer
    products are exact, the denominator sums the unquantised P^;
  * the router and the linear branch keep the unquantised inputs.
"""

from __future__ import annotations

import numpy as np

from .sla import _f64, block_ranges, block_states, forward_head

__all__ = ["INT8_MAX", "int8_encode", "quantize_blocks_int8", "forward_int8_head", "forward_int8"]

INT8_MAX = 127.0


def int8_encode(y) -> np.ndarray:
    """Signed 8-bit codes of float values: round to nearest, ties to even, saturating at +-127."""
    y = np.asarray(y, dtype=np.float64)
    return np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8)


def quantize_blocks_int8(X, block: int = 64):
    """Per-(block) absmax quantisation of one head's [N, d] tensor to int8.

    SLA2 (Arabic summary) section 2.jim: the forward pass quantises Q, K and V.
    Returns (codes int8 [N, d], scales float32 [n_b], dequantised float64 [N, d]).
    """
    X = _f64(X)
    starts, ends, _ = block_ranges(X.shape[0], block)
    codes = np.zeros(X.shape, dtype=np.int8)
    deq = np.zeros(X.shape)
    scales = np.ones(len(starts), dtype=np.float32)
    for t, (a, b) in enumerate(zip(starts, ends)):
        xb = X[a:b].astype(np.float32)  # exact: the inputs are bf16 or fp32 values
        amax = np.float32(np.abs(xb).max())
        if amax == 0:
            continue  # scale 1, codes 0
        inv = np.float32(np.float32(INT8_MAX) / amax)
        scales[t] = np.float32(amax / np.float32(INT8_MAX))
        codes[a:b] = int8_encode((xb * inv).astype(np.float32))
        deq[a:b] = codes[a:b].astype(np.float64) * np.float64(scales[t])
    return codes, scales, deq


def forward_int8_head(Q, K, V, idx, alpha, block: int = 64, q_blocks=None, states=None, trace=None):
    """SLA2 output rows of one head with the sparse branch on int8 Q, K, P, V.

    SLA2 (Italian summary) section 2.C, (Arabic summary) section 2.jim.  The linear branch and
    the combine are those of forward_head (unquantised inputs).  Returns (O, O_s, O_l) lists of
    [r_i, d] float64 arrays in the order of q_blocks.  ``trace``, a list, receives (query block,
    key block, P^ tile, sP) for every kept tile (as in forward_fp8_head).
    """
    Q64 = _f64(Q)
    K64 = _f64(K)
    V64 = _f64(V)
    alpha = _f64(alpha)
    idx = np.asarray(idx)
    N, d = Q64.shape
    starts, ends, _ = block_ranges(N, block)
    n_b = len(starts)
    if q_blocks is None:
        q_blocks = list(range(n_b))
    if states is None:
        states = block_states(K64, V64, block)
    _, _, O_l = forward_head(Q64, K64, V64, idx, alpha, block, q_blocks=q_blocks, states=states)
    q8, sq, _ = quantize_blocks_int8(Q64, block)
    k8, sk, _ = quantize_blocks_int8(K64, block)
    v8, sv, _ = quantize_blocks_int8(V64, block)
    q8, k8, v8 = (x.astype(np.int64) for x in (q8, k8, v8))
    scale = 1.0 / np.sqrt(d)
    outs, outs_s = [], []
    for n, i in enumerate(q_blocks):
        a, b = starts[i], ends[i]
        sel = np.asarray(idx[i], dtype=np.int64)
        if len(sel) == 0:
            o_s = np.zeros((b - a, V64.shape[1]))
        else:
            # exact integer products, then the block scales
            S = [(q8[a:b] @ k8[starts[j]:ends[j]].T).astype(np.float64) * (float(sq[i]) * float(sk[j]) * scale)
                 for j in sel]
            m = np.max([s.max(axis=1) for s in S], axis=0)[:, None]
            P = [np.exp(s - m) for s in S]
            den = np.sum([p.sum(axis=1) for p in P], axis=0)[:, None]
            num = np.zeros((b - a, V64.shape[1]))
            for p, j in zip(P, sel):
                sP = p.max() / INT8_MAX
                if trace is not None:
                    trace.append((i, int(j), p, sP))
                if sP == 0:
                    continue
                p8 = int8_encode(p / sP).astype(np.int64)
                num += (p8 @ v8[starts[j]:ends[j]]).astype(np.float64) * (sP * float(sv[j]))
            o_s = num / den
        al = alpha[a:b, None]
        outs.append(al * o_s + (1.0 - al) * O_l[n])
        outs_s.append(o_s)
    return outs, outs_s, O_l


def forward_int8(Q, K, V, idx, alpha, block: int = 64):
    """Whole int8-sparse-branch forward over [B, H, N, d]; returns (O, O_s, O_l) float64."""
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    alpha = _f64(alpha)
    idx = np.asarray(idx)
    B, H, N, _ = Q.shape
    shape = (B, H, N, V.shape[-1])
    O = np.empty(shape)
    Os = np.empty(shape)
    Ol = np.empty(shape)
    for bb in range(B):
        for hh in range(H):
            o, os_, ol = forward_int8_head(Q[bb, hh], K[bb, hh], V[bb, hh], idx[bb, hh], alpha[bb, hh], block)
            O[bb, hh] = np.concatenate(o)
            Os[bb, hh] = np.concatenate(os_)
            Ol[bb, hh] = np.concatenate(ol)
    return O, Os, Ol
