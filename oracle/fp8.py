"""fp8 (QAT-forward) sparse branch of the SLA2 forward, in float64 around an exact e4m3 codec.

TEST INFRASTRUCTURE ONLY (see the package docstring).

SLA2 (Italian summary) section 2.C and (Arabic summary) section 2.jim: low-bit attention (INT8
or FP8) is used in the sparse branch only, and the forward pass quantises Q, K, P and V.
The pages fix neither the format nor the scale granularity; the readings used here are:

  * format: OCP E4M3FN (bias 7, three mantissa bits, largest finite 448, subnormals down to
    2^-9, no infinities), round to nearest even, saturating at +-448;
  * Q, K, V: one scale per (batch, head, 64-token block) over all channels.  With a = max|x|
    over the block's valid rows, inv = fp32(448 / a), s = fp32(a / 448),
    code = e4m3(fp32(x * inv)); an all-zero block gets s = 1 and codes 0;
  * P: the unnormalised probabilities P^ = exp(S - m) use the exact row maximum m over all
    kept keys; one scale per (query block x KV block) tile, sP = max(tile) / 448, codes
    e4m3(P^ / sP);
  * O_s = sum_j (P8 * sP) @ (V8_j * sV_j) / sum P^, the denominator over the unquantised P^;
  * the router and the linear branch keep the unquantised inputs.
"""

from __future__ import annotations

import numpy as np

from .sla import _f64, block_ranges, block_states, forward_head

__all__ = [
    "E4M3_MAX",
    "e4m3_encode",
    "e4m3_decode",
    "quantize_blocks",
    "forward_fp8_head",
    "forward_fp8",
]

E4M3_MAX = 448.0
_E4M3_BIAS = 7
_E4M3_MIN_NORMAL_EXP = -6  # smallest normal is 2^-6
_E4M3_SUB_STEP = 2.0 ** -9  # subnormal spacing


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3FN encoding (sign, 4 exponent bits with bias 7, 3 mantissa bits) of float values.

    Round to nearest, ties to even; magnitudes at or above 448 saturate to 448 (code 0x7E);
    NaN maps to 0x7F.  Works on the exact float64 value of its input, so a float32 input is
    encoded from its own value with a single rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    code = np.zeros(x.shape, dtype=np.int64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    sat = a >= E4M3_MAX
    normal = (a >= 2.0 ** _E4M3_MIN_NORMAL_EXP) & ~sat
    sub = ~normal & ~sat
    # subnormals (and zero): value = m * 2^-9 with m in 0..7; m = 8 is the smallest normal,
    # whose code is exactly 8, so the integer carries straight into the exponent field
    code = np.where(sub, np.rint(np.where(sub, a, 0.0) / _E4M3_SUB_STEP).astype(np.int64), code)
    # normals: a = (1 + f) * 2^e, mantissa field = rint(8 f); a carry to 8 bumps the exponent
    mant, e2 = np.frexp(np.where(normal, a, 1.0))  # a = mant * 2^e2, mant in [0.5, 1)
    e = e2 - 1
    m8 = np.rint((mant * 2.0 - 1.0) * 8.0).astype(np.int64)
    e = np.where(m8 == 8, e + 1, e)
    m8 = np.where(m8 == 8, 0, m8)
    ncode = ((e + _E4M3_BIAS) << 3) | m8
    code = np.where(normal, ncode, code)
    # rounding past 448 (only possible from below 448 when it rounds up to 480) saturates too
    code = np.where(sat | (code > 0x7E), 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Value of OCP E4M3FN codes as float64; 0x7F and 0xFF are NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    val = np.where(
        E == 0,
        M * _E4M3_SUB_STEP,
        (1.0 + M / 8.0) * np.exp2((E - _E4M3_BIAS).astype(np.float64)),
    )
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def quantize_blocks(X, block: int = 64, codec=None):
    """Per-(block) absmax quantisation of one head's [N, d] tensor to e4m3.

    SLA2 (Arabic summary) section 2.jim: the forward pass quantises Q, K and V.
    Returns (codes uint8 [N, d], scales float32 [n_b]).  ``codec`` (float32 array -> float64
    values) replaces encode+decode for the structural pin; by default the codes are the e4m3
    encoding and the dequantised values are decode(codes) * scale.
    """
    X = _f64(X)
    starts, ends, _ = block_ranges(X.shape[0], block)
    codes = np.zeros(X.shape, dtype=np.uint8)
    deq = np.zeros(X.shape)
    scales = np.ones(len(starts), dtype=np.float32)
    for t, (a, b) in enumerate(zip(starts, ends)):
        xb = X[a:b].astype(np.float32)  # exact: the inputs are bf16 or fp32 values
        amax = np.float32(np.abs(xb).max())
        if amax == 0:
            continue  # scale 1, codes 0
        inv = np.float32(np.float32(E4M3_MAX) / amax)
        scales[t] = np.float32(amax / np.float32(E4M3_MAX))
        y = (xb * inv).astype(np.float32)
        if codec is None:
            codes[a:b] = e4m3_encode(y)
            deq[a:b] = e4m3_decode(codes[a:b]) * np.float64(scales[t])
        else:
            deq[a:b] = codec(y) * np.float64(scales[t])
    return codes, scales, deq


def forward_fp8_head(Q, K, V, idx, alpha, block: int = 64, q_blocks=None, codec=None, states=None, trace=None):
    """SLA2 output rows of one head with the sparse branch on quantised Q, K, P, V.

    SLA2 (Italian summary) section 2.C, (Arabic summary) section 2.jim: low-bit attention in the
    sparse branch only; the forward pass quantises Q, K, P and V.  The linear branch and the
    combine are those of forward_head (unquantised inputs).  ``codec`` replaces the e4m3
    encode/decode pair (identity: the structural pin).  Returns (O, O_s, O_l) lists of [r_i, d].
    ``trace``, a list, receives (query block, key block, P^ tile, sP) for every kept tile: the
    values the P codes are rounded from, exposed for tests that bound the effect of rounding.
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
    _, sq, Qd = quantize_blocks(Q64, block, codec)
    _, sk, Kd = quantize_blocks(K64, block, codec)
    _, sv, Vd = quantize_blocks(V64, block, codec)
    enc = (lambda y: e4m3_decode(e4m3_encode(y))) if codec is None else codec
    scale = 1.0 / np.sqrt(d)
    outs, outs_s = [], []
    for n, i in enumerate(q_blocks):
        a, b = starts[i], ends[i]
        sel = np.asarray(idx[i], dtype=np.int64)
        if len(sel) == 0:
            o_s = np.zeros((b - a, V64.shape[1]))
        else:
            # Qd, Kd already carry their block scales: S = (Q8 K8^T) sQ_i sK_j / sqrt(d)
            S = [(Qd[a:b] @ Kd[starts[j]:ends[j]].T) * scale for j in sel]
            m = np.max([s.max(axis=1) for s in S], axis=0)[:, None]
            P = [np.exp(s - m) for s in S]
            den = np.sum([p.sum(axis=1) for p in P], axis=0)[:, None]
            num = np.zeros((b - a, V64.shape[1]))
            for p, j in zip(P, sel):
                sP = p.max() / E4M3_MAX
                if trace is not None:
                    trace.append((i, int(j), p, sP))
                if sP == 0:
                    continue
                num += (enc(p / sP) * sP) @ Vd[starts[j]:ends[j]]
            o_s = num / den
        al = alpha[a:b, None]
        outs.append(al * o_s + (1.0 - al) * O_l[n])
        outs_s.append(o_s)
    return outs, outs_s, O_l


def forward_fp8(Q, K, V, idx, alpha, block: int = 64, codec=None):
    """Whole fp8-sparse-branch forward over [B, H, N, d]; returns (O, O_s, O_l) float64."""
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
            o, os_, ol = forward_fp8_head(
                Q[bb, hh], K[bb, hh], V[bb, hh], idx[bb, hh], alpha[bb, hh], block, codec=codec
            )
            O[bb, hh] = np.concatenate(o)
            Os[bb, hh] = np.concatenate(os_)
            Ol[bb, hh] = np.concatenate(ol)
    return O, Os, Ol
