"""Pins of the CPU oracle: checks against something other than the oracle itself.

Each ``pin_*`` takes the oracle module (the real one, or a planted mutant in
test_oracle_mutations.py) and raises AssertionError when the oracle disagrees with a library
routine, a closed form, a hand-derived worked example under tests/golden/, dense brute force on
a tiny input, or an invariant of the method.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _rand_idx(n_b, k, seed, rows=None):
    rng = np.random.default_rng(seed)
    rows = n_b if rows is None else rows
    return np.stack([np.sort(rng.choice(n_b, size=k, replace=False)) for _ in range(rows)]).astype(np.int32)


def _sdpa(Q, K, V, mask=None):
    """torch's scaled_dot_product_attention on CPU in float64 (its math path)."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m).numpy()


# ----------------------------------------------------------------------------------------------
# whole-output reductions


def pin_full_attention(orc):
    """All blocks kept and alpha = 1: the output is full softmax attention (torch SDPA)."""
    N, d, blk = 200, 16, 64  # 4 blocks, the last one 8 tokens
    Q, K, V = (_rand((N, d), s) for s in (1, 2, 3))
    n_b = -(-N // blk)
    idx = np.tile(np.arange(n_b, dtype=np.int32), (n_b, 1))
    O, O_s, O_l = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], np.ones((1, 1, N)), blk)
    ref = _sdpa(Q, K, V)
    np.testing.assert_allclose(O[0, 0], ref, rtol=0, atol=1e-12)
    assert np.all(O_l == 0.0), "an empty unselected set must give a zero linear branch"


def pin_linear_attention(orc):
    """Nothing kept and alpha = 0: plain ReLU linear attention phi(Q)phi(K)^T V / row sums,
    evaluated densely over all N tokens with torch."""
    N, d, blk = 150, 8, 32
    Q, K, V = (_rand((N, d), s) for s in (4, 5, 6))
    n_b = -(-N // blk)
    idx = np.zeros((n_b, 0), dtype=np.int32)
    O, O_s, _ = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], np.zeros((1, 1, N)), blk)
    q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
    w = torch.relu(q) @ torch.relu(k).T
    den = w.sum(dim=1, keepdim=True)
    ref = torch.where(den > 0, (w @ v) / den, torch.zeros_like(v)).numpy()
    assert (den == 0).any() and (den > 0).sum() > N // 2  # both cases occur
    np.testing.assert_allclose(O[0, 0], ref, rtol=1e-12, atol=1e-12)
    assert np.all(O_s == 0.0), "no kept block must give a zero sparse branch"


def pin_sparse_is_masked_sdpa(orc):
    """alpha = 1 with any mask: SDPA with the token-level boolean mask expanded from M."""
    N, d, blk, k = 176, 16, 32, 2  # 6 blocks, last one 16 tokens
    Q, K, V = (_rand((N, d), s, 1.5) for s in (7, 8, 9))
    n_b = -(-N // blk)
    idx = _rand_idx(n_b, k, 10)
    O, _, _ = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], np.ones((1, 1, N)), blk)
    blk_of = np.arange(N) // blk
    mask = np.zeros((N, N), dtype=bool)
    for q in range(N):
        mask[q] = np.isin(blk_of, idx[blk_of[q]])
    np.testing.assert_allclose(O[0, 0], _sdpa(Q, K, V, mask), rtol=0, atol=1e-12)


def pin_dense_brute_force(orc):
    """Tiny inputs: the dense token-level P = alpha P_s + (1 - alpha) P_l, built entry by entry
    with Python loops, is row-stochastic and O = P V."""
    N, d, blk, k = 22, 3, 4, 2  # 6 blocks, the last one 2 tokens
    Q, K, V = (_rand((N, d), s) for s in (11, 12, 13))
    alpha = np.random.default_rng(14).uniform(0.05, 0.95, N)
    n_b = -(-N // blk)
    idx = _rand_idx(n_b, k, 15)
    O, _, _ = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], alpha[None, None], blk)
    P = np.zeros((N, N))
    rowsum = np.zeros(N)  # alpha + (1 - alpha) when the linear denominator is positive, else alpha
    for q in range(N):
        kept = [n for n in range(N) if (n // blk) in set(idx[q // blk].tolist())]
        rest = [n for n in range(N) if n not in kept]
        logit = {n: sum(Q[q, c] * K[n, c] for c in range(d)) / math.sqrt(d) for n in kept}
        mx = max(logit.values())
        zs = sum(math.exp(logit[n] - mx) for n in kept)
        lin = {n: sum(max(Q[q, c], 0.0) * max(K[n, c], 0.0) for c in range(d)) for n in rest}
        zl = sum(lin.values())
        for n in kept:
            P[q, n] += alpha[q] * math.exp(logit[n] - mx) / zs
        for n in rest:
            P[q, n] += (1.0 - alpha[q]) * (lin[n] / zl if zl > 0 else 0.0)
        rowsum[q] = alpha[q] + ((1.0 - alpha[q]) if zl > 0 else 0.0)
    assert np.all(P >= 0)
    assert np.sum(rowsum == 1.0) >= N // 2  # most rows have a positive linear denominator
    np.testing.assert_allclose(P.sum(axis=1), rowsum, atol=1e-12)
    np.testing.assert_allclose(O[0, 0], P @ V, rtol=0, atol=1e-12)
    Pd, _, _ = orc.dense_P(Q, K, idx, alpha, blk)
    np.testing.assert_allclose(Pd, P, rtol=0, atol=1e-12)


def pin_forward_worked_example(orc):
    """The hand-derived worked example in tests/golden/forward_worked_example.json."""
    with open(os.path.join(GOLDEN, "forward_worked_example.json")) as f:
        g = json.load(f)
    a = math.sqrt(2.0) * math.log(2.0)

    def val(x):
        if x == "a":
            return a
        if isinstance(x, str):
            return float(Fraction(x))
        return float(x)

    arr = lambda rows: np.array([[val(x) for x in r] for r in rows])  # noqa: E731
    Q, K, V = arr(g["Q"]), arr(g["K"]), arr(g["V"])
    alpha = np.array(g["alpha"], dtype=np.float64)
    idx = np.array(g["idx"], dtype=np.int32)
    O, O_s, O_l = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], alpha[None, None], g["block"])
    np.testing.assert_allclose(O_s[0, 0], arr(g["expected_O_s"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(O_l[0, 0], arr(g["expected_O_l"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(O[0, 0], arr(g["expected_O"]), rtol=0, atol=1e-12)


def pin_block_constant_closed_form(orc):
    """Keys constant inside each block: both branches reduce to block sums of V.
    O_s = sum_sel r_j-weighted e^{q.k_j/sqrt d} vbar_j / ..., O_l likewise with phi(q).phi(k_j)."""
    N, d, blk, k = 45, 5, 8, 3  # 6 blocks, the last one 5 tokens
    n_b = -(-N // blk)
    kb = _rand((n_b, d), 21)
    K = np.repeat(kb, blk, axis=0)[:N]
    Q, V = _rand((N, d), 22), _rand((N, d), 23)
    alpha = np.random.default_rng(24).uniform(0, 1, N)
    idx = _rand_idx(n_b, k, 25)
    O, _, _ = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], alpha[None, None], blk)
    vsum = np.array([V[j * blk : (j + 1) * blk].sum(axis=0) for j in range(n_b)])
    cnt = np.array([min(blk, N - j * blk) for j in range(n_b)], dtype=np.float64)
    for q in range(N):
        i = q // blk
        sel = list(idx[i])
        uns = [j for j in range(n_b) if j not in sel]
        e = {j: math.exp(float(Q[q] @ kb[j]) / math.sqrt(d)) for j in sel}
        o_s = sum(e[j] * vsum[j] for j in sel) / sum(e[j] * cnt[j] for j in sel)
        w = {j: float(np.maximum(Q[q], 0) @ np.maximum(kb[j], 0)) for j in uns}
        den = sum(w[j] * cnt[j] for j in uns)
        o_l = sum(w[j] * vsum[j] for j in uns) / den if den > 0 else 0.0 * o_s
        np.testing.assert_allclose(O[0, 0, q], alpha[q] * o_s + (1 - alpha[q]) * o_l, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# invariants of the method


def _small_case(seed, N=150, d=8, blk=16, k=3, B=1, H=2):
    """Random inputs whose channel 0 of Q and K is positive, so no linear denominator is 0."""
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    Q[..., 0] = np.abs(Q[..., 0]) + 0.1
    K[..., 0] = np.abs(K[..., 0]) + 0.1
    alpha = rng.uniform(0, 1, (B, H, N))
    n_b = -(-N // blk)
    idx = np.stack([np.stack([_rand_idx(n_b, k, seed + 100 * b + h) for h in range(H)]) for b in range(B)])
    return Q, K, V, alpha, idx, blk


def pin_convexity(orc):
    """Every output row is a convex combination of V rows (the output stays row-normalised)."""
    Q, K, V, alpha, idx, blk = _small_case(31)
    O, _, _ = orc.forward(Q, K, V, idx, alpha, blk)
    lo = V.min(axis=2, keepdims=True)
    hi = V.max(axis=2, keepdims=True)
    assert np.all(O >= lo - 1e-12) and np.all(O <= hi + 1e-12)


def pin_v_affine(orc):
    """O(a V + 1 c^T) = a O(V) + 1 c^T: both branches are row-stochastic and linear in V."""
    Q, K, V, alpha, idx, blk = _small_case(32)
    c = np.random.default_rng(33).standard_normal(V.shape[-1])
    O1, _, _ = orc.forward(Q, K, V, idx, alpha, blk)
    O2, _, _ = orc.forward(Q, K, -2.5 * V + c, idx, alpha, blk)
    np.testing.assert_allclose(O2, -2.5 * O1 + c, rtol=0, atol=1e-11)


def pin_within_block_permutation(orc):
    """Permuting tokens inside blocks (Q, K, V, alpha together) leaves the mask unchanged and
    permutes the output rows the same way."""
    Q, K, V, alpha, idx, blk = _small_case(34)
    rng = np.random.default_rng(35)
    W = [rng.standard_normal((Q.shape[-1],) * 2) for _ in range(2)]
    N = Q.shape[2]
    perm = np.concatenate([s + rng.permutation(min(blk, N - s)) for s in range(0, N, blk)])
    r1 = orc.route(Q, K, W[0], W[1], 3, blk)
    r2 = orc.route(Q[:, :, perm], K[:, :, perm], W[0], W[1], 3, blk)
    assert np.array_equal(r1["idx"], r2["idx"])
    O1, _, _ = orc.forward(Q, K, V, r1["idx"], alpha, blk)
    O2, _, _ = orc.forward(Q[:, :, perm], K[:, :, perm], V[:, :, perm], r1["idx"], alpha[:, :, perm], blk)
    np.testing.assert_allclose(O2, O1[:, :, perm], rtol=0, atol=1e-12)


def pin_alpha_isolates_branches(orc):
    """alpha = 1 returns O_s, alpha = 0 returns O_l, and any alpha mixes them linearly."""
    Q, K, V, alpha, idx, blk = _small_case(36)
    O1, Os, Ol = orc.forward(Q, K, V, idx, np.ones_like(alpha), blk)
    O0, _, _ = orc.forward(Q, K, V, idx, np.zeros_like(alpha), blk)
    Oa, _, _ = orc.forward(Q, K, V, idx, alpha, blk)
    np.testing.assert_array_equal(O1, Os)
    np.testing.assert_array_equal(O0, Ol)
    np.testing.assert_allclose(Oa, alpha[..., None] * O1 + (1 - alpha[..., None]) * O0, atol=1e-13)


# ----------------------------------------------------------------------------------------------
# router


def pin_pool_is_avg_pool(orc):
    """Block means equal torch's avg_pool1d with ceil_mode (a short last window is averaged over
    its valid entries)."""
    X = _rand((2, 3, 203, 5), 41)
    ref = torch.nn.functional.avg_pool1d(
        torch.from_numpy(X).reshape(6, 203, 5).transpose(1, 2), 64, 64, ceil_mode=True
    ).transpose(1, 2).reshape(2, 3, 4, 5).numpy()
    np.testing.assert_allclose(orc.pool_blocks(X, 64), ref, rtol=0, atol=1e-14)


def pin_router_worked_example(orc):
    """The hand-derived router example in tests/golden/router_worked_example.json."""
    with open(os.path.join(GOLDEN, "router_worked_example.json")) as f:
        g = json.load(f)
    blk, d, N = g["block"], g["d"], g["N"]

    def tokens(means, offs):
        rows = []
        for n in range(N):
            rows.append(np.array(means[n // blk], float) + (-1) ** (n % blk) * np.array(offs, float))
        return np.stack(rows)

    Q = tokens(g["q_block_means"], g["q_token_offsets"])
    K = tokens(g["k_block_means"], g["k_token_offsets"])
    r = orc.route(Q, K, np.array(g["Wq"], float), np.array(g["Wk"], float), g["topk"], blk)
    np.testing.assert_allclose(r["scores"], np.array(g["expected_scores"], float), rtol=0, atol=1e-14)
    assert r["idx"].tolist() == g["expected_idx"]
    np.testing.assert_allclose(r["probs"].sum(axis=-1), 1.0, atol=1e-14)


def pin_router_matches_torch_topk(orc):
    """On distinct scores the kept set equals torch.topk's, sorted ascending."""
    Q, K = _rand((1, 2, 700, 16), 42), _rand((1, 2, 700, 16), 43)
    Wq, Wk = _rand((16, 16), 44, 0.25), _rand((16, 16), 45, 0.25)
    k = 5
    r = orc.route(Q, K, Wq, Wk, k, 64)
    qt = torch.nn.functional.avg_pool1d(torch.from_numpy(Q[0]).transpose(1, 2), 64, 64, ceil_mode=True).transpose(1, 2)
    kt = torch.nn.functional.avg_pool1d(torch.from_numpy(K[0]).transpose(1, 2), 64, 64, ceil_mode=True).transpose(1, 2)
    s = torch.matmul(qt @ torch.from_numpy(Wq), (kt @ torch.from_numpy(Wk)).transpose(1, 2)) / 4.0
    ref = torch.sort(torch.topk(s, k, dim=-1).indices, dim=-1).values.numpy()
    assert np.array_equal(r["idx"][0], ref)
    np.testing.assert_allclose(r["probs"][0], torch.softmax(s, dim=-1).numpy(), atol=1e-14)
    assert r["mask"].sum(axis=-1).max() == k and r["mask"].sum(axis=-1).min() == k


def pin_router_invariances(orc):
    """Positive rescaling of proj_q or proj_k, and the presence of V, do not change the mask;
    permuting whole KV blocks permutes the kept indices."""
    Q, K = _rand((1, 1, 512, 8), 46), _rand((1, 1, 512, 8), 47)
    Wq, Wk = _rand((8, 8), 48), _rand((8, 8), 49)
    k = 3
    base = orc.route(Q, K, Wq, Wk, k, 64)["idx"]
    assert np.array_equal(orc.route(Q, K, 3.0 * Wq, Wk, k, 64)["idx"], base)
    assert np.array_equal(orc.route(Q, K, Wq, 0.1 * Wk, k, 64)["idx"], base)
    perm = np.random.default_rng(50).permutation(8)  # block permutation
    Kp = K.reshape(1, 1, 8, 64, 8)[:, :, perm].reshape(1, 1, 512, 8)
    got = orc.route(Q, Kp, Wq, Wk, k, 64)["idx"]
    inv = np.argsort(perm)  # block j of K sits at position inv[j] of Kp
    assert np.array_equal(got[0, 0], np.sort(inv[base[0, 0]], axis=-1))


def pin_router_ties_and_edges(orc):
    """Exact ties keep the lowest block indices; k = 0 keeps nothing; k = n_b keeps all."""
    Q = np.ones((1, 1, 300, 4))
    K = np.ones((1, 1, 300, 4))
    W = np.eye(4)
    r = orc.route(Q, K, W, W, 3, 64)  # every score equal
    assert r["idx"].tolist() == [[[[0, 1, 2]] * 5]]
    assert orc.route(Q, K, W, W, 0, 64)["idx"].shape == (1, 1, 5, 0)
    assert orc.route(Q, K, W, W, 5, 64)["idx"].tolist() == [[[[0, 1, 2, 3, 4]] * 5]]


# ----------------------------------------------------------------------------------------------
# fp8


def _torch_e4m3_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_decode_all_codes(orc):
    """All 254 finite codes decode to torch's float8_e4m3fn values; 0x7F/0xFF are NaN."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin], ref[fin])
    assert orc.e4m3_decode(np.uint8(0x7E)) == 448.0 and orc.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9


def pin_e4m3_encode_exhaustive_bf16(orc):
    """Every bf16 value with |x| < 464 (torch turns larger ones into NaN, the codec saturates)
    encodes to torch's round-to-nearest-even float8_e4m3fn bits."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    ok = np.isfinite(x) & (np.abs(x) < 464.0)
    x = x[ok]
    assert np.array_equal(orc.e4m3_encode(x), _torch_e4m3_bits(x))


def pin_e4m3_encode_fp32_ties_and_saturation(orc):
    """Random fp32 values, exact ties between neighbouring codes, and saturation above 448."""
    rng = np.random.default_rng(51)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-12, 9, 200_000))).astype(np.float32)
    x = x[np.abs(x) < 464]
    assert np.array_equal(orc.e4m3_encode(x), _torch_e4m3_bits(x))
    codes = np.arange(0x7E, dtype=np.uint8)
    v = orc.e4m3_decode(codes)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # exact midpoints: ties go to the even code
    assert np.array_equal(orc.e4m3_encode(mid), _torch_e4m3_bits(mid))
    assert np.all(orc.e4m3_encode(np.array([448.0, 470.0, 1e6, -1e30])) == np.array([0x7E, 0x7E, 0x7E, 0xFE]))
    assert orc.e4m3_encode(np.array([-0.0]))[0] == 0x80


def pin_quantize_blocks(orc):
    """Per-block absmax codes equal torch's e4m3 cast of fp32(x * fp32(448 / absmax)); a zero
    block keeps scale 1 and codes 0; the largest magnitude maps to 448."""
    X = (_rand((150, 16), 52) * 3).astype(np.float32).astype(np.float64)
    X[64:128] = 0.0
    codes, scales, deq = orc.quantize_blocks(X, 64)
    for t, (a, b) in enumerate([(0, 64), (64, 128), (128, 150)]):
        xb = X[a:b].astype(np.float32)
        amax = np.abs(xb).max()
        if amax == 0:
            assert scales[t] == 1.0 and np.all(codes[a:b] == 0)
            continue
        inv = np.float32(448.0) / np.float32(amax)
        assert scales[t] == np.float32(np.float32(amax) / np.float32(448.0))
        assert np.array_equal(codes[a:b], _torch_e4m3_bits(xb * inv))
        assert np.abs(deq[a:b]).max() == np.float64(scales[t]) * 448.0
    np.testing.assert_allclose(deq, X, rtol=0.0625, atol=np.abs(X).max() * 2.0 ** -9)


def pin_fp8_identity_codec(orc):
    """With the e4m3 codec replaced by the identity, the fp8 forward equals the unquantised one
    up to the fp32 rounding of the scales."""
    Q, K, V, alpha, idx, blk = _small_case(53, N=200, d=16, blk=64, k=2)
    O, Os, Ol = orc.forward(Q, K, V, idx, alpha, blk)
    O8, Os8, Ol8 = orc.forward_fp8(Q, K, V, idx, alpha, blk, codec=lambda y: np.asarray(y, np.float64))
    np.testing.assert_array_equal(Ol8, Ol)
    np.testing.assert_allclose(Os8, Os, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(O8, O, rtol=1e-5, atol=1e-6)


def pin_fp8_error_scale(orc):
    """With the real codec the fp8 sparse branch differs from the exact one by the size e4m3
    rounding predicts (three mantissa bits: a few per cent on unconcentrated iid data), and the
    linear branch is untouched."""
    Q, K, V, alpha, idx, blk = _small_case(54, N=256, d=32, blk=64, k=2)
    _, Os, Ol = orc.forward(Q, K, V, idx, alpha, blk)
    _, Os8, Ol8 = orc.forward_fp8(Q, K, V, idx, alpha, blk)
    np.testing.assert_array_equal(Ol8, Ol)
    rel = np.linalg.norm(Os8 - Os) / np.linalg.norm(Os)
    assert 5e-3 < rel < 0.1, rel


def _lowbit_golden(kind):
    """Inputs of tests/golden/lowbit_p_worked_example.json for 'fp8' or 'int8' (the carrier
    value c makes every block's Q, K, V quantisation exact)."""
    with open(os.path.join(GOLDEN, "lowbit_p_worked_example.json")) as f:
        g = json.load(f)
    c = g["carrier"][kind]
    arr = lambda rows: np.array([[c if x == "c" else float(x) for x in r] for r in rows])  # noqa: E731
    return g, arr(g["Q"]), arr(g["K"]), arr(g["V"]), np.array(g["idx"], dtype=np.int32), c


def _lowbit_expected_from_codes(g, kind, V):
    """O_s of the worked example's query block from its hand-listed codes: the sum over keys of
    code * (tile maximum / largest code) * v, over the sum of the unquantised exp(S - m)."""
    qmax = 448.0 if kind == "fp8" else 127.0
    blk = g["block"]
    ex = np.array(g["exponents_S_minus_m"], dtype=np.float64)
    tile = np.exp(np.array(g["tile_max_exponent"], dtype=np.float64))
    deq = np.array(g["codes"][kind], dtype=np.float64) * (tile[np.arange(ex.shape[1]) // blk] / qmax)[None, :]
    return (deq @ V) / np.exp(ex).sum(axis=1, keepdims=True)


def pin_fp8_p_quantisation_worked_example(orc):
    """The hand-derived e4m3 case in tests/golden/lowbit_p_worked_example.json: one P scale per
    (query block x key block) tile, the exact row maximum, the denominator over the unquantised
    P^.  Rows with different maxima inside one tile and a tile holding no row maximum make a
    per-row or per-query-block scale, or a dequantised denominator, give other values."""
    g, Q, K, V, idx, _ = _lowbit_golden("fp8")
    want = np.array(g["expected_O_s"]["fp8"])
    np.testing.assert_allclose(_lowbit_expected_from_codes(g, "fp8", V), want, rtol=0, atol=1e-13)
    qb = g["query_block"]
    _, Os, _ = orc.forward_fp8_head(Q, K, V, idx, np.ones(g["N"]), g["block"], q_blocks=[qb])
    np.testing.assert_allclose(Os[0], want, rtol=0, atol=1e-12)


def pin_int8_p_quantisation_worked_example(orc):
    """The int8 half of tests/golden/lowbit_p_worked_example.json (same readings as the e4m3
    case, largest code 127, round to nearest integer)."""
    g, Q, K, V, idx, _ = _lowbit_golden("int8")
    want = np.array(g["expected_O_s"]["int8"])
    np.testing.assert_allclose(_lowbit_expected_from_codes(g, "int8", V), want, rtol=0, atol=1e-13)
    qb = g["query_block"]
    _, Os, _ = orc.forward_int8_head(Q, K, V, idx, np.ones(g["N"]), g["block"], q_blocks=[qb])
    np.testing.assert_allclose(Os[0], want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# backward (training path)


def _torch_sla_forward(Q, K, V, idx, alpha, blk):
    """A dense float64 torch re-statement of the SLA2 forward of one head (token-level masks),
    written independently of the oracle, for autograd."""
    N, d = Q.shape
    bid = torch.arange(N) // blk
    kept = torch.zeros((N, N), dtype=torch.bool)
    for t in range(N):
        kept[t] = torch.isin(bid, torch.as_tensor(np.asarray(idx[int(bid[t])], dtype=np.int64)))
    x = (Q @ K.T) / math.sqrt(d)
    any_kept = kept.any(dim=1, keepdim=True)
    p = torch.softmax(torch.where(kept, x, torch.full_like(x, -1e300)), dim=1)
    O_s = torch.where(any_kept, p @ V, torch.zeros_like(Q))
    w = (torch.relu(Q) @ torch.relu(K).T) * (~kept)
    num, den = w @ V, w.sum(dim=1, keepdim=True)
    safe = torch.where(den != 0, den, torch.ones_like(den))
    O_l = torch.where(den != 0, num / safe, torch.zeros_like(num))
    a = alpha[:, None]
    return a * O_s + (1 - a) * O_l


def _bwd_case(seed, N=150, d=8, blk=32, k=2):
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    alpha = rng.uniform(0, 1, N)
    n_b = -(-N // blk)
    idx = _rand_idx(n_b, k, seed + 1)
    return Q, K, V, dO, alpha, idx, blk


def pin_backward_matches_autograd(orc):
    """dQ, dK, dV, dalpha equal torch.autograd's gradients of an independent dense torch
    forward (float64), for k in {0, 2, n_b} with a short last block, and rows whose linear
    denominator is exactly 0 (queries with no positive channel)."""
    for seed, k in ((111, 2), (113, 0), (115, 5)):
        Q, K, V, dO, alpha, idx, blk = _bwd_case(seed, k=k)
        Q[3] = -np.abs(Q[3])  # relu(q) = 0: zero linear denominator
        got = orc.backward_head(Q, K, V, idx, alpha, dO, blk)
        ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V, alpha)]
        O = _torch_sla_forward(ts[0], ts[1], ts[2], idx, ts[3], blk)
        (O * torch.from_numpy(dO)).sum().backward()
        for name, gv, tv in zip(("dQ", "dK", "dV", "dalpha"), got, ts):
            np.testing.assert_allclose(gv, tv.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=f"k={k} {name}")


def pin_backward_finite_differences(orc):
    """Central differences of sum(O * dO) through the oracle's own forward match the backward on a
    tiny head (entries kept away from the ReLU kink)."""
    Q, K, V, dO, alpha, idx, blk = _bwd_case(117, N=40, d=4, blk=8, k=2)
    for X in (Q, K):
        X[np.abs(X) < 0.05] += 0.1
    dQ, dK, dV, da = orc.backward_head(Q, K, V, idx, alpha, dO, blk)
    L = lambda Q_, K_, V_, a_: float((orc.forward(Q_[None, None], K_[None, None], V_[None, None], idx[None, None], a_[None, None], blk)[0][0, 0] * dO).sum())  # noqa: E731
    eps = 1e-6
    rng = np.random.default_rng(118)
    for which, G in ((0, dQ), (1, dK), (2, dV)):
        for _ in range(6):
            r, c = rng.integers(0, 40), rng.integers(0, 4)
            args_p = [Q.copy(), K.copy(), V.copy(), alpha.copy()]
            args_m = [Q.copy(), K.copy(), V.copy(), alpha.copy()]
            args_p[which][r, c] += eps
            args_m[which][r, c] -= eps
            fd = (L(*args_p) - L(*args_m)) / (2 * eps)
            assert abs(fd - G[r, c]) < 1e-6 * (1 + abs(fd)), (which, r, c, fd, G[r, c])
    for r in (0, 17, 39):
        ap, am = alpha.copy(), alpha.copy()
        ap[r] += eps
        am[r] -= eps
        fd = (L(Q, K, V, ap) - L(Q, K, V, am)) / (2 * eps)
        assert abs(fd - da[r]) < 1e-6 * (1 + abs(fd)), (r, fd, da[r])


# ----------------------------------------------------------------------------------------------
# int8 sparse branch


def pin_int8_encode_matches_torch_round(orc):
    """Codes of a grid with every half-way point: torch.round (ties to even) clamped to +-127."""
    y = np.arange(-140.0, 140.0, 0.25)
    ref = torch.clamp(torch.round(torch.from_numpy(y)), -127, 127).numpy().astype(np.int8)
    assert np.array_equal(orc.int8_encode(y), ref)
    assert orc.int8_encode(np.array([0.5, 1.5, 2.5, -0.5, -2.5])).tolist() == [0, 2, 2, 0, -2]


def pin_int8_quantize_blocks(orc):
    """Per-block absmax: the largest magnitude maps to +-127, every value is reconstructed within
    half a step (s / 2), s = fp32(a / 127); an all-zero block keeps s = 1 and codes 0; the short
    last block's scale comes from its valid rows only."""
    X = _rand((150, 16), 101)
    X[64:128] = 0.0
    X[140, 3] = 9.0  # the last block (rows 128..149) has its own maximum
    codes, scales, deq = orc.quantize_blocks_int8(X, 64)
    assert scales[1] == 1.0 and np.all(codes[64:128] == 0)
    for t, (a, b) in enumerate(((0, 64), (128, 150))):
        blk = X[a:b]
        amax = np.float32(np.abs(blk).max())
        s = scales[0 if t == 0 else 2]
        assert s == np.float32(amax / np.float32(127.0))
        assert np.abs(codes[a:b]).max() == 127
        assert np.all(np.abs(deq[a:b] - blk) <= 0.5 * float(s) * (1 + 1e-6))
    assert codes[140, 3] == 127


def pin_int8_forward_error_bound(orc):
    """Q, K, V whose block values are exact multiples of 2^-4 within +-127 steps quantise without
    error, so the only error left is P's rounding: |O_int8 - O| <= sum_j (sP_j / 2) sum_n |v_n|
    / sum P^ per row (each P code is off by at most half a step), and the bound is met while
    the error is not zero."""
    N, d, blk, k = 128, 16, 64, 2
    rng = np.random.default_rng(102)
    Q, K, V = (rng.integers(-127, 128, (N, d)).astype(np.float64) / 16.0 for _ in range(3))
    for X in (Q, K, V):
        for t in range(0, N, blk):
            X[t, 0] = 127.0 / 16.0  # each block's absmax is exactly 127 steps
    idx = np.array([[0, 1], [0, 1]], dtype=np.int32)
    alpha = np.ones(N)
    O8, Os8, _ = orc.forward_int8_head(Q, K, V, idx, alpha, blk)
    _, Os, _ = orc.forward_head(Q, K, V, idx, alpha, blk)
    for i in range(2):
        q = Q[i * blk : (i + 1) * blk]
        S = [(q @ K[j * blk : (j + 1) * blk].T) / 4.0 for j in range(2)]
        m = np.maximum(S[0].max(axis=1), S[1].max(axis=1))[:, None]
        P = [np.exp(s - m) for s in S]
        den = (P[0].sum(axis=1) + P[1].sum(axis=1))[:, None]
        bound = sum((p.max() / 127.0 / 2.0) * np.abs(V[j * blk : (j + 1) * blk]).sum(axis=0)[None, :] for j, p in enumerate(P)) / den
        err = np.abs(Os8[i] - Os[i])
        assert np.all(err <= bound * (1 + 1e-9) + 1e-12), (err - bound).max()
        assert err.max() > 0
        np.testing.assert_allclose(O8[i], Os8[i], rtol=0, atol=1e-15)


def pin_int8_error_scale(orc):
    """On random data the int8 sparse branch stays within a few percent of the exact one, and the
    linear branch is untouched."""
    Q, K, V, alpha, idx, blk = _small_case(103, N=256, d=32, blk=64, k=2)
    _, Os, Ol = orc.forward(Q, K, V, idx, alpha, blk)
    _, Os8, Ol8 = orc.forward_int8(Q, K, V, idx, alpha, blk)
    np.testing.assert_array_equal(Ol8, Ol)
    rel = np.linalg.norm(Os8 - Os) / np.linalg.norm(Os)
    assert 1e-3 < rel < 0.05, rel


# ----------------------------------------------------------------------------------------------
# branch dropping


def _drop_case():
    B, H, N, d, blk, k = 1, 5, 150, 8, 32, 2
    rng = np.random.default_rng(61)
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    alpha = rng.uniform(0.0, 1.0, (B, H, N))
    alpha[0, 0] = 1.0                            # linear weight exactly 0
    alpha[0, 1] = 0.0                            # sparse weight exactly 0
    alpha[0, 2] = rng.uniform(0.97, 1.0, N)      # linear weight at most 0.03
    alpha[0, 2, 7] = 1.0 - 0.03125               # exactly at the threshold below (a float32 value)
    alpha[0, 3] = rng.uniform(0.0, 0.02, N)      # sparse weight at most 0.02
    n_b = -(-N // blk)
    idx = np.stack([_rand_idx(n_b, k, 62 + h) for h in range(H)])[None]
    return Q, K, V, idx, alpha, blk


def pin_branch_drop_exact_at_zero(orc):
    """tau = 0 drops only branches whose weight is exactly 0 everywhere, so the output equals the
    undropped forward bit for bit."""
    Q, K, V, idx, alpha, blk = _drop_case()
    O, _, _ = orc.forward(Q, K, V, idx, alpha, blk)
    Od, dl, ds = orc.forward_dropped(Q, K, V, idx, alpha, 0.0, blk)
    assert dl.tolist() == [[True, False, False, False, False]], dl
    assert ds.tolist() == [[False, True, False, False, False]], ds
    assert np.array_equal(Od, O)


def pin_branch_drop_threshold(orc):
    """tau = 1/32: the head whose linear weight reaches 1/32 (inclusive) loses exactly
    (1 - alpha) O_l, the head whose sparse weight stays below it loses exactly alpha O_s, the
    others are untouched; tau outside [0, 0.5) is refused."""
    Q, K, V, idx, alpha, blk = _drop_case()
    O, Os, Ol = orc.forward(Q, K, V, idx, alpha, blk)
    Od, dl, ds = orc.forward_dropped(Q, K, V, idx, alpha, 0.03125, blk)
    assert dl.tolist() == [[True, False, True, False, False]], dl
    assert ds.tolist() == [[False, True, False, True, False]], ds
    a = alpha[..., None]
    np.testing.assert_allclose(Od[0, 2], O[0, 2] - (1 - a[0, 2]) * Ol[0, 2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Od[0, 3], O[0, 3] - a[0, 3] * Os[0, 3], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(Od[0, 4], O[0, 4])
    _, dl2, _ = orc.forward_dropped(Q, K, V, idx, alpha, 0.0312, blk)
    assert not dl2[0, 2], "1 - alpha = 1/32 exceeds a threshold just below it"
    for bad in (-1e-3, 0.5):
        try:
            orc.branch_drops(alpha, bad)
        except ValueError:
            continue
        raise AssertionError(f"tau {bad} accepted")


# ----------------------------------------------------------------------------------------------
# PISA (exact-or-approximate) forward and covariance-aware routing


def _pisa_golden():
    with open(os.path.join(GOLDEN, "pisa_worked_example.json")) as f:
        g = json.load(f)
    a = math.sqrt(2.0) * math.log(2.0)

    def val(x):
        if isinstance(x, str) and x.lstrip("-") == "a":
            return -a if x.startswith("-") else a
        return float(Fraction(x)) if isinstance(x, str) else float(x)

    return g, (lambda rows: np.array([[val(x) for x in r] for r in rows]))  # noqa: E731


def pin_pisa_worked_example(orc):
    """The hand-derived example in tests/golden/pisa_worked_example.json: block statistics,
    covariance norms, both routings and the output (exact rationals plus multiples of ln 2)."""
    g, arr = _pisa_golden()
    Q, K, V = arr(g["Q"]), arr(g["K"]), arr(g["V"])
    blk = g["block"]
    st = orc.pisa_block_stats(K, V, blk)
    np.testing.assert_allclose(st["centroid"], arr(g["expected_centroid"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st["vsum"], arr(g["expected_vsum"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st["H"], np.array(g["expected_H"], dtype=np.float64), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st["Hbar"], arr(g["expected_Hbar"]), rtol=0, atol=1e-14)
    M2 = np.array([float(Fraction(x)) for x in g["expected_M_squared"]])
    np.testing.assert_allclose(orc.pisa_cov_norms(st["H"], st["Hbar"]) ** 2, M2, rtol=1e-13)
    rc = orc.pisa_route(Q, K, V, g["topk"], blk, covariance=True)
    rp = orc.pisa_route(Q, K, V, g["topk"], blk, covariance=False)
    assert np.array_equal(rc["idx"], np.array(g["expected_idx_covariance"])), rc["idx"]
    assert np.array_equal(rp["idx"], np.array(g["expected_idx_plain"])), rp["idx"]
    O = orc.pisa_forward(Q[None, None], K[None, None], V[None, None], np.array(g["idx"])[None, None], blk)
    ln2 = math.log(2.0)
    exp = np.array([[float(Fraction(c0)) + float(Fraction(c1)) * ln2 for c0, c1 in row] for row in g["expected_O"]])
    np.testing.assert_allclose(O[0, 0], exp, rtol=0, atol=1e-13)


def pin_pisa_all_selected_is_full_attention(orc):
    """Every block kept: nothing is approximated and PISA is full softmax attention (torch SDPA)."""
    N, d, blk = 200, 16, 64
    Q, K, V = (_rand((N, d), s) for s in (71, 72, 73))
    n_b = -(-N // blk)
    idx = np.tile(np.arange(n_b, dtype=np.int32), (n_b, 1))
    O = orc.pisa_forward(Q[None, None], K[None, None], V[None, None], idx[None, None], blk)
    np.testing.assert_allclose(O[0, 0], _sdpa(Q, K, V), rtol=0, atol=1e-12)


def pin_pisa_constant_block_keys_exact(orc):
    """Keys constant inside each block (short last block included): every H_j is 0 and the
    zero-order block term is exact, so PISA equals full attention for any kept set, k = 0 too."""
    N, d, blk = 45, 6, 8
    n_b = -(-N // blk)
    kb = _rand((n_b, d), 74, 1.5)
    K = np.repeat(kb, blk, axis=0)[:N]
    Q, V = _rand((N, d), 75, 1.5), _rand((N, d), 76)
    ref = _sdpa(Q, K, V)
    for k, seed in ((0, 0), (2, 77), (n_b - 1, 78)):
        idx = _rand_idx(n_b, k, seed) if k else np.zeros((n_b, 0), np.int32)
        O = orc.pisa_forward(Q[None, None], K[None, None], V[None, None], idx[None, None], blk)
        np.testing.assert_allclose(O[0, 0], ref, rtol=0, atol=1e-12)
    st = orc.pisa_block_stats(K, V, blk)
    assert np.abs(st["H"]).max() < 1e-12 and np.abs(st["Hbar"]).max() < 1e-12


def pin_pisa_first_order_convergence(orc):
    """Keys kbar_j + eps * delta_n with one zero-sum offset pattern for every block and values
    v0_n + c_j: all H_j equal Hbar, so the first-order correction is exact and the error against
    full attention falls as eps^2 (ratio ~4 when eps halves).  Without the correction, or with it
    mis-scaled, the error is first order (ratio ~2)."""
    blk, n_b, d = 16, 6, 8
    N = blk * n_b
    delta = _rand((blk, d), 81)
    delta -= delta.mean(axis=0)
    v0 = _rand((blk, d), 82)
    cen = _rand((n_b, d), 83, 0.7)
    c = _rand((n_b, d), 84)
    V = np.concatenate([v0 + c[j] for j in range(n_b)])
    Q = _rand((N, d), 85, 1.2)
    idx = _rand_idx(n_b, 2, 86)
    errs = []
    for eps in (0.08, 0.04, 0.02):
        K = np.concatenate([cen[j] + eps * delta for j in range(n_b)])
        O = orc.pisa_forward(Q[None, None], K[None, None], V[None, None], idx[None, None], blk)
        errs.append(np.abs(O[0, 0] - _sdpa(Q, K, V)).max())
        st = orc.pisa_block_stats(K, V, blk)
        assert np.abs(orc.pisa_cov_norms(st["H"], st["Hbar"])).max() < 1e-12 * (1 + np.abs(st["Hbar"]).max())
    r1, r2 = errs[0] / errs[1], errs[1] / errs[2]
    assert 3.4 < r1 < 4.6 and 3.4 < r2 < 4.6, (errs, r1, r2)


def pin_pisa_stats_invariances(orc):
    """H_j and M_j ignore a constant shift of a block's keys (centering) and of its values (the
    offsets sum to zero); H_j has rank <= r_j - 1; scaling V scales Hbar and M alike."""
    N, d, blk = 100, 12, 8  # 13 blocks, the last one 4 tokens (rank <= 3 < d)
    K, V = _rand((N, d), 91), _rand((N, d), 92)
    st = orc.pisa_block_stats(K, V, blk)
    M = orc.pisa_cov_norms(st["H"], st["Hbar"])
    K2, V2 = K.copy(), V.copy()
    K2[16:24] += _rand((d,), 93, 5.0)
    V2[96:] += _rand((d,), 94, 5.0)
    st2 = orc.pisa_block_stats(K2, V2, blk)
    np.testing.assert_allclose(st2["H"], st["H"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(orc.pisa_cov_norms(st2["H"], st2["Hbar"]), M, rtol=1e-12)
    np.testing.assert_allclose(st2["centroid"][2] - st["centroid"][2], K2[16] - K[16], atol=1e-12)
    np.testing.assert_allclose(st2["vsum"][12] - st["vsum"][12], 4 * (V2[96] - V[96]), atol=1e-11)
    for j, r in enumerate(st["count"]):
        sv = np.linalg.svd(st["H"][j], compute_uv=False)
        assert np.all(sv[int(r) - 1 :] < 1e-10 * sv[0]), (j, sv)
    st3 = orc.pisa_block_stats(K, -2.5 * V, blk)
    np.testing.assert_allclose(st3["Hbar"], -2.5 * st["Hbar"], atol=1e-12)
    np.testing.assert_allclose(orc.pisa_cov_norms(st3["H"], st3["Hbar"]), 2.5 * M, rtol=1e-12)


def pin_pisa_route_minimises_error_bound(orc):
    """Brute force over every kept set of size k on a tiny head: the covariance-aware choice
    minimises the summed first-order error bound sum_{j not kept} e^{s_ij} ||H_j - Hbar||, with
    s from torch's average pooling; the plain choice maximises the kept scores."""
    import itertools

    N, d, blk, k = 6 * 8 - 3, 4, 8, 2
    Q, K, V = _rand((N, d), 95), _rand((N, d), 96), _rand((N, d), 97)
    n_b = -(-N // blk)
    pool = lambda X: torch.nn.functional.avg_pool1d(torch.from_numpy(X).T[None], blk, blk, ceil_mode=True)[0].T.numpy()  # noqa: E731
    s = pool(Q) @ pool(K).T / math.sqrt(d)
    Hs = []
    for j in range(n_b):
        kk, vv = K[j * blk : (j + 1) * blk], V[j * blk : (j + 1) * blk]
        Hs.append(sum(np.outer(kk[n] - kk.mean(axis=0), vv[n]) for n in range(len(kk))))
    Hb = sum(Hs) / n_b
    M = np.array([np.linalg.norm(h - Hb) for h in Hs])
    rc = orc.pisa_route(Q, K, V, k, blk, covariance=True)
    rp = orc.pisa_route(Q, K, V, k, blk, covariance=False)
    np.testing.assert_allclose(rc["scores"], s, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rc["M"], M, rtol=1e-12)
    for i in range(n_b):
        best = min(itertools.combinations(range(n_b), k),
                   key=lambda S: sum(math.exp(s[i, j]) * M[j] for j in range(n_b) if j not in S))
        assert tuple(rc["idx"][i]) == best, (i, rc["idx"][i], best)
        top = max(itertools.combinations(range(n_b), k), key=lambda S: sum(s[i, j] for j in S))
        assert tuple(rp["idx"][i]) == top, (i, rp["idx"][i], top)



# ---------------------------------------------------------------------------------------- SVOO


def _svoo_planted(seed, pi, n_b=8, blk=8, d=16, scale=4.0, noise=0.05, misplaced=2):
    """Queries and keys in n_b blocks of blk tokens along orthonormal directions e_0..e_{n_b-1}:
    query block c holds blk - misplaced tokens of direction pi[c], key block c of direction c,
    and each block's remaining tokens take other directions so that every direction has blk
    tokens in all.  Returns (Q, K, query directions, key directions)."""
    rng = np.random.default_rng(seed)

    def dirs(major):
        lab = np.repeat(major, blk)
        # swap `misplaced` tokens of each block with tokens of the next block (cyclically), so
        # direction counts stay blk each and every block keeps its majority
        for c in range(n_b):
            nxt = (c + 1) % n_b
            for m in range(misplaced):
                a, b = c * blk + m, nxt * blk + blk - 1 - m
                lab[a], lab[b] = lab[b], lab[a]
        return lab

    dq = dirs(np.asarray(pi))
    dk = dirs(np.arange(n_b))
    E = np.eye(d)[:n_b]
    Q = scale * E[dq] + noise * rng.standard_normal((n_b * blk, d))
    K = scale * E[dk] + noise * rng.standard_normal((n_b * blk, d))
    return Q, K, dq, dk


def pin_svoo_recovers_planted_coclusters(orc):
    """Planted co-clusters: query block c mostly of direction pi(c), key block c mostly of
    direction c, a quarter of each block misplaced.  A key of direction a has its largest
    affinity with the query centroid whose block looks for a, cluster pi^-1(a); the queries then
    follow the key centroids.  So every token lands in cluster pi^-1(its direction), from the
    first iteration on, and the stable order lists each cluster's tokens in their original order
    (a non-identity pi separates the query-driven key step from a key-only clustering)."""
    pi = np.array([3, 0, 6, 1, 7, 2, 5, 4])
    inv = np.argsort(pi)
    Q, K, dq, dk = _svoo_planted(211, pi)
    for iters in (1, 3):
        qa, ka = orc.svoo_cocluster_head(Q, K, iters, block=8)
        np.testing.assert_array_equal(qa, inv[dq], err_msg=f"queries, {iters} iterations")
        np.testing.assert_array_equal(ka, inv[dk], err_msg=f"keys, {iters} iterations")
    order = orc.svoo_order(qa)
    want = np.concatenate([np.flatnonzero(inv[dq] == c) for c in range(8)])
    np.testing.assert_array_equal(order, want)


def pin_svoo_fixed_point_on_coclustered_input(orc):
    """Input already co-clustered (block c of Q and K both of direction c): every token stays in
    its block's cluster, both permutations are the identity, and the forward on the permuted
    sequence is the plain forward."""
    n_b, blk = 8, 8
    E = np.eye(16)[:n_b]
    rng = np.random.default_rng(212)
    lab = np.repeat(np.arange(n_b), blk)
    Q = 4.0 * E[lab] + 0.05 * rng.standard_normal((n_b * blk, 16))
    K = 4.0 * E[lab] + 0.05 * rng.standard_normal((n_b * blk, 16))
    qa, ka = orc.svoo_cocluster_head(Q, K, 2, block=blk)
    np.testing.assert_array_equal(qa, lab)
    np.testing.assert_array_equal(ka, lab)
    np.testing.assert_array_equal(orc.svoo_order(qa), np.arange(n_b * blk))
    V = rng.standard_normal((1, 1, n_b * blk, 16))
    alpha = rng.uniform(0, 1, (1, 1, n_b * blk))
    W = rng.standard_normal((16, 16)) / 4
    ident = np.arange(n_b * blk)[None, None]
    O, idx = orc.svoo_forward(Q[None, None], K[None, None], V, W, W.T, alpha, 3, ident, ident, blk)
    ref_idx = orc.route(Q[None, None], K[None, None], W, W.T, 3, blk)["idx"]
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(O, orc.forward(Q[None, None], K[None, None], V, ref_idx, alpha, blk)[0],
                               rtol=0, atol=0)


def pin_svoo_assign_and_centroid_worked_example(orc):
    """Hand-computed: rows [1, 0], [1, 3], [2, 0] against centroids [1, 0], [1, 0], [0, 1] have
    affinities [1, 1, 0], [1, 1, 3], [2, 2, 0]: clusters 0 (a tie of 0 and 1 goes to the lower
    index), 2, 0 with leads 0, 2, 0.  Cluster 0's members average to [1.5, 0], cluster 1 is
    empty and keeps its previous centroid, cluster 2's one member is its mean."""
    X = np.array([[1.0, 0.0], [1.0, 3.0], [2.0, 0.0]])
    cent = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    a, lead = orc.svoo_assign(X, cent)
    np.testing.assert_array_equal(a, [0, 2, 0])
    np.testing.assert_allclose(lead, [0.0, 2.0, 0.0], rtol=0, atol=0)
    prev = np.array([[9.0, 9.0], [7.0, -7.0], [5.0, 5.0]])
    c = orc.svoo_centroids(X, a, prev)
    np.testing.assert_allclose(c, [[1.5, 0.0], [7.0, -7.0], [1.0, 3.0]], rtol=0, atol=0)


def pin_svoo_order_is_counting_sort(orc):
    """The permutation equals a counting sort written out: clusters in index order, each
    cluster's tokens in their original order (many equal keys, long enough that an unstable
    sort reorders them)."""
    rng = np.random.default_rng(213)
    a = rng.integers(0, 5, (2, 300))
    got = orc.svoo_order(a)
    for r in range(2):
        want = [t for c in range(5) for t in range(300) if a[r, t] == c]
        np.testing.assert_array_equal(got[r], want)


def pin_svoo_forward_permutation_invariant_limits(orc):
    """Random permutations of queries and keys: with every block kept the linear branch is empty
    and the output is alpha times full softmax attention of the unpermuted inputs; with none
    kept it is (1 - alpha) times global ReLU linear attention.  Both limits ignore the blocking,
    so only a correct gather of Q, alpha, K, V and scatter of O reproduce them."""
    rng = np.random.default_rng(214)
    N, d, blk = 90, 8, 16
    n_b = -(-N // blk)
    Q, K, V = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    alpha = rng.uniform(0.1, 0.9, (1, 2, N))
    W = rng.standard_normal((d, d)) / math.sqrt(d)
    pq = np.stack([rng.permutation(N) for _ in range(2)])[None]
    pk = np.stack([rng.permutation(N) for _ in range(2)])[None]
    x = Q @ np.swapaxes(K, -1, -2) / math.sqrt(d)
    p = np.exp(x - x.max(axis=-1, keepdims=True))
    full = (p / p.sum(axis=-1, keepdims=True)) @ V
    O, _ = orc.svoo_forward(Q, K, V, W, W, alpha, n_b, pq, pk, blk)
    np.testing.assert_allclose(O, alpha[..., None] * full, rtol=1e-10, atol=1e-12)
    rq, rk = np.maximum(Q, 0), np.maximum(K, 0)
    lin = (rq @ (np.swapaxes(rk, -1, -2) @ V)) / (rq @ rk.sum(axis=-2)[..., None])
    O, _ = orc.svoo_forward(Q, K, V, W, W, alpha, 0, pq, pk, blk)
    np.testing.assert_allclose(O, (1 - alpha[..., None]) * lin, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# SoftTop-k training path


def pin_soft_topk_budget_and_hard_limit(orc):
    """Every row of the soft mask sums to k with entries in (0, 1), ranks like the scores, and as
    the temperature goes to 0 it becomes the HardTop-k mask (scores with distinct values)."""
    rng = np.random.default_rng(301)
    s = rng.standard_normal((3, 4, 40))
    for k in (1, 7, 39):
        M = orc.soft_topk(s, k, 0.5)
        np.testing.assert_allclose(M.sum(axis=-1), k, rtol=0, atol=1e-10)
        assert np.all((M > 0) & (M < 1))
        order = np.argsort(s, axis=-1)
        assert np.all(np.diff(np.take_along_axis(M, order, axis=-1), axis=-1) >= 0)
        hard = orc.hard_topk(s, k)[1]
        np.testing.assert_allclose(orc.soft_topk(s, k, 1e-5), hard, rtol=0, atol=1e-6)
    np.testing.assert_array_equal(orc.soft_topk(s, 0, 0.5), 0.0)
    np.testing.assert_array_equal(orc.soft_topk(s, 40, 0.5), 1.0)


def pin_soft_topk_backward_finite_differences(orc):
    """The implicit gradient of the budget-constrained mask matches central differences of the
    forward along random directions (tau re-solved at every point)."""
    rng = np.random.default_rng(302)
    s = rng.standard_normal((2, 25))
    T, k, eps = 0.7, 6, 1e-6
    M = orc.soft_topk(s, k, T)
    for _ in range(3):
        dM = rng.standard_normal(s.shape)
        u = rng.standard_normal(s.shape)
        num = ((orc.soft_topk(s + eps * u, k, T) - orc.soft_topk(s - eps * u, k, T)) * dM).sum() / (2 * eps)
        ana = (orc.soft_topk_backward(M, dM, T, k) * u).sum()
        np.testing.assert_allclose(ana, num, rtol=1e-6, atol=1e-9)


def _soft_case(seed, N=150, d=8, blk=32):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Q[:, 0] = np.abs(Q[:, 0]) + 0.1  # no zero linear denominators
    K[:, 0] = np.abs(K[:, 0]) + 0.1
    nb = -(-N // blk)
    M = rng.uniform(0.05, 0.95, (nb, nb))
    alpha = rng.uniform(0.1, 0.9, N)
    return Q, K, V, M, alpha, blk


def pin_soft_forward_binary_mask_is_hard_forward(orc):
    """A 0/1 soft mask gives exactly the HardTop-k forward of the kept sets it encodes."""
    Q, K, V, _, alpha, blk = _soft_case(303)
    nb = -(-Q.shape[0] // blk)
    idx = _rand_idx(nb, 2, 304)
    M = np.zeros((nb, nb))
    for i in range(nb):
        M[i, idx[i]] = 1.0
    O, Os, Ol, _, _ = orc.forward_soft_head(Q, K, V, M, alpha, blk)
    Oh, Osh, Olh = orc.forward(Q[None, None], K[None, None], V[None, None], idx[None, None], alpha[None, None], blk)
    np.testing.assert_allclose(Os, Osh[0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Ol, Olh[0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O, Oh[0, 0], rtol=1e-12, atol=1e-12)


def pin_soft_forward_limits(orc):
    """M = 1 with alpha = 1 is full softmax attention (torch SDPA); M = 0 with alpha = 0 is plain
    ReLU linear attention over every key."""
    Q, K, V, _, _, blk = _soft_case(305)
    N = Q.shape[0]
    nb = -(-N // blk)
    O1 = orc.forward_soft_head(Q, K, V, np.ones((nb, nb)), np.ones(N), blk)[0]
    np.testing.assert_allclose(O1, _sdpa(Q, K, V), rtol=1e-10, atol=1e-12)
    O0 = orc.forward_soft_head(Q, K, V, np.zeros((nb, nb)), np.zeros(N), blk)[0]
    rq, rk = np.maximum(Q, 0), np.maximum(K, 0)
    np.testing.assert_allclose(O0, (rq @ (rk.T @ V)) / (rq @ rk.sum(axis=0))[:, None], rtol=1e-10, atol=1e-12)


def _torch_soft_forward(Q, K, V, M, alpha, blk):
    """A dense float64 torch re-statement of the soft-mask forward (token-level weights), written
    independently of the oracle, for autograd."""
    N, d = Q.shape
    bid = torch.arange(N) // blk
    W = M[bid][:, bid]  # weight of key n for query t: M[block(t), block(n)]
    x = (Q @ K.T) / math.sqrt(d)
    e = W * torch.exp(x - x.max(dim=1, keepdim=True).values)
    Os = (e @ V) / e.sum(dim=1, keepdim=True)
    lin = (1.0 - W) * (torch.relu(Q) @ torch.relu(K).T)
    Ol = (lin @ V) / lin.sum(dim=1, keepdim=True)
    return alpha[:, None] * Os + (1.0 - alpha[:, None]) * Ol


def pin_soft_backward_matches_autograd(orc):
    """dM and dalpha of the oracle's soft backward equal torch.autograd's gradients of the dense
    re-statement, for a random upstream gradient."""
    Q, K, V, M, alpha, blk = _soft_case(306)
    dO = np.random.default_rng(307).standard_normal(Q.shape)
    Mt = torch.tensor(M, requires_grad=True)
    at = torch.tensor(alpha, requires_grad=True)
    O = _torch_soft_forward(torch.tensor(Q), torch.tensor(K), torch.tensor(V), Mt, at, blk)
    np.testing.assert_allclose(O.detach().numpy(), orc.forward_soft_head(Q, K, V, M, alpha, blk)[0], rtol=1e-10, atol=1e-12)
    (O * torch.tensor(dO)).sum().backward()
    dM, dal = orc.backward_soft_head(Q, K, V, M, alpha, dO, blk)
    np.testing.assert_allclose(dM, Mt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dal, at.grad.numpy(), rtol=1e-9, atol=1e-11)


def pin_stage1_finite_differences(orc):
    """The stage-1 gradients (proj_q, proj_k, alpha: soft router, soft forward, SoftTop-k's
    implicit gradient, the projection chain) match central differences of the stage-1 loss."""
    rng = np.random.default_rng(308)
    B, H, N, d, blk, k, T = 1, 2, 96, 8, 16, 2, 0.3
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    Q[..., 0] = np.abs(Q[..., 0]) + 0.1
    K[..., 0] = np.abs(K[..., 0]) + 0.1
    Wq, Wk = (rng.standard_normal((d, d)) / math.sqrt(d) for _ in range(2))
    alpha = rng.uniform(0.2, 0.8, (B, H, N))
    Of = orc.full_attention(Q, K, V)
    g = orc.stage1_grads(Q, K, V, Wq, Wk, alpha, k, T, Of, blk)
    L = lambda wq, wk, al: orc.stage1_loss(Q, K, V, wq, wk, al, k, T, Of, blk)  # noqa: E731
    eps = 1e-5
    for name, X in (("dWq", Wq), ("dWk", Wk), ("dalpha", alpha)):
        u = rng.standard_normal(X.shape)
        args_p = [Wq, Wk, alpha]
        args_m = [Wq, Wk, alpha]
        pos = {"dWq": 0, "dWk": 1, "dalpha": 2}[name]
        args_p[pos] = X + eps * u
        args_m[pos] = X - eps * u
        num = (L(*args_p) - L(*args_m)) / (2 * eps)
        ana = (g[name] * u).sum()
        np.testing.assert_allclose(ana, num, rtol=2e-5, atol=1e-10)
    assert abs(g["loss"] - L(Wq, Wk, alpha)) < 1e-15


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
