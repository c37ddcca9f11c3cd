"""Planted mistakes in a copy of the oracle must each fail at least one pin (CPU only).

Each mutation edits the oracle's source in a temporary copy of the package (one line, or a few
lines that only make sense together; the real oracle is never touched), imports the copy, and runs
every pin against it.
"""

import importlib.util
import os
import shutil
import sys
import uuid

import pytest

import numpy as np

import gen
import oracle
from tests import lowbit_slack
from tests.oracle_pins import ALL_PINS

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTATIONS = {
    "no_sparse_scale": ("sla.py", "scale = 1.0 / np.sqrt(d)\n    outs", "scale = 1.0\n    outs"),
    "no_router_scale": ("sla.py", "return (qt @ np.swapaxes(kt, -1, -2)) / np.sqrt(d)", "return qt @ np.swapaxes(kt, -1, -2)"),
    "transposed_proj_q": ("sla.py", "qt = pool_blocks(Q, block) @ Wq", "qt = pool_blocks(Q, block) @ Wq.T"),
    "pool_divides_by_block": ("sla.py", "/ float(b - a)", "/ float(block)"),
    "no_relu_on_q": ("sla.py", "pq = np.maximum(q, 0.0)", "pq = q"),
    "no_relu_on_k": ("sla.py", "pk = np.maximum(K[a:b], 0.0)", "pk = np.abs(K[a:b])"),
    "alpha_swapped": ("sla.py", "outs.append(al * o_s + (1.0 - al) * o_l)", "outs.append(al * o_l + (1.0 - al) * o_s)"),
    "linear_over_kept": ("sla.py", "unsel = (~keep).astype(np.float64)", "unsel = np.ones(n_b)"),
    "ties_to_higher_index": ("sla.py", 'order = np.argsort(-s, axis=-1, kind="stable")[..., :k]', 'order = np.argsort(s, axis=-1, kind="stable")[..., ::-1][..., :k]'),
    "unsorted_indices": ("sla.py", "idx = np.sort(order, axis=-1).astype(np.int32)", "idx = order.astype(np.int32)"),
    "sparse_norm_wrong_axis": ("sla.py", "o_s = (p @ V[tok]) / p.sum(axis=1, keepdims=True)", "o_s = (p @ V[tok]) / p.sum()"),
    "no_zero_denominator_guard": ("sla.py", "o_l[nz] = num[nz] / den[nz, None]", "o_l = num / den[:, None]"),
    "fp8_scale_dropped": ("fp8.py", "deq[a:b] = e4m3_decode(codes[a:b]) * np.float64(scales[t])", "deq[a:b] = e4m3_decode(codes[a:b])"),
    "fp8_truncating_round": ("fp8.py", "m8 = np.rint((mant * 2.0 - 1.0) * 8.0)", "m8 = np.floor((mant * 2.0 - 1.0) * 8.0)"),
    "fp8_bias_off_by_one": ("fp8.py", "_E4M3_BIAS = 7", "_E4M3_BIAS = 8"),
    "bwd_no_D_term": ("train.py", "ds = p * (dp - D)", "ds = p * dp"),
    "bwd_dk_unscaled": ("train.py", "dK[tok] += (ds.T @ q) * scale", "dK[tok] += ds.T @ q"),
    "bwd_no_relu_mask_q": ("train.py", "dQ[a:b] += dphi * (q > 0.0)", "dQ[a:b] += dphi"),
    "bwd_den_grad_sign": ("train.py", "e = -(g * o_l).sum(axis=1)", "e = (g * o_l).sum(axis=1)"),
    "bwd_dalpha_sign": ("train.py", "dalpha[a:b] = (g_o * (o_s - o_l)).sum(axis=1)", "dalpha[a:b] = (g_o * (o_l - o_s)).sum(axis=1)"),
    "bwd_no_linear_dv": ("train.py", "dV[a:b] += pK[a:b] @ dh[j]", "dV[a:b] += 0.0"),
    "bwd_dz_dropped": ("train.py", "dK[a:b] += (V[a:b] @ dh[j].T + dz[j][None, :]) * (K[a:b] > 0.0)", "dK[a:b] += (V[a:b] @ dh[j].T) * (K[a:b] > 0.0)"),
    "bwd_linear_over_kept": ("train.py", "dh[uns] += dA[None]", "dh[:] += dA[None]"),
    "int8_truncating_round": ("int8.py", "return np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8)", "return np.clip(np.trunc(y), -INT8_MAX, INT8_MAX).astype(np.int8)"),
    "int8_clamp_128": ("int8.py", "return np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8)", "return np.clip(np.rint(y), -128, 127).astype(np.int8)"),
    "int8_scale_over_128": ("int8.py", "scales[t] = np.float32(amax / np.float32(INT8_MAX))", "scales[t] = np.float32(amax / np.float32(128.0))"),
    "int8_p_scale_dropped": ("int8.py", "num += (p8 @ v8[starts[j]:ends[j]]).astype(np.float64) * (sP * float(sv[j]))", "num += (p8 @ v8[starts[j]:ends[j]]).astype(np.float64) * float(sv[j])"),
    "int8_k_scale_of_query_block": ("int8.py", "(float(sq[i]) * float(sk[j]) * scale)", "(float(sq[i]) * float(sk[i]) * scale)"),
    "drop_strict_threshold": ("sla.py", "return (1.0 - a).max(axis=-1) <= t, a.max(axis=-1) <= t", "return (1.0 - a).max(axis=-1) < t, a.max(axis=-1) <= t"),
    "drop_by_mean_weight": ("sla.py", "return (1.0 - a).max(axis=-1) <= t, a.max(axis=-1) <= t", "return (1.0 - a).mean(axis=-1) <= t, a.max(axis=-1) <= t"),
    "drop_sparse_by_min": ("sla.py", "return (1.0 - a).max(axis=-1) <= t, a.max(axis=-1) <= t", "return (1.0 - a).max(axis=-1) <= t, a.min(axis=-1) <= t"),
    "drop_renormalises": ("sla.py", "O = np.where(ds[..., None, None], 0.0, a * Os) + np.where(dl[..., None, None], 0.0, (1.0 - a) * Ol)", "O = np.where(ds[..., None, None], 0.0 * Os, a * Os) + np.where(dl[..., None, None], Os - a * Os, (1.0 - a) * Ol)"),
    "pisa_no_first_order": ("pisa.py", "num = e @ V[tok] + al @ vsum[uns] + (q @ Hbar) * al.sum(axis=1, keepdims=True)", "num = e @ V[tok] + al @ vsum[uns]"),
    "pisa_first_order_unscaled": ("pisa.py", "+ (q @ Hbar) * al.sum(", "+ (Q[a:b] @ Hbar) * al.sum("),
    "pisa_den_without_counts": ("pisa.py", "den = e.sum(axis=1) + al @ cnt[uns]", "den = e.sum(axis=1) + al.sum(axis=1)"),
    "pisa_uncentered_H": ("pisa.py", "H[j] = (K[a:b] - centroid[j]).T @ V[a:b]", "H[j] = K[a:b].T @ V[a:b]"),
    "pisa_hbar_sum": ("pisa.py", '"Hbar": H.mean(axis=0)', '"Hbar": H.sum(axis=0)'),
    "pisa_cov_sign": ("pisa.py", "sel = s + np.log(M)[None, :]", "sel = s - np.log(M)[None, :]"),
    "pisa_vsum_mean": ("pisa.py", "vsum[j] = V[a:b].sum(axis=0)", "vsum[j] = V[a:b].mean(axis=0)"),
    "pisa_centroid_over_block": ("pisa.py", "centroid[j] = K[a:b].mean(axis=0)", "centroid[j] = K[a:b].sum(axis=0) / block"),
    "pisa_kept_also_approximated": ("pisa.py", "uns = np.flatnonzero(~keep)", "uns = np.arange(n_b)"),
    "pisa_no_centroid_scale": ("pisa.py", "y = q @ kbar[uns].T", "y = Q[a:b] @ kbar[uns].T"),
    "pisa_route_unscaled": ("pisa.py", "s = (qbar @ st[\"centroid\"].T) / np.sqrt(Q.shape[1])", "s = qbar @ st[\"centroid\"].T"),
    "svoo_argmin": ("svoo.py", "assign = np.argmax(aff, axis=1)", "assign = np.argmin(aff, axis=1)"),
    "svoo_keys_by_key_centroids": ("svoo.py", "k_assign, k_margin = svoo_assign(K, q_cent)", "k_assign, k_margin = svoo_assign(K, k_cent)"),
    "svoo_queries_by_stale_key_centroids": ("svoo.py", "q_assign, q_margin = svoo_assign(Q, k_cent)", "q_assign, q_margin = svoo_assign(Q, pool_blocks(K, block))"),
    "svoo_empty_cluster_zeroed": ("svoo.py", "out = np.array(_f64(prev), copy=True)", "out = np.zeros_like(_f64(prev))"),
    "svoo_centroid_sum_not_mean": ("svoo.py", "out[c] = members.sum(axis=0) / len(members)", "out[c] = members.sum(axis=0)"),
    "svoo_unstable_order": ("svoo.py", 'axis=-1, kind="stable")', 'axis=-1, kind="quicksort")'),
    "svoo_scatter_as_gather": ("svoo.py", "np.put_along_axis(O, pq[..., None], Op, axis=2)", "O = np.take_along_axis(Op, pq[..., None], axis=2)"),
    "svoo_alpha_unpermuted": ("svoo.py", "ap = np.take_along_axis(alpha, pq, axis=2)", "ap = alpha"),
    "svoo_v_by_query_perm": ("svoo.py", "Vp = np.take_along_axis(V, pk[..., None], axis=2)", "Vp = np.take_along_axis(V, pq[..., None], axis=2)"),
    "fp8_tile_scale_dropped": ("fp8.py", "num += (enc(p / sP) * sP) @ Vd[starts[j]:ends[j]]", "num += enc(p / sP) @ Vd[starts[j]:ends[j]]"),
    # low-bit P quantisation: other granularities of the P scale and a denominator over the
    # dequantised P (SLA2, Arabic summary section 2.jim fixes neither; the readings are one scale
    # per query-block x key-block tile and the unquantised P^ in the denominator)
    "fp8_p_scale_per_row": ("fp8.py", [
        ("sP = p.max() / E4M3_MAX", "sP = p.max(axis=1, keepdims=True) / E4M3_MAX"),
        ("if sP == 0:\n                    continue\n                ", "")]),
    "fp8_p_scale_per_query_block": ("fp8.py", "sP = p.max() / E4M3_MAX", "sP = max(x.max() for x in P) / E4M3_MAX"),
    "fp8_dequantised_denominator": ("fp8.py", "den = np.sum([p.sum(axis=1) for p in P], axis=0)[:, None]",
                                    "den = np.sum([(enc(p / (p.max() / E4M3_MAX)) * (p.max() / E4M3_MAX)).sum(axis=1) for p in P], axis=0)[:, None]"),
    "int8_p_scale_per_row": ("int8.py", [
        ("sP = p.max() / INT8_MAX", "sP = p.max(axis=1, keepdims=True) / INT8_MAX"),
        ("if sP == 0:\n                    continue\n                ", "")]),
    "int8_p_scale_per_query_block": ("int8.py", "sP = p.max() / INT8_MAX", "sP = max(x.max() for x in P) / INT8_MAX"),
    "int8_dequantised_denominator": ("int8.py", "den = np.sum([p.sum(axis=1) for p in P], axis=0)[:, None]",
                                     "den = np.sum([(int8_encode(p / (p.max() / INT8_MAX)) * (p.max() / INT8_MAX)).sum(axis=1) for p in P], axis=0)[:, None]"),
    # SoftTop-k training path
    "soft_tau_direction": ("soft.py", "above = tot > k  # the threshold is too low: raise it", "above = tot < k"),
    "soft_backward_no_tau_term": ("soft.py", "return (sp / T) * (dM - corr)", "return (sp / T) * dM"),
    "soft_backward_no_temperature": ("soft.py", "return (sp / T) * (dM - corr)", "return sp * (dM - corr)"),
    "soft_sparse_weight_dropped": ("soft.py", "e = w[None, :] * np.exp(x - m)", "e = np.exp(x - m)"),
    "soft_linear_weight_not_complement": ("soft.py", "A = np.tensordot(1.0 - M[i], h, axes=(0, 0))", "A = np.tensordot(M[i], h, axes=(0, 0))"),
    "soft_linear_dm_sign": ("soft.py", "dM[i] -= np.tensordot(h, dT, axes=([1, 2], [0, 1])) + z @ dzeta",
                            "dM[i] += np.tensordot(h, dT, axes=([1, 2], [0, 1])) + z @ dzeta"),
    "soft_dalpha_sign": ("soft.py", "dalpha = (dO * (Os - Ol)).sum(axis=1)", "dalpha = (dO * (Ol - Os)).sum(axis=1)"),
    "router_backward_dk_untransposed": ("soft.py", "dkt = (np.swapaxes(ds, -1, -2) @ qt) / np.sqrt(d)", "dkt = (ds @ qt) / np.sqrt(d)"),
    "stage1_dO_halved": ("soft.py", "dO = 2.0 * diff / diff.size", "dO = diff / diff.size"),
}


def _load_mutant(tmp_path, fname, *edit):
    """Copy the oracle, apply the edit (one (old, new) pair, or a list of them) and import it."""
    pairs = edit[0] if len(edit) == 1 else [edit]
    name = f"oracle_mutant_{uuid.uuid4().hex[:8]}"
    dst = tmp_path / name
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    src = path.read_text()
    for old, new in pairs:
        assert src.count(old) == 1, f"mutation anchor not unique in {fname}: {old!r}"
        src = src.replace(old, new)
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(name, dst / "__init__.py", submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # a mutant may divide by zero on purpose
@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, mutation):
    mod = _load_mutant(tmp_path, *MUTATIONS[mutation])
    caught = []
    for name, pin in ALL_PINS.items():
        try:
            pin(mod)
        except Exception:  # an AssertionError, or the mutant crashing on a pin's input
            caught.append(name)
    assert caught, f"no pin catches the planted mistake '{mutation}'"


READING_MUTATIONS = ["fp8_p_scale_per_row", "fp8_p_scale_per_query_block", "fp8_dequantised_denominator",
                     "int8_p_scale_per_row", "int8_p_scale_per_query_block", "int8_dequantised_denominator"]
# an implementation with the oracle's readings whose P^ carries a relative error of 3e-6 (about
# the fp32 rounding of the kernels' exponent argument at logits near 30)
P_NOISE = ("P = [np.exp(s - m) for s in S]",
           "P = [np.exp(s - m) * (1 + 3e-6 * np.random.default_rng(1).standard_normal(s.shape)) for s in S]")


@pytest.fixture(scope="module")
def _reading_case():
    wl = gen.workload("video_l", H=1, N=3600, grid=(1, 45, 80), topk=6)  # 57 blocks, last 16 tokens
    c = gen.draw(wl, 0)
    idx = oracle.route(c["Q"], c["K"], c["Wq"].double(), c["Wk"].double(), wl.topk, 64)["idx"][0, 0]
    starts, ends, _ = oracle.block_ranges(wl.N, 64)
    args = (c["Q"][0, 0], c["K"][0, 0], c["V"][0, 0], idx, np.ones(wl.N), 64)
    ref = {}
    for fmt, head, quant in (("fp8", oracle.forward_fp8_head, oracle.quantize_blocks),
                             ("int8", oracle.forward_int8_head, oracle.quantize_blocks_int8)):
        trace = []
        Os = np.concatenate(head(*args, trace=trace)[1])
        Qd, Kd, Vd = (quant(c[n][0, 0], 64)[2] for n in ("Q", "K", "V"))
        sl = lowbit_slack.slack_rows(trace, Vd, starts, ends, range(wl.n_blocks), fmt, Qd, Kd)
        ref[fmt] = (Os, np.concatenate([s_ for s_, _ in sl]), np.concatenate([m_ for _, m_ in sl]))
    return args, ref


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mutation", READING_MUTATIONS + ["fp8_noise", "int8_noise"])
def test_lowbit_slack_separates_readings(tmp_path, _reading_case, mutation):
    """On the small ragged clustered workload of the GPU reading test, the flip-aware bound of
    tests/lowbit_slack.py accepts an implementation of the oracle's readings whose P^ carries
    fp32-sized errors (rel-L2 about 4e-4 from code flips alone) and rejects every other reading
    of the P step on many elements."""
    args, ref = _reading_case
    kind = mutation.split("_")[0]
    fname = "fp8.py" if kind == "fp8" else "int8.py"
    mod = _load_mutant(tmp_path, fname, *P_NOISE) if mutation.endswith("noise") else _load_mutant(tmp_path, *MUTATIONS[mutation])
    head = mod.forward_fp8_head if kind == "fp8" else mod.forward_int8_head
    got = np.concatenate(head(*args)[1])
    res = lowbit_slack.check_within_slack(got, *ref[kind])
    if mutation.endswith("noise"):
        assert res["violations"] == 0, res
    else:
        assert res["violations"] > 1000, (mutation, res)
