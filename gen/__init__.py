"""Seeded synthetic inputs for the SLA2 forward: the only module both the HIP path's tests/bench
and the CPU oracle use.

It draws tensors and nothing else: no pooling, projection, scoring, softmax or selection lives
here.  Callers that need the router's k-th/(k+1)-th score gap (the tests) check it with the oracle
and ask this module to redraw single query blocks (``query_noise_means`` then
``realize_query_blocks``).

Workloads (the pages measure on Wan2.1 video DiT attention, which is not available; these
tensors stand in for it with the same shapes and an attention-concentrating structure):

* ``tiny``       B=1 H=2  N=1024  d=64  k=4   fp32, Q/K/V iid N(0,1).
* ``video_s``    B=1 H=12 N=32768 d=128 k=51  bf16, latent 8x64x64 (t, h, w) flattened.
* ``video_l``    B=1 H=40 N=75600 d=128 k=60  bf16, latent 21x45x80, last block 16 tokens.
* ``sweep``      B=2 H=12 N=32768 d=128, keep in {20,10,5,3}% (k = round(keep*512)),
                 cluster scale in {0.5,1,2}, alpha fixed 0.5 or random.
* ``video_l_fp8`` the ``video_l`` tensors, for the fp8 sparse-branch path.
* ``pisa_video_s``, ``pisa_video_l`` the ``video_s`` / ``video_l`` tensors with 12.5 % of the
                 KV blocks kept (k = 64 of 512, 148 of 1182), the 87.5 % sparsity at which the
                 PISA summary reports its Wan2.1-14B result, for the PISA forward.
* ``svoo_video_s`` the ``video_s`` tensors, for the path on SVOO co-clustered blocks.

Clustered Q/K: the latent grid is cut into boxes of (2, 8, 8) tokens (smaller at the edges);
per (batch, head, box) a centre mu ~ N(0, s^2 I_d) is shared by the box's queries and keys,
Q_n = mu + e_q, K_n = mu + e_k with e ~ N(0, 0.3) (0.3 read as the variance).  V ~ N(0, 1),
alpha = sigmoid(N(0, 1)) per (batch, head, token), proj_q and proj_k ~ N(0, 1/d) (variance).
Every stream is a numpy PCG64 seeded by SeedSequence([seed, workload id, tensor id, b, h, ...]).
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import functools
import math
import os

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "sweep_workloads",
    "draw",
    "noise_std",
    "query_block_centres",
    "query_noise_means",
    "realize_query_blocks",
]

NOISE_VAR = 0.3
BOX = (2, 8, 8)

# tensor ids of the seed streams
(_T_Q, _T_K, _T_V, _T_ALPHA, _T_WQ, _T_WK, _T_CENTRE, _T_QNOISE, _T_KNOISE, _T_REDRAW,
 _T_REALIZE) = range(11)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    topk: int
    dtype: str  # "fp32" or "bf16"
    kind: str  # "iid" or "clustered"
    grid: tuple = ()
    cluster_scale: float = 1.0
    alpha: str = "random"  # "random" (sigmoid(N(0,1))) or "half" (0.5)
    fp8: bool = False
    block: int = 64
    wid: int = 0  # seed-stream id of the workload

    @property
    def n_blocks(self) -> int:
        return -(-self.N // self.block)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, 4, "fp32", "iid", wid=1),
    "video_s": Workload("video_s", 1, 12, 32768, 128, 51, "bf16", "clustered", (8, 64, 64), wid=2),
    "video_l": Workload("video_l", 1, 40, 75600, 128, 60, "bf16", "clustered", (21, 45, 80), wid=3),
    "video_l_fp8": Workload(
        "video_l_fp8", 1, 40, 75600, 128, 60, "bf16", "clustered", (21, 45, 80), fp8=True, wid=3
    ),
    "pisa_video_s": Workload("pisa_video_s", 1, 12, 32768, 128, 64, "bf16", "clustered", (8, 64, 64), wid=2),
    "pisa_video_l": Workload("pisa_video_l", 1, 40, 75600, 128, 148, "bf16", "clustered", (21, 45, 80), wid=3),
    "svoo_video_s": Workload("svoo_video_s", 1, 12, 32768, 128, 51, "bf16", "clustered", (8, 64, 64), wid=2),
}


def workload(name: str, **kw) -> Workload:
    return WORKLOADS[name].with_(**kw) if kw else WORKLOADS[name]


def sweep_workloads():
    """The sparsity sweep: keep {20,10,5,3}% x cluster scale {0.5,1,2} x alpha {0.5, random}."""
    out = []
    for keep in (0.20, 0.10, 0.05, 0.03):
        for s in (0.5, 1.0, 2.0):
            for a in ("half", "random"):
                k = int(round(keep * 512))
                out.append(
                    Workload(
                        f"sweep_k{k}_s{s:g}_{a}", 2, 12, 32768, 128, k, "bf16", "clustered",
                        (8, 64, 64), cluster_scale=s, alpha=a, wid=4,
                    )
                )
    return out


def workers() -> int:
    """Host threads for per-head work: the affinity mask, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


@functools.lru_cache(maxsize=8)
def _cluster_ids(grid) -> tuple[np.ndarray, int]:
    """Box id of every token of a (T, Hh, W) latent grid flattened as n = (t*Hh + h)*W + w."""
    T, Hh, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    nt, nh, nw = (math.ceil(T / BOX[0]), math.ceil(Hh / BOX[1]), math.ceil(W / BOX[2]))
    cid = ((t // BOX[0]) * nh + (h // BOX[1])) * nw + (w // BOX[2])
    return cid.reshape(-1), nt * nh * nw


def _round(x: np.ndarray, dtype: str):
    """float32 numpy -> torch CPU tensor of the workload dtype (bf16 by torch's RNE cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _head_qk(wl: Workload, seed: int, b: int, h: int):
    """Float32 Q and K of one head before rounding."""
    N, d = wl.N, wl.d
    if wl.kind == "iid":
        q = _rng(seed, wl.wid, _T_Q, b, h).standard_normal((N, d), dtype=np.float32)
        k = _rng(seed, wl.wid, _T_K, b, h).standard_normal((N, d), dtype=np.float32)
        return q, k
    cid, ncl = _cluster_ids(wl.grid)
    assert len(cid) == N, (wl.grid, N)
    mu = _centres(seed, wl, b, h)
    sd = np.float32(math.sqrt(NOISE_VAR))
    eq = _rng(seed, wl.wid, _T_QNOISE, b, h).standard_normal((N, d), dtype=np.float32)
    ek = _rng(seed, wl.wid, _T_KNOISE, b, h).standard_normal((N, d), dtype=np.float32)
    c = mu[cid]
    return c + sd * eq, c + sd * ek


def draw(wl: Workload, seed: int = 0) -> dict:
    """All inputs of one workload as CPU torch tensors.

    Returns {'Q','K','V': [B,H,N,d] (fp32 or bf16), 'Wq','Wk': [d,d] fp32, 'alpha': [B,H,N]
    fp32, 'workload': wl, 'seed': seed}.
    """
    import torch

    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    Q = torch.empty((B, H, N, d), dtype=tdt)
    K = torch.empty((B, H, N, d), dtype=tdt)
    V = torch.empty((B, H, N, d), dtype=tdt)
    alpha = torch.empty((B, H, N), dtype=torch.float32)

    def one_head(bh):
        b, h = divmod(bh, H)
        q, k = _head_qk(wl, seed, b, h)
        Q[b, h] = _round(q, wl.dtype)
        K[b, h] = _round(k, wl.dtype)
        v = _rng(seed, wl.wid, _T_V, b, h).standard_normal((N, d), dtype=np.float32)
        V[b, h] = _round(v, wl.dtype)
        if wl.alpha == "half":
            alpha[b, h] = 0.5
        else:
            x = _rng(seed, wl.wid, _T_ALPHA, b, h).standard_normal(N)
            alpha[b, h] = torch.from_numpy((1.0 / (1.0 + np.exp(-x))).astype(np.float32))

    # every head has its own seed streams, so the result does not depend on the thread count
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers()) as ex:
        list(ex.map(one_head, range(B * H)))
    sw = 1.0 / math.sqrt(d)
    Wq = torch.from_numpy(_rng(seed, wl.wid, _T_WQ).normal(0.0, sw, (d, d)).astype(np.float32))
    Wk = torch.from_numpy(_rng(seed, wl.wid, _T_WK).normal(0.0, sw, (d, d)).astype(np.float32))
    return {"Q": Q, "K": K, "V": V, "Wq": Wq, "Wk": Wk, "alpha": alpha, "workload": wl, "seed": seed}


def noise_std(wl: Workload) -> float:
    """Standard deviation of the per-token query/key noise."""
    return math.sqrt(NOISE_VAR) if wl.kind == "clustered" else 1.0


def query_block_centres(inputs: dict, b: int, h: int, block: int) -> np.ndarray:
    """The cluster-centre part of the query tokens of one block (zeros for iid workloads),
    float32 [r, d] with r the block's number of tokens."""
    wl: Workload = inputs["workload"]
    a = block * wl.block
    e = min(a + wl.block, wl.N)
    if wl.kind != "clustered":
        return np.zeros((e - a, wl.d), dtype=np.float32)
    cid, ncl = _cluster_ids(wl.grid)
    mu = _centres(inputs["seed"], wl, b, h)
    return mu[cid[a:e]]


def _centres(seed, wl, b, h):
    mu = _rng(seed, wl.wid, _T_CENTRE, b, h).standard_normal((_cluster_ids(wl.grid)[1], wl.d), dtype=np.float32)
    return mu * np.float32(wl.cluster_scale)


def query_noise_means(inputs: dict, b: int, h: int, blocks, attempt: int, count: int,
                      chunk: int = 0) -> np.ndarray:
    """`count` candidate values, per listed block of head (b, h), of the mean over the block's
    r tokens of their i.i.d. N(0, 1) query noise: N(0, 1/r) per channel, float32
    [len(blocks), count, d], from the stream (seed, workload, b, h, attempt, chunk)."""
    wl: Workload = inputs["workload"]
    blocks = np.asarray(blocks, dtype=np.int64)
    r = np.minimum(wl.block, wl.N - blocks * wl.block).astype(np.float32)
    z = _rng(inputs["seed"], wl.wid, _T_REDRAW, b, h, int(attempt), int(chunk)).standard_normal(
        (len(blocks), count, wl.d), dtype=np.float32
    )
    return z / np.sqrt(r)[:, None, None]


def realize_query_blocks(inputs: dict, b: int, h: int, blocks, noise_means, attempt: int,
                         chunk: int = 0) -> None:
    """Redraw, in place, the query tokens of the listed blocks (ascending) so that each block's
    noise has the given mean (noise_means [len(blocks), d]).

    The noise of a block with r tokens is Z - mean(Z) + noise_mean with Z i.i.d. N(0, 1) [r, d]
    (one stream keyed by (seed, workload, b, h, attempt, chunk) for all listed blocks): for
    i.i.d. Gaussian noise the mean is independent of the deviations from it, so drawing the mean
    first (query_noise_means) and the deviations here gives tokens with the same distribution as
    a direct draw.  Cluster centres (and K, V, alpha) are kept, so only these blocks' rows of the
    block-score map move.
    """
    import torch

    wl: Workload = inputs["workload"]
    blk, N, d = wl.block, wl.N, wl.d
    blocks = np.asarray(blocks, dtype=np.int64)
    if len(blocks) == 0:
        return
    z = _rng(inputs["seed"], wl.wid, _T_REALIZE, b, h, int(attempt), int(chunk)).standard_normal(
        (len(blocks), blk, d), dtype=np.float32
    )
    r = np.minimum(blk, N - blocks * blk)
    valid = np.arange(blk)[None, :] < r[:, None]  # [n, blk]
    zsum = (z * valid[..., None]).sum(axis=1)
    noise = z - (zsum / r[:, None])[:, None, :] + np.asarray(noise_means, np.float32)[:, None, :]
    rows = (blocks[:, None] * blk + np.arange(blk)[None, :])[valid]
    noise = noise[valid]  # [sum r, d]
    if wl.kind == "clustered":
        cid, _ = _cluster_ids(wl.grid)
        noise = _centres(inputs["seed"], wl, b, h)[cid[rows]] + np.float32(noise_std(wl)) * noise
    inputs["Q"][b, h, torch.from_numpy(rows)] = _round(noise, wl.dtype)
