"""Plain, slow CPU float64 oracle for the SLA2 hybrid sparse-linear attention inference forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use
it.  It shares no code, header, table or helper with the HIP library in
``block_sparse_linear_02_amd/``; the two meet only in the seeded inputs drawn by ``gen/``.

Sources (cited by page title and section; the summaries number their sections themselves):

* "SLA2: Sparse-Linear Attention with Learnable Routing and QAT" - Italian summary
  (gist.science/it/paper/2602.12675), sections 1, 2.A, 2.B, 2.C; and the Arabic summary of the
  same paper (gist.science/ar/paper/2602.12675), sections 1 and 2 (alef, ba, jim, dal).
* "PISA - Piecewise Sparse Attention per Efficient Diffusion Transformers" - Italian technical
  summary (gist.science/it/paper/2602.01077), section 2 (exact-or-approximate forward,
  covariance-aware routing): ``pisa.py``.
* "Training-Free Sparse Attention for Fast Video Generation via Offline Layer-Wise Sparsity
  Profiling and Online Bidirectional Co-Clustering" (SVOO) - Italian summary
  (gist.science/it/paper/2603.18636), section 2.B (online bidirectional co-clustering):
  ``svoo.py``.
* SLA2's training path (SoftTop-k router, soft-mask forward and its gradients, the stage-1 MSE
  fit of proj_q, proj_k and alpha): ``soft.py``.
* "SALAD: Achieve High-Sparsity Attention via Efficient Linear Attention Tuning for Video
  Diffusion Transformer" (gist.science/it/paper/2601.16515), section 2 (ReLU kernel function,
  linear branch sharing Q, K, V with the sparse branch).

Pins: every function here is checked by ``tests/test_oracle_*.py`` (CPU, ``-m "not gpu"``)
against library routines, closed forms, hand-derived worked examples under ``tests/golden/``,
dense brute force on tiny inputs and invariants.  No function is "parity unpinned".
"""

from .sla import (  # noqa: F401
    block_ranges,
    pool_blocks,
    router_scores,
    hard_topk,
    route,
    block_states,
    forward_head,
    forward,
    branch_drops,
    forward_dropped,
    dense_P,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_encode,
    e4m3_decode,
    quantize_blocks,
    forward_fp8_head,
    forward_fp8,
)
from .pisa import (  # noqa: F401
    pisa_block_stats,
    pisa_cov_norms,
    pisa_route,
    pisa_forward_head,
    pisa_forward,
)
from .int8 import (  # noqa: F401
    INT8_MAX,
    int8_encode,
    quantize_blocks_int8,
    forward_int8_head,
    forward_int8,
)
from .train import backward_head, backward  # noqa: F401
from .svoo import (  # noqa: F401
    svoo_assign,
    svoo_centroids,
    svoo_cocluster_head,
    svoo_cocluster,
    svoo_order,
    svoo_forward,
)
from .soft import (  # noqa: F401
    soft_topk,
    soft_topk_backward,
    soft_route,
    forward_soft_head,
    forward_soft,
    backward_soft_head,
    backward_soft,
    router_backward,
    full_attention,
    stage1_loss,
    stage1_grads,
)
