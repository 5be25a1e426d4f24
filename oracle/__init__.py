"""fp64 CPU oracle for training-free block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  The product
path (``block_mean_pool_amd``) never imports, calls or links anything here,
and nothing here imports the product path: the two share no code.

Sources followed (the method as the pages state it):

* SpargeAttn abstract (taxoreview.com page, and the same abstract on the
  huggingface-mirror search page): a two-stage online filter; stage one
  rapidly predicts the attention map so that some matrix multiplications can
  be skipped, stage two is a softmax-aware filter inside the online softmax
  that skips further multiplications; the attention is also quantized.
* iCATS abstract (arxivdaily.com page, English abstract): training-free
  sparse attention estimates the importance of query-key regions, derives a
  sparse mask, and computes only the important candidates; prior work
  estimates scores from tokens grouped independently on the query and the
  key side; masks are built with a top-p rule.
* DynSparse story (embedding.report page): top-p vs top-k selection and a
  threshold built from the cumulative energy of the selected tokens, a
  quantity the flash-attention operator already holds.
* iCATS abstract again, and the PARO abstract (huggingface-mirror search
  page): tokens grouped by the query-key interaction (a quadratic form)
  and reordered so that the attention pattern becomes block-wise, with the
  tails of irregular clusters merged instead of padded (``cluster.py``).

Every concrete choice the pages leave open (block-mean pooling as the
grouping, block sizes, the tie order, the cut rule, the lambda test, the
quantisation formats) is a stated reading, listed in the module docstrings.

Parity status: every function here is pinned by the CPU tests
(``tests/test_oracle_*.py``) against brute force, closed forms, invariants
or an independent library routine.  The pages' end-to-end model figures
(VBench, PSNR) are parity unpinned: no weights or suites exist here.
"""
from .sparse_attn_oracle import (  # noqa: F401
    Params,
    n_blocks,
    pool_means,
    admissible_blocks,
    block_scores,
    block_weights,
    forced_blocks,
    processing_order,
    cut_length,
    predict_head,
    predict_from_means,
    group_skip,
    sparse_attention_head,
    dense_attention_head,
    oracle_head,
)
from .quant import (  # noqa: F401
    e4m3_round,
    e4m3_flip_slack,
    e4m3_encode,
    int8_quantize_blocks,
    int_quantize_blocks,
    fp8_quantize_v_blocks,
    pow2_scale,
    fp8_quantize_v_blocks_pow2,
    sparse_attention_quant_head,
)
from .schedule import step_plan, sequence_head, call_tau, dense_params  # noqa: F401
from .cluster import (  # noqa: F401
    ClusterParams,
    second_moment,
    metric_matrix,
    quad_dist,
    seeds,
    assign,
    update,
    cluster_tokens,
    token_order,
    reorder_perms,
    reordered_attention_head,
    reordered_head,
)
from .metrics import (  # noqa: F401
    rel_l1,
    max_abs,
    admissible_counts,
    block_sparsity,
    real_groups,
    skip_fraction,
    predicted_kept_mass,
    true_recall,
)
