"""fp64 CPU oracle of the focused block-diffusion step (score -> select -> compact -> attend).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's CPU-baseline leg,
never by the product path.  It shares no code with the HIP library.
"""
from .focus_oracle import (  # noqa: F401
    adaptive_threshold, bf16_to_f64, block_commit, compact, kth_boundary, kv_pack, kv_writeback,
    layer_importance,
    layer_importance_full, prefix_keys, ragged_paged_attn, request_budget, request_kv, score_l01,
    score_l01_full, select_budget, step, to_f64,
)
