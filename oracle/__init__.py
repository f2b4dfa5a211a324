"""CPU oracle for the Jenga token-sparse attention hot path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import
this package.  It shares no code with the HIP path.
"""
from .jenga_oracle import *  # noqa: F401,F403
from .jenga_oracle import (SELECT_TOPK, SELECT_THRESH_REL, SELECT_THRESH_ABS, attn_bwd,
                           attn_bwd_compact, attn_bwd_masked, attn_bwd_sampled, attn_fwd,
                           attn_fwd_compact, attn_fwd_masked, attn_fwd_rows, block_scores,
                           block_scores_eq2, eq2_tile_max, lm_head_ce, proj_gather,
                           proj_scatter_add, proj_gather_scatter_add, MLP_RELU,
                           MLP_SILU_GATED, mlp_activation, mlp_token_scores,
                           mlp_block_scores, mlp_sparse_forward,
                           default_scale, keep_count, kv_head_of,
                           received_mass, residual_add, select_blocks, stack_forward,
                           threshold_value, token_positions)
