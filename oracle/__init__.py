"""fp64 CPU oracle of the TokenGate gated-prefill step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.  It shares no
code with the HIP library under ``learned_token_pruning_06_amd``.
"""
from . import readings
from .ref import (silu, ref_score, ref_rmsnorm, ref_score_prenorm, ref_normalise, rank_order, ref_select, ref_kept_sizes,
                  ref_gather, length_factor, ref_gated_attn, ref_gated_attn_lse2, ref_gated_attn_masked,
                  ref_gated_attn_multiplicative, ref_gated_attn_loggate,
                  ref_gated_attn_bruteforce, ref_gated_attn_bwd, ref_gated_attn_bwd_rows, ref_score_bwd,
                  ref_score_prenorm_bwd,
                  ref_project,
                  ref_rope, ref_project_qk_rope,
                  ref_gate)
from .costs import token_layer_passes, attention_pair_ratio, causal_attention_flops
