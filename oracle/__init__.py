"""CPU fp64 oracle for BDLM-masked core attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.
"""
from .bdlm_attention import (NEG_INF, attention_bwd, attention_fwd, bdlm_bwd, bdlm_fwd,  # noqa: F401
                             bdlm_keys, bdlm_mask, bdlm_mask_fn, combined_mask, count_pairs, delta_rows,
                             lse_merge, softmax_probs, task_bwd, task_fwd, task_mask, task_mask_fn,
                             varlen_bwd, varlen_fwd, varlen_mask, varlen_mask_fn)
