"""CPU fp64 oracle of the MoE layer forward -- test infrastructure only (tests, smoke check,
the bench's CPU-baseline leg). The HIP library neither imports nor links anything here."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (FLAG_BAD_INDEX, FLAG_NONFINITE_LOGIT, capacity, combine, expert_ffn,
                         forward, gate_logits, gather_rows, gelu, grouped_ffn, permute_indices,
                         select_experts, selection_margin, silu, softmax, topk_weights,
                         valid_slots)
