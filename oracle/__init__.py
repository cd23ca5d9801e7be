"""CPU oracle (test infrastructure only; see ssa_oracle's header)."""
from .ssa_oracle import (  # noqa: F401
    Params,
    PrefillOracle,
    as_f64,
    attend,
    block_stats,
    decode_step,
    dropped_mass,
    key_set,
    planted_recall,
    prefill_row,
    recovery_weight,
    routable_blocks,
    route_scores,
    route_scores_from_logits,
    select_topk,
)
