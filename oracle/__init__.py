"""CPU oracle (test infrastructure only; see dcp_oracle for what it computes)."""
from .dcp_oracle import (  # noqa: F401
    NEG_INF, MLA_DV, owner_of, owned_tokens, owned_count, owned_slots, attend,
    attend_bruteforce, gqa_shard, gqa_full, mla_shard, mla_full, merge, check_parallel,
    query_positions, gqa_shard_mq, gqa_full_mq, mla_shard_mq, mla_full_mq,
)
