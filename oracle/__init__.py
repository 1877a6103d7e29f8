"""CPU oracle for paged-KV block transfer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the oracle leg of ``bench.py``
(its verification step against the timed path, and its ``cpu_baseline``) may
import this package.  The HIP library never routes through
it, and it imports nothing from the HIP library.  See ``kv_oracle`` for the
definitions and the passages of the pages each one follows.
"""
from .kv_oracle import (  # noqa: F401
    HND, NHD, K, V, Geometry, OracleError, Plan, Pool, Request, Run,
    block_pairs, blocks_in_use, copy_heads, copy_heads_plain, copy_heads_region,
    head_rows, last_block_fill, make_plan, pack, plan_runs, push, push_plain,
    push_region, push_scales, reusable_prefix, reuse_request, should_reuse,
    staging_bytes, staging_region_bytes, tokens_to_move, triples, unpack, validate,
    Segment, token_segments, triples_reblock, window_start,
    StateGeometry, StatePool, StatePlan, make_state_plan, pack_state, push_state,
    push_state_plain, state_staging_bytes, unpack_state, validate_state,
)
