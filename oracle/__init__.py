"""CPU oracle for position-independent KV-cache reuse (test infrastructure).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does, and shares no code with it.
"""
from .pic_oracle import (  # noqa: F401
    TARGET_AUTO, PlannedSpan, assemble, attention, empty_prefix,
    new_token_positions, plan_spans, prologue, query_prefill_layer,
    rope_frequencies, rotate, round_bf16, round_f32, to_storage,
)
