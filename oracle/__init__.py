"""CPU oracle (test infrastructure).

Plain, slow, float64 implementations of what the library computes.  Only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg may
import this package; the library itself never does.
"""
from .oracle import (  # noqa: F401
    rope_tables, rope_tables_at, segment_arrays, qk_rmsnorm, qk_rmsnorm_bwd, rope_apply, rope_apply_inverse,
    qknorm_rope_fwd, qknorm_rope_bwd, attention_fwd, attention_bwd,
    forward, backward, decode, split_heads, merge_heads, qkv_proj, out_proj, qkv_proj_bwd,
    out_proj_bwd,
)
