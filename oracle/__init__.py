"""Test-infrastructure oracle for block-sparse flash attention (CPU, float64).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The product package never imports it.
"""
from .bsa_oracle import (FULL, PARTIAL, allowed_count, allowed_keys, allowed_queries,
                         attend_row, backward, backward_dkv_keys, backward_dq_rows,
                         forward, forward_query_range, grad_row, kv_head, lse_merge, plan,
                         tile_counts)

__all__ = ["FULL", "PARTIAL", "allowed_count", "allowed_keys", "allowed_queries",
           "attend_row", "backward", "backward_dkv_keys", "backward_dq_rows",
           "forward", "forward_query_range", "grad_row", "kv_head", "lse_merge", "plan",
           "tile_counts"]
