"""fp64 CPU oracle for streaming-prefill attention -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and there is no CPU
fallback through it.

Every function here is pinned by `-m "not gpu"` tests against something other
than itself (closed forms, brute force, library special cases, invariants);
see `tests/test_oracle_pins.py`.  Nothing here is "parity unpinned".
"""
from .fd_oracle import (  # noqa: F401
    inv_freq,
    rope,
    StreamWindow,
    window_positions,
    new_query_positions,
    attend,
    oracle_stream,
    oracle_verify,
    expected_ring_rows,
    expected_cache,
    run_stream_workload,
)
