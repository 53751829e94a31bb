"""Float64 CPU oracle for the JVP flash-attention forward (test infrastructure).

This package is test infrastructure, not product code. Only the test suite,
the smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it. The GPU library never calls it and has no CPU fallback.
"""
from .attention import oracle_fwd, oracle_fwd_head
from .attention_bwd import oracle_bwd, oracle_bwd_head

__all__ = ["oracle_fwd", "oracle_fwd_head", "oracle_bwd", "oracle_bwd_head"]
