"""fp64 CPU oracle (test infrastructure only; see oracle/attention.py).

Only the test suite, ``__graft_entry__.smoke()`` and bench.py's cpu_baseline leg
may import this package.  The HIP product path never does.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_probs,
    attention_varlen_backward,
    attention_varlen,
    decode,
    decode_paged,
    decode_varlen,
    gather_pages,
    kv_cache_write,
    kv_cache_write_paged,
    kv_head_of,
    page_slot,
    sequence_bounds,
    varlen_causal_offset,
    visibility,
)
