"""Test infrastructure: the plain CPU oracle for paged KV-cache attention.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the library and its binding never do.
"""

from .paged_attention import (  # noqa: F401
    causal_allowed,
    decode,
    gather_kv,
    lse_merge,
    partial_softmax,
    slot_of,
    softmax_attention,
    varlen,
    widen,
    write_kv,
)
