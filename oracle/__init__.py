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
from .int8_kv import (  # noqa: F401
    decode_int8,
    dequantize_int8,
    quantize_int8,
    write_kv_int8,
)
from .block_manager import BlockManager, copy_blocks  # noqa: F401
from .variants import attend, decode_ext, varlen_ext  # noqa: F401
