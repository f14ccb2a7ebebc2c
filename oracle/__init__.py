"""fp64 CPU oracle for the paged-attention path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""

from .paged_attention import (  # noqa: F401
    RAW_TYPES,
    attend,
    decode,
    gather,
    merge,
    prefill,
    slot_of,
    softmax,
    split_partials,
    store,
    to_f64,
)
from .norm_rope import (  # noqa: F401
    qk_norm_rope,
    qk_norm_rope_store,
    rms_norm,
    rope,
    rope_frequencies,
    rotate_pair,
    split_qkv,
)
