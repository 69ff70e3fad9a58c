"""Exact backward-over-backward through softmax attention on MI355X (gfx950).

The computation runs in the HIP kernels of libflashbob.so (C ABI in
include/flashbob.h); this package is the thin Python binding around it.
"""

from .binding import (  # noqa: F401
    FlashBoBError,
    LIB_PATH,
    SIGNATURES,
    attn_bwd,
    attn_fwd,
    bob_attention,
    bob_attention_alloc,
    bob_attention_fourpass,
    bob_attention_noalloc,
    bob_attention_with_stats,
    load_library,
    probe_gq_atomics,
    profile_start,
    profile_stop,
    set_alloc_limit,
    set_reduction,
    set_tuning,
    workspace_bytes,
)
from .autograd import attention  # noqa: F401
