"""Lightning Attention prefill, multi-token decode and speculative verify / commit on AMD Instinct MI355X (gfx950).

The computation lives in liblaprefill.so (C ABI: include/la_prefill.h); this package is its Python binding.
Importing it fails loudly when the library has not been built.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LA_DECAY_PER_QK_HEAD,
    LA_ERR_HIP,
    LA_ERR_INVALID_ARG,
    LA_ERR_UNSUPPORTED,
    LA_OK,
    LA_SCHED_AUTO,
    LA_SCHED_NONPERSISTENT,
    LA_SCHED_PERSISTENT,
    LA_STATE_READ,
    LA_STATE_WRITE,
    LaError,
    la_decode_mtp,
    la_prefill_fwd,
    la_prefill_fwd_ex,
    la_prefill_fwd_seg,
    la_prefill_fwd_seg_noalloc,
    la_prefill_seg_noalloc_max_bytes,
    la_prefill_seg_workspace_bytes,
    la_prefill_fwd_varlen,
    la_prefill_fwd_varlen_ex,
    la_state_commit,
    la_state_commit_kvbuffer,
    la_verify_kvbuffer,
    lib,
)
