"""Fused attention forward (bf16, fp32 and FP8 inputs), its recompute backward, paged decode and
chunked prefill against the paged cache, for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a small C ABI (``include/fa.h``,
built as ``libfa.so`` next to this file).  This package is the thin Python binding over it:
it marshals torch device tensors into pointers and sizes and calls the library on torch's
current HIP stream.  It never computes attention itself, and it raises if the library is
missing.
"""

from ._binding import (  # noqa: F401
    FA_BF16,
    FA_F32,
    FaError,
    fa_bwd,
    fa_bwd_workspace_bytes,
    fa_fwd,
    fa_fwd_fp8,
    fa_fwd_unfused,
    fa_fwd_unfused_workspace_bytes,
    fa_paged_decode,
    fa_paged_decode_noalloc,
    fa_paged_decode_workspace_bytes,
    fa_paged_prefill,
    fa_paged_prefill_workspace_bytes,
    fa_status_str,
    library_path,
    load_library,
)
