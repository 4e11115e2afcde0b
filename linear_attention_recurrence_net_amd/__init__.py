"""MI355X (gfx950) gated delta net (GDN) recurrence.

A thin Python binding over the C-ABI library ``libgdn.so`` (declared in
``include/gdn.h``).  Every step of the computation runs in the library's HIP
kernels; this package only checks torch tensors and passes their device
pointers and the current HIP stream.  There is no CPU fallback: if the
library is missing or a tensor is not on the GPU, the call raises.

Entry points (same names as the C ABI):
  gdn_forward, gdn_forward_snapshots, gdn_rollback_select,
  gdn_forward_snapshots_after_rollback,
  gdn_prefill_workspace_size, gdn_prefill_chunked,
  gdn_forward_qk_broadcast, gdn_prefill_chunked_qk_broadcast,
  gdn_prefill_varlen_workspace_size, gdn_prefill_chunked_varlen,
  gdn_prefill_chunked_snapshots, gdn_prefill_kda_workspace_size,
  gdn_prefill_chunked_kda, gdn_prefill_workspace_size_ex, gdn_prefill_chunked_ex,
  gdn_prefill_chunked_ex_after_rollback, gdn_prefill_chunked_ex_noalloc,
  gdn_prefill_varlen_workspace_size_ex, gdn_prefill_chunked_varlen_ex
"""

from ._binding import (  # noqa: F401
    GDN_BF16,
    GDN_F32,
    GDN_GATE_HEAD,
    GDN_GATE_KEY,
    GdnError,
    gdn_forward,
    gdn_forward_qk_broadcast,
    gdn_forward_snapshots,
    gdn_forward_snapshots_after_rollback,
    gdn_prefill_chunked,
    gdn_prefill_chunked_qk_broadcast,
    gdn_prefill_chunked_ex,
    gdn_prefill_chunked_ex_after_rollback,
    gdn_prefill_chunked_ex_noalloc,
    gdn_prefill_chunked_kda,
    gdn_prefill_chunked_snapshots,
    gdn_prefill_kda_workspace_size,
    gdn_prefill_chunked_varlen,
    gdn_prefill_chunked_varlen_ex,
    gdn_prefill_varlen_workspace_size,
    gdn_prefill_varlen_workspace_size_ex,
    gdn_prefill_workspace_size,
    gdn_prefill_workspace_size_ex,
    gdn_rollback_select,
    library,
    library_path,
)
