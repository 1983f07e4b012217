"""CPR Gated DeltaNet layer for MI355X (gfx950): HIP kernels behind a C ABI.

The C ABI lives in include/gdn_cpr.h; this package holds the sources
(csrc/), the build script and a thin ctypes binding (api).
"""

from .api import (  # noqa: F401
    CprCache,
    LayerShape,
    StageEvents,
    alloc_cache,
    alloc_workspace,
    gdn_cmp_chunk_decode_step,
    gdn_cmp_decode_step,
    gdn_cmp_prefill,
    gdn_cmp_workspace,
    gdn_cpr_cache_state,
    gdn_cpr_decode_step,
    gdn_cpr_decode_step_noalloc,
    gdn_cpr_fwd_bwd,
    gdn_cpr_last_error,
    gdn_cpr_numerics_id,
    gdn_cpr_prefill,
    gdn_cpr_prefill_continue,
    gdn_cpr_wait_status,
    gdn_cpr_workspace_size,
)
from ._lib import (  # noqa: F401
    GDN_OP_DECODE,
    GDN_OP_FWD_BWD,
    GDN_OP_PREFILL,
    GDN_OP_PREFILL_CONTINUE,
    GDN_CMP_CHUNKWISE,
    GDN_CMP_RECURRENT,
    GdnError,
)
