"""libgdn: the Gated DeltaNet layer core as hand-written HIP kernels for
AMD MI355X (gfx950), behind a C ABI (include/gdn.h).

This package is the thin torch-facing binding; the kernels live in
libgdn.so, built from csrc/ by build.py.
"""
from ._lib import (GDN_BF16, GDN_DEVERR_ACCEPTED, GDN_DEVERR_BATCH, GDN_DEVERR_CACHE,  # noqa: F401
                   GDN_DEVERR_PAGE, GDN_DEVERR_PARITY, GDN_F32, GDN_PATH_CHUNKED, GDN_NOALLOC_SYNC_WORDS, GDN_PATH_TOKEN,
                   GDN_MIXED_AUTO, GDN_MIXED_ONE_LAUNCH, GDN_MIXED_TWO_LAUNCHES, GDN_PREFILL_MAX_DEFAULT,
                   GDN_SPEC_ONEPAGE, GDN_SPEC_SLOTS, load)
from .ops import (Batch, ConvPool, Dims, GdnError, Params, PrefixCache, SpecPages, StatePool,  # noqa: F401
                  gdn_abi_version, gdn_chunked_prefill, gdn_chunked_workspace_bytes, gdn_conv_update,
                  gdn_mixed_launches, gdn_mixed_step, gdn_prefill, gdn_prefill_path, gdn_prefix_restore, gdn_recurrent_seq,
                  gdn_recurrent_seq_noalloc,
                  gdn_spec_page_layout, gdn_spec_verify)
