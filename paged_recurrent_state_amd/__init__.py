"""Gated Delta-Rule prefill and decode on a paged recurrent-state pool, MI355X (gfx950).

The compute runs in hand-written HIP kernels in ``libgdn_paged.so`` (C ABI:
``include/gdn_paged.h``); this package only marshals torch tensors into it.
Build the library with ``python -m paged_recurrent_state_amd.build``.
"""

from ._lib import (  # noqa: F401
    DecodeSlots,
    GDNError,
    Options,
    PrefillSlots,
    CHECK_BITS,
    block_table_to_csr,
    check_paged,
    checked,
    csr_to_block_table,
    decode,
    decode_paged,
    decode_slots,
    load,
    lib_path,
    prefill,
    prefill_paged,
    prefill_paged_noalloc,
    prefill_slots,
    prefill_workspace_size,
    stream_copy,
    version,
)
