"""CPU oracle for paged Gated Delta-Rule prefill and decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may use it.  It shares no code with the HIP library.

Everything here is plain, slow and meant to be read against the pages:

* ``csr``   -- CSR page tables from sequence lengths and back (FlashInfer CSR
  paging drill, sections 2 and 3).
* ``slots`` -- the pool rows each paged call derives from a page table
  (flashinfer.gdn_paged, "Page table" and "Slot arguments").
* ``gdn``   -- the token-by-token fp64 recurrence, the general slot-argument
  prefill/decode and the paged wrappers.

Pins (see ``tests/test_oracle_*.py``): the worked examples the pages print,
closed forms, special cases and brute force on tiny inputs.  Random-input
numerics beyond those are "parity unpinned": the pages print no output or
state values, so this oracle is the only reference for them.
"""

from . import csr, slots, gdn  # noqa: F401
