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
closed forms, special cases and brute force on tiny inputs; every function
here is held by at least one of them.  The pages print no output or state
values, so on random inputs the recurrence is held by the closed form (an
independent product of per-token maps, on random inputs with small heads) and
by invariants (split invariance, linearity in the start state, decode as a
one-token prefill) rather than by printed numbers.
"""

from . import csr, slots, gdn  # noqa: F401
