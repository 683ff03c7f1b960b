"""Float64 CPU oracle for paged decode attention and its work queue.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path (the C-ABI library and its Python binding) never
does, and the oracle never imports the product.  The two share no code: the
only thing both sides consume is the seeded input generator, which holds none
of the method's arithmetic.

Modules
  paged_attention  softmax(q K^T * scale) V over block-table pages, the
                   per-range partial state, and the exact log-sum-exp merge.
  work_queue       the adaptive split policy and the compact work queue.

Every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` and ``tests/test_queue_oracle.py`` against
closed forms, invariants, a library routine (PyTorch's float64 scaled
dot-product attention on contiguous inputs) and brute-force enumeration.
"""

from . import paged_attention, work_queue  # noqa: F401
