"""CPU oracle for document-masked varlen attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written float64 reference the HIP library is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path in
``load_balance_amd/`` never imports, calls or links anything here, and nothing
here imports ``load_balance_amd``; the two share only the seeded input
generators in ``workloads/``.

Modules
-------
``attention``  explicit-mask attention per document / pack / block, the
               log-sum-exp merge and the zigzag ring fold.
``plan``       the reference tile enumerator: which (query tile, key span)
               pairs hold visible pairs, their exact pair counts, the key
               blocks each sweeps, and the longest-first order.
``sharding``   which tokens each context-parallel rank holds (sequence zigzag,
               per-document, striped, mask-area dispatch) and one rank's sharded
               ring fold.
``backward``   the gradients dq, dk, dv of the varlen forward and of one ring
               step (from the whole-row lse and D = <dout, out>).

Pins (what each function is checked against, in ``tests/test_oracle_*.py``):
every function here is pinned by closed forms, special cases, a library
routine (torch ``scaled_dot_product_attention`` in float64) or brute force on
tiny inputs; none is marked "parity unpinned".
"""
from . import attention, backward, plan, sharding  # noqa: F401
