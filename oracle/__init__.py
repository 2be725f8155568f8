"""CPU oracle for paged KV-cache decode — TEST INFRASTRUCTURE, not product.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import anything here.  The HIP library never calls it
and shares no code with it: this package imports nothing from
``paged_kv_cache_08_amd``, and the library imports nothing from here.

What it computes, in plain, slow, obviously-correct NumPy (fp64 for every
floating-point result):

* ``accounting``  — KV bytes per token (2·L·H·d·b, the budget formula of
  «Servicio…presupuesto de memoria» §3 and «¿Cuánta memoria reservar para la caché KV?» "Plantear la fórmula"), blocks per request
  (ceil(T/B), «Servicio…presupuesto de memoria» §5, «Paged Attention optimiza el uso de memoria»), tail waste and utilisation («Servicio…presupuesto de memoria» §5,
  «Paged Attention optimiza el uso de memoria»).
* ``allocator``   — the block pool: free stack, reference counts, per-sequence
  block tables, fork with shared blocks and copy-on-write of the block a
  writer shares («¿Cómo gestiona Paged Attention la caché KV…?» "PagedAttention divide el estado KV…", "Los bloques
  liberados…", «PagedAttention e vLLM» "Approfondimento tecnico", «Paged Attention optimiza el uso de memoria» on CoW).
* ``pool``        — the physical K/V pool in the library's documented byte
  layout; scatter of new tokens into slots, gather of a sequence's blocks
  into a contiguous array through its block table («¿Cómo gestiona Paged Attention la caché KV…?»: the table maps
  logical order to physical blocks; indirection changes placement, not
  meaning).
* ``fp8``         — the 8-bit (E4M3) cache codes: value table from the bit
  fields, round-to-nearest-even encoding, one fp32 scale per (token, head)
  row (readings stated in the module).
* ``attention``   — exact attention softmax(q·Kᵀ·scale)·V in fp64 on the
  gathered arrays («Servicio…presupuesto de memoria» §6), with GQA head grouping («¿Cuánta memoria reservar para la caché KV?» "Emplear las
  cabezas KV"); plus the blockwise running-statistics form and the
  partition-merge form used only to pin the reading of the split-K step.

Pins (all in ``tests/``, marked ``not gpu``): the pages' worked numbers
(``tests/golden/accounting.json``), hand-derived allocator snapshots
(``tests/golden/allocator_scripts.json``), pure-Python brute-force attention,
``torch.nn.functional.scaled_dot_product_attention`` in fp64 on CPU,
closed-form special cases, permutation / copy-on-write invariance, and
mutation tests that plant mistakes here and check that a pin fails.

Parity unpinned: the six-request page-assignment example of «Servicio…presupuesto de memoria» §9
(results box ``page_tail_slots = 32``) — its request lengths are not printed,
so it is not reproduced.
"""
from . import accounting, allocator, attention, fp8, pool, replay  # noqa: F401
