"""CPU oracle for paged decode attention and the KV append.

Test infrastructure, not product code: only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the device library and never imports it; it reads the
same bytes the device path reads (raw storage arrays copied to the host) and
computes every result in float64 with plain numpy.

Modules:

* ``numerics`` - storage-format decoders (bf16, fp8 e4m3fn) written from the
  bit layouts.
* ``decode``   - gather each sequence's blocks into a contiguous buffer, then
  softmax(q K^T * scale) V per query head.
* ``append``   - byte copy of new tokens' K/V into their pool slots.
* ``capacity`` - the block/byte arithmetic and the contiguous-vs-paged
  capacity example.
* ``quant``    - the quantising append into an fp8 e4m3fn pool (nearest
  e4m3fn value of x / scale, saturating, ties to even).
* ``prefill``  - chunked-prefill attention: each chunk token attends to the
  cached tokens before it and to the chunk up to itself.

Every function is pinned by ``tests/test_oracle.py``,
``tests/test_quant.py`` and ``tests/test_prefill_oracle.py`` against
library routines, closed forms, invariants, brute force and the pages'
printed example; none is "parity unpinned".
"""
from . import append, capacity, decode, numerics, prefill, quant  # noqa: F401
from .append import kv_append  # noqa: F401
from .decode import paged_decode, attention_weights  # noqa: F401
from .prefill import paged_prefill, prefill_flops  # noqa: F401
