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

Every function is pinned against something other than itself, with
planted mistakes that must break the pin:

* ``decode.paged_decode``, ``decode.gather_sequence``: torch SDPA in float64
  on contiguous K/V the test scatters into a pool, pure-Python brute force,
  closed forms and invariants (``tests/test_oracle.py``);
* ``decode.attention_weights``: torch SDPA with identity values, whose
  output is the weight vector (``tests/test_oracle.py``);
* ``append.kv_append``: the appended token is the last one each table walk
  reaches and nothing else changes (``tests/test_oracle.py``);
* ``append.copy_blocks``: a fork through the block manager diverging by
  copy-on-write reads the parent's stored tokens then its own, untouched
  blocks keep their bytes; a swapped copy, a K-only copy and an append
  before the copy each break it (``tests/test_oracle.py``);
* ``numerics``: every bf16 and e4m3fn code against torch's casts;
* ``capacity``: the pages' printed capacity example (``tests/golden``);
* ``quant``: torch's float32 -> e4m3fn cast and the e4m3fn definition
  (``tests/test_quant.py``);
* ``prefill``: masked torch SDPA in float64 (``tests/test_prefill_oracle.py``).

No function is "parity unpinned".
"""
from . import append, capacity, decode, numerics, prefill, quant  # noqa: F401
from .append import kv_append  # noqa: F401
from .decode import paged_decode, attention_weights  # noqa: F401
from .prefill import paged_prefill, prefill_flops  # noqa: F401
