"""CPU oracle for the INT4 KV-cache path (quantize, dequantize, decode attention, codec).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
execute anything in this package; only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library in ``int4_quantized_kv_amd/csrc``; the two
meet only on the seeded inputs produced by ``synth.py``.

Every function is written from the pages it cites, as plainly as possible: NumPy,
fp64 wherever the definition does not itself fix fp32, no blocking, fusion or
reordering beyond the definition.  Each function's docstring names the passage it
follows and the reading taken where the text is silent or garbled.

Modules
  quant      INT4 group quantize / dequantize, nibble packing, INT8 per-token variant
  attention  plain softmax decode attention with GQA and a sliding-window horizon
  codec      Walsh-Hadamard rotation + Lloyd-Max 4-bit codec
  memory     KV-cache size and effective-bit closed forms
  paged      the paged layout: the page allocation policy, pool rows, fragmentation

Pinning status: every public function is pinned by ``tests/test_oracle_*.py``
against values printed on the pages (``tests/golden``), closed forms, textbook
tables, library routines or brute force.  No function is "parity unpinned".
"""

from . import quant, attention, codec, memory, paged  # noqa: F401
