"""fp64 CPU oracle of the CSA/HCA attention core.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
does, and the oracle imports nothing from the product path: the two share no
code.  The only common dependency is the seeded input generator package
``synth``, which holds no arithmetic of the method.

Contents:

* ``oracle.codecs`` – exact bf16 / e4m3fn decoders and RNE encoders written
  from the format definitions.
* ``oracle.csa``    – the method's steps in fp64, in the order the pages give
  them: compressor (pool, RMSNorm, partial RoPE), lightning-indexer score,
  top-k, shared-KV MQA with sliding window and sink (CSA sparse / HCA dense).

Pinning: every function is checked by ``tests/test_oracle_pins.py`` against
facts that do not come from the oracle itself (closed forms, invariants,
special cases that reduce to library routines, brute-force ranking on tiny
inputs, hand-derived fixtures under ``tests/golden/``).  No function is
"parity unpinned".
"""
from . import codecs, csa  # noqa: F401
