"""CPU oracle for compressed-KV key quantisation and decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
loads this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check and to time against.

It is a plain, slow, float64 (numpy) restatement of what the pages describe,
written step by step so a reader can check each step against the text:

* ``codebook``  -- Lloyd-Max scalar quantiser for one coordinate of a random
  unit vector after rotation (TurboQuant article §二, the coarse Lloyd-Max step).
* ``rotation``  -- random orthogonal rotation from a QR decomposition
  (TurboQuant article §二, the normalise-and-rotate step).
* ``keys``      -- norm, rotation, Lloyd-Max index, residual, QJL sign sketch,
  residual norm, and the bit layouts those are stored in (§二, §五).
* ``values``    -- min-max grouped value quantisation (component table, §七).
* ``attention`` -- query rotation/sketch, the unbiased score estimator in its
  dequantised-key form (§五), softmax attention over dequantised values (§六).

Pins (tests that tie each function to something other than itself) live in
``tests/test_oracle_*.py``.  Functions without such a pin say
"parity unpinned" in their docstring.  The oracle shares no code with the HIP
path; the only module both sides use is the seeded input generator
``kv_cache_compression_quantize_amd.inputs``, which holds no method arithmetic
(and which the oracle itself does not import).
"""
from . import codebook, rotation, keys, values, attention, layout  # noqa: F401
