"""CPU oracle for paged, quantized KV attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``.  The product path (the HIP
library and its Python binding) never imports it, and the oracle imports
nothing from the product path: the two share no kernels, headers, helpers,
tables or pre/post-processing.  Only ``synth`` (seeded inputs, no method
arithmetic) feeds both.

Precision: the codecs run in emulated IEEE fp32 (numpy float32 element-wise
operations, each rounded to nearest even, no fused multiply-add), because codes
and metadata must match the GPU bit for bit; gather and softmax attention run
in fp64.

Sources (the three pages this library is built from):
  * "KV at 9 KB a token" (ignis, why-ignis/kv-in-bytes): the hq-e8-2b row of
    64 B of 2-bit code plus an 8-byte metadata row per head per token, the
    per-token byte table, 64-token pages, the byte-budgeted pool, admission
    reservation, prefill reading the compressed cache, the garbage-filled
    workspace check.
  * "The KV cache and prompt reuse" (ignis, concepts): one pool shared by all
    lanes, fixed 64-token pages, the window of exact recent keys.
  * "Half the Cache, Twice the Context" (ml.co.ke): the bytes-per-token
    formula, the symmetric absmax quantizer, per-channel K / per-token V
    scaling, the outlier recipe, the accumulator-precision model.

Parity status of every function is stated in its module docstring; there is
no function marked "parity unpinned".
"""

from . import accounting, bf16, codec, layout, pool, attention, experiments  # noqa: F401
