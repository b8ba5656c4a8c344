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
    lanes, fixed 64-token pages, recent keys held unquantized.
  * "Half the Cache, Twice the Context" (ml.co.ke): the bytes-per-token
    formula, the symmetric absmax quantizer, per-channel K / per-token V
    scaling, the outlier recipe, the accumulator-precision model.

Pins: every function is checked against something other than itself, in
the ``-m "not gpu"`` suite:
  * accounting: the pages' byte figures (9,216 vs 65,536 B a token, 7.11x,
    12.5 %, 3.02 GB vs 20.0 GiB) and the sizing table of "Half the Cache,
    Twice the Context" (tests/golden/block1_sizing.txt, kv_bytes.txt);
  * bf16, codec.sym_*: that page's printed reconstruction, needle and
    flat-sum tables reproduced digit for digit (tests/golden/block2_*.txt,
    block3_flat_sum.txt);
  * codec (2-bit, 8-bit, rotation): closed-form invariants, round-half-even
    ties, constant rows, exact rational arithmetic for the fused
    multiply-add, scipy's Hadamard matrix;
  * layout: byte positions worked out by hand (tests/golden/layout_cases.txt)
    and a frozen block image (tests/golden/q2_block_d128.hex);
  * pool: permutation invariance, untouched fill bytes, the bf16 block read
    back by hand, fork and window identities;
  * attention.decode / prefill / split and merge: closed forms (one key,
    equal keys, a dominant key, the 131,072-token flat case), a pure-Python
    loop on small inputs, the split-merge identity, prefill rows against
    decode; attention.scores: the GQA head mapping and basis-key closed
    forms, and softmax of the scores against decode; planted_rank: worked
    ties.
No function is left "parity unpinned".
"""

from . import accounting, bf16, codec, layout, pool, attention, experiments  # noqa: F401
