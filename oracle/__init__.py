"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or falls back to it.  It shares no
code, constants or helpers with the HIP path.

Pages cited (titles as published):

* [IO-aware]   "FlashAttention: making attention IO-aware"
               (tingtang.site/blog/flash-attention)
* [IO-algos]   "Flash Attention & IO-Aware Algorithms"
               (chatwhole.com/learn/ai-ml-premium/39-flash-attention)
* [Why-faster] "Why is FlashAttention faster?"
               (fanout.sh/blog/why-is-flash-attention-faster)

Contents:

* ``attention``  -- the plain definition (explicit S, row softmax, P V, the
  logsumexp L) and the textbook backward, per head, in float64.
* ``online``     -- the tiled online-softmax recurrence the pages describe,
  in float64, used only to check that the recurrence equals the definition.
* ``splitkv``    -- the split-KV merge rule (Flash-Decoding), in float64,
  used only to check that merging per-run results equals the definition.
* ``fp8``        -- the FP8 forward with incoherent processing (Hadamard
  rotation of Q and K, per-block E4M3 quantisation, E4M3 P), in float64.
* ``dropout``    -- Philox4x32-10 and the dropout keep masks it defines;
  ``attention`` takes the keep mask (and a key-padding length) as inputs.

Every function here is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_fp8.py``, ``tests/test_oracle_dropout.py`` against closed
forms, invariants, finite differences, independent library routines and a
constructed worked example (``tests/golden/``).  No function is
parity-unpinned.
"""
from .attention import (  # noqa: F401
    keep_matrix, forward_head, backward_head, forward, backward,
    delta_closed_form, softmax_rows,
)
from .online import online_forward_head  # noqa: F401
from .splitkv import split_forward_head  # noqa: F401
from . import fp8  # noqa: F401
from . import dropout  # noqa: F401
