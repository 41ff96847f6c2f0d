"""CPU float64 oracle for exact scaled dot-product attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package. The product path (``exact_tiled_attention_05_amd``) never
imports it, links it or falls back to it, and the oracle shares no code with the GPU path.

Contents
--------
attention.py  -- the plain definition: materialise S = scale * Q K^T, mask, stable softmax,
                 O = P V and LSE = m + ln(l), in float64, one (batch, head) at a time; and the
                 grouped-K/V-head form (each query head with its assigned K/V head), the
                 decoding form (N_q queries that are the last N_q of N_kv tokens), and the score
                 modifiers (sliding window, ALiBi, additive bias) of attention_ext.
backward.py   -- the gradients of the plain definition (dQ, dK, dV from dO), dense, in float64,
                 per head and with grouped K/V heads.
online.py     -- the pages' streaming recurrences (online normaliser, blockwise (m, l, a)
                 merge, tiled forward with queries outermost). A test model only: it is pinned
                 to attention.py, it is not what the GPU is compared against.

Every function is pinned by ``tests/test_oracle*.py`` and ``tests/test_online_model.py`` to
something other than itself: the worked example printed on the pages, closed forms,
invariants, brute force in scalar Python, and float64 library routines.
"""
from .attention import (attention, attention_decode, attention_ext, attention_gqa,  # noqa: F401
                        attention_head, dense_scores, kv_head_of)
from .backward import attention_backward, attention_backward_head  # noqa: F401
from .online import online_normalizer, blockwise_row, tiled_attention  # noqa: F401
