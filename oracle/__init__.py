"""CPU fp64 oracle for the exact-attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, headers, tables or helpers with the HIP library.

Sources (the web pages this work is built from):

* [P5] "FlashAttention simplified: tiling + online softmax forward pass",
  the teaching script page at forceinjection.github.io (flash_attention.py):
  functions ``standard_attention`` and ``flash_attention_forward`` (its
  numbered online-softmax steps 1-5 and the final normalisation).
* [P3] "2.3 FlashAttention and IO-aware attention" (aiknowledge.cn):
  section 1.1 (standard three-step attention on [batch, heads, seq, head_dim],
  masking with ``masked_fill(mask == 0, -inf)``).
* [P2] "PyTorch 2.2 FlashAttention-2 measured on an RTX 4070" (jsqmd.com):
  section 2 (softmax of the scaled product times V).
* [P1] "Compiling Flash Attention 2.8.3 on Windows with an RTX 3090"
  (intelliparadigm.com): section 5.2 / 10.1 (``softmax_scale=None`` means
  1/sqrt(d); ``causal`` flag; ``window_size`` local-attention window);
  section 9.2 item 2 (the backward recomputes instead of storing); section
  11.2 (inference over long contexts, the use of split-KV partial results
  and their merge).

Parity status: every public function here is pinned by CPU tests (brute force
in 40-digit decimal arithmetic, closed forms, invariants, a hand-derived
fixture and a library cross-check); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    allowed_ref,
    attention_ref,
    attention_tiled_ref,
    scores_ref,
    softmax_rows_ref,
)
from .backward import attention_bwd_ref  # noqa: F401
from .bruteforce import attention_bruteforce  # noqa: F401
from .splitkv import merge_ref, partial_ref  # noqa: F401
