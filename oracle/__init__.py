"""CPU oracle for blockwise ring attention -- test infrastructure only.

This package is the plain, slow, obviously correct CPU statement of what the
GPU hot path computes.  It is used only by the test suite, by the smoke check
and by the benchmark's CPU-baseline leg; the product path never imports it
and shares no code with it (no kernels, headers, helpers or constants).

Sources (the pages are the authority on *what* is computed):

* "手把手拆解RingAttention" (bjdmk.com.cn), section 1 and its comparison
  table: ring attention keeps the *complete* global attention map -- every
  query block sees every key/value block as K/V travel round the ring while
  each device keeps its query block.
* "RingAttention核心功能全解析" (wmrh.cn), sections "分块注意力计算" and
  "快速上手": the call takes an additive ``attention_bias``, ``segment_ids``,
  ``query_chunk_size`` / ``key_chunk_size`` and ``causal_block_size=1`` for
  causal attention, with a recompute policy (``nothing_saveable``) for the
  backward pass.

Modules
-------
``attention``  the plain definition, softmax(scale*QK^T + bias + mask) V, and
               its gradients, in float64 (``forward``, ``backward``,
               ``bias_grad``, ``probabilities``).
``ffn``        the blockwise feed-forward (SwiGLU) and its gradients, in
               float64.
``blockwise``  the method's own procedure -- ring-order steps over K/V
               blocks, query/key chunks, online-softmax merge -- in float64,
               used to pin the claim that the procedure is exact.

Parity status: every function here is pinned by CPU tests (brute force,
library special case, closed forms, finite differences, invariants); none is
"parity unpinned".
"""
from .attention import (forward, backward, bias_grad, probabilities, query_positions, visible_pairs,  # noqa: F401
                        causal_block)
from .blockwise import ring_forward  # noqa: F401
from .ffn import ffn_forward, ffn_backward  # noqa: F401
