"""Oracle for the exact attention forward: a plain, slow, float64 CPU
implementation of what the fused kernel must compute.

TEST INFRASTRUCTURE ONLY.  This package is imported by the test suite, by the
package's ``smoke()`` check and by the benchmark's CPU-baseline leg, and by
nothing else.  The GPU path neither imports it nor shares any code with it;
the two meet only in the seeded inputs (``seeded_inputs``), which hold no
attention arithmetic.

Contents
  attention        -- materialised definition (scores, mask, row softmax, PV,
                      log-sum-exp); pinned by tests/test_oracle_pins.py.
  backward         -- gradients dQ, dK, dV (and Delta) of the materialised
                      definition for an upstream gradient dO; pinned by
                      tests/test_oracle_bwd_pins.py.
  decode           -- a few new queries over a key/value cache (queries at the
                      last positions, bottom-right causal mask); pinned by
                      tests/test_oracle_decode_pins.py.
  gqa              -- grouped key/value heads (query head h reads key/value
                      head h // (H / H_kv)) for the forward and the backward;
                      pinned by tests/test_oracle_gqa_pins.py.
  online_model     -- a float64 model of the tiled recurrence with running
                      max, running normaliser and rescaled accumulator, plus
                      the per-tile-normalisation negative control.  It is not
                      the oracle; it checks the method itself against the
                      oracle.

Pages followed (cited by title and section):
  [P1] "Why Attention Is Difficult to Optimize" (llm-systems-engineering)
  [P2] "Attention Mechanism: Computation & Memory Patterns" (grasp.study)
  [P3] "FlashAttention -- avoid writing the giant intermediate" (sanketn26)

Parity unpinned: nothing in this package.  Every function is pinned by at
least one test that checks it against a value the pages print, a closed form,
an invariant or an independent brute force.
"""
from .attention import attention, attention_head, attention_heads  # noqa: F401
from .backward import attention_head_bwd  # noqa: F401
from .decode import attention_decode, attention_decode_head  # noqa: F401
from .gqa import attention_gqa, attention_gqa_bwd, kv_head  # noqa: F401
from .online_model import online_attention_head, tile_local_softmax_head  # noqa: F401
