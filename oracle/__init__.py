"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and nothing
here imports the product path.

Sources (the three web pages on FlashAttention; cited by title + section):

* [DEC] "FlashAttention, Decoded: What 'IO-Aware' Actually Means"
  (pinghaoyang.com.cn) — sections "The Passage" (the abstract),
  "Decoding the Abstract" (Sentence 1 ... Sentences 5-8),
  "The Hardware Picture: Why Tiling Wins", "Key Vocabulary".
* [HFL] "FlashAttention: A Novel Attention Algorithm with IO Awareness, Fast
  and Memory-Efficient" (high-flyer.in.suopu.cc post 504) — sections
  "contexts", "Standard Attention Algorithm", "FlashAttention".
* [ODP] "FlashAttention: Fast and Memory-Efficient Exact Attention with
  IO-Awareness" (opendecode.dev paper page) — sections "What problem it
  solved", "The key idea", "Why it mattered".

Modules:

* :mod:`oracle.attention` — the definition of attention written out in numpy
  fp64 (materialised score matrix, row softmax, P·V) and its analytic
  backward; sampled-row variants for long sequences; and a CPU model of the
  tiled online-softmax method, used only to check the pages' exactness claim.
* :mod:`oracle.bruteforce` — pure-Python loops with ``math.exp``/``math.fsum``
  for tiny shapes.
* :mod:`oracle.closed_forms` — attention at q = 0 (uniform rows) from running
  or per-block sums, exact at the full workload sizes.

Every function here is pinned by ``tests/test_oracle.py`` (and the dropout
functions by ``tests/test_oracle_dropout.py``) against closed forms,
invariants, finite differences, a library routine (torch autograd in
float64 on the CPU), published known-answer vectors of the random number
generator and a hand-derived worked example in ``tests/golden/``.  Nothing
in this package is "parity unpinned".
"""

from .attention import (  # noqa: F401
    allowed_mask,
    attention_fwd,
    attention_bwd,
    attention_rows,
    attention_key_grads,
    online_softmax_attention,
)
from .closed_forms import q_zero_attention  # noqa: F401
from .dropout import (  # noqa: F401
    attention_bwd_dropout,
    attention_fwd_dropout,
    drop_threshold,
    keep_mask,
    philox4x32_10,
)
