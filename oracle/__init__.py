"""Plain, slow, fp64 CPU oracle for fused training attention and for the
soft-target log-softmax loss that follows it in EAGLE3 training.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
helper with the HIP library in ``flash_attention_fa_amd/``.

Every result here is the textbook definition written out in float64 with the
whole S x S score matrix materialised (row-blocked only to bound RAM; every
score row is complete), or the whole [rows, vocabulary] logit matrix for the
loss.  See ``oracle/attention.py`` and ``oracle/loss.py`` for the citations.

Parity pins (tests/test_oracle_pins.py): fp64 torch SDPA and torch autograd
(library routines), central finite differences, closed forms in
tests/golden/, invariants, the step-by-step EAGLE3 TTT formulation
(``oracle/ttt_steps.py``) and brute-force predicate enumeration; for the loss
(tests/test_oracle_pins_loss.py) torch's cross_entropy on one-hot targets,
closed forms, invariants and finite differences.  No function in this
package is "parity unpinned".
"""
from .attention import (  # noqa: F401
    FULL, CAUSAL, TTT, WINDOW,
    allowed, attention_forward, attention_backward, attention_ref,
    allowed_pair_count, attention_key_grads,
)
from .ttt_steps import ttt_stepwise_forward  # noqa: F401
from .loss import logsoftmax_loss_forward, logsoftmax_loss_backward  # noqa: F401
