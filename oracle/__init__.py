"""CPU reference (the oracle) for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, helpers, constants or pre/post-processing).

Contents
--------
attention.py  plain float64 numpy definition of attention forward (two-pass
              softmax, never online) and of its gradient (softmax Jacobian).
brute.py      40-digit ``decimal`` brute force of the forward for tiny shapes,
              used only to pin ``attention.py``.

Parity status: every public function here is pinned by ``tests/test_oracle.py``
(brute force, closed forms, invariants, finite differences, mutation checks).
"""

from .attention import attention_fwd, attention_fwd_head, attention_bwd, attention_bwd_head
from .brute import brute_fwd_decimal

__all__ = [
    "attention_fwd",
    "attention_fwd_head",
    "attention_bwd",
    "attention_bwd_head",
    "brute_fwd_decimal",
]
