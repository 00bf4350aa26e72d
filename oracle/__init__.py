"""CPU reference (the oracle) for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, helpers, constants or pre/post-processing).

Contents
--------
attention.py  plain float64 numpy definition of attention forward (two-pass
              softmax, never online) and of its gradient (softmax Jacobian).
kvcache.py    plain float64 definition of a few new queries attending to a
              key/value cache (fewer queries than keys, bottom-right causal
              mask, per-batch filled lengths), its gradient (softmax
              Jacobian), and variable-length packed batches built from both.
brute.py      40-digit ``decimal`` brute force of both forwards for tiny
              shapes, used only to pin ``attention.py`` and ``kvcache.py``.

Parity status: every public function here is pinned by ``tests/test_oracle.py``
(brute force, closed forms, invariants, finite differences, mutation checks).
"""

from .attention import attention_fwd, attention_fwd_head, attention_bwd, attention_bwd_head
from .brute import brute_fwd_decimal, brute_kvcache_decimal
from .kvcache import kvcache_bwd_head, kvcache_fwd, kvcache_fwd_head, varlen_bwd, varlen_bwd_causal, varlen_fwd

__all__ = [
    "attention_fwd",
    "attention_fwd_head",
    "attention_bwd",
    "attention_bwd_head",
    "brute_fwd_decimal",
    "brute_kvcache_decimal",
    "kvcache_fwd",
    "kvcache_fwd_head",
    "varlen_fwd",
    "varlen_bwd_causal",
    "kvcache_bwd_head",
    "varlen_bwd",
]
