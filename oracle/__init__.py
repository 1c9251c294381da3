"""CPU oracle for the structured-sparse plus low-rank linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
load this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library.

It is a plain, slow, obviously correct restatement of what the layer
computes, in float64 over inputs that hold the exact storage-dtype values:

* ``oracle.nm``    N:M magnitude pruning along the reduction dim, the canonical
                   compressed format, and the double-pruned transpose
                   (SLoPe paperlayer summary, §1 and §2.1 "Double-pruned
                   backward pass"; §2.3 "Sparse kernels").
* ``oracle.ffi``   fixed fan-in selection (exactly k kept per output row) and
                   the exact transpose (SQuAsh project update; SLoPe §2.3 keeps
                   a format for the weight and one for its transpose).
* ``oracle.layer`` forward ``Y = X Ws^T + (X A^T) B^T`` and the backward
                   ``dU, dB, dA, dX`` (SLoPe §2.2 "Lazy low-rank adapters";
                   LoRA as described in "efficient training for the gpu-poor",
                   section PEFT).

* ``oracle.layer`` also holds SQuAsh's variant, an adapter whose down-projection
                   factor is itself fixed-fan-in sparse (SQuAsh project update,
                   first paragraph), and the masked weight gradient and sparse
                   update of SLoPe's sparse training (§2.1, §2.3).

Every function is pinned by ``tests/test_oracle_pins.py`` against brute force,
invariants, library routines (torch autograd, ``F.linear``) and the added
sparsity that SLoPe's Lemma 2.1 (§2.1, proof in App. T.1) predicts, at 1:2,
2:4 and 2:8.  The page's printed 2:8 figure itself is not reproduced by the
binomial model the same appendix describes; it is recorded, not enforced.
"""
from . import ffi, layer, nm  # noqa: F401
