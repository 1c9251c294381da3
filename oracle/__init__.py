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

Every function is pinned by ``tests/test_oracle_pins.py`` against brute force,
invariants, library routines (torch autograd, ``F.linear``) and the added
sparsity that SLoPe's Lemma 2.1 (§2.1, proof in App. T.1) predicts.  The one
unpinned figure is Lemma 2.1's 2:8 value (parity unpinned: the printed number
does not follow from the binomial model the same appendix describes).
"""
from . import ffi, layer, nm  # noqa: F401
