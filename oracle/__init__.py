"""CPU oracle for the activation-sparse linear layer: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``sparse_input_gemv_amd/`` never imports it, and it imports nothing from the
library: the two share no code.  Inputs reach both sides from ``synthetic``.

Every function is the plain definition of what the pages compute, written in
fp64 numpy with no blocking, fusion or reordering beyond that definition.
fp16 inputs are widened to fp64 exactly before any arithmetic.

Pages cited (by title; "replies" = the authors' answers to reviewers):

* Q-Sparse: All Large Language Models can be Fully Sparsely-Activated (replies)
* TEAL: Training-Free Activation Sparsity in Large Language Models (README)
* Adaptive Rank Allocation: Speeding Up Modern Transformers with RaNA Adapters
  (replies)
* ProSparse: Introducing and Enhancing Intrinsic Activation Sparsity within
  Large Language Models (summary)
* Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity via
  Benchmarking Lightweight Post-Training Sparsification Approaches (summary)

Modules:

* ``sparsify``  threshold, per-token Top-K and N:M masks, tile-shared N:M;
  sparsity; mask packing
* ``gemv``      sparse / dense / batched-union GEMV; FLOP count
* ``swiglu``    SiLU, CATS and RaNA neuron masks, masked down projection
* ``rana``      RaNA linear-layer rank adapter A (m ⊙ B x)
* ``correct``   weight-aware selection, static shift, variance correction
* ``spmm``      batched N:M activation-sparse matmul (per-token and tile-shared)
* ``calibrate`` empirical-quantile thresholds
* ``brute``     exhaustive enumeration for tiny inputs

Every function is pinned by ``tests/test_oracle_*.py`` (run with
``-m "not gpu"``); none is "parity unpinned".
"""

from . import brute, calibrate, correct, gemv, rana, sparsify, spmm, swiglu  # noqa: F401
