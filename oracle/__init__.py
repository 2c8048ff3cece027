"""CPU oracle for the Mamba-3 physical-frame state moments (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``mamba_ssm_chunkwise_amd``)
never imports it, and it imports nothing from the product path.

Two independent CPU implementations live here:

* ``moments_oracle.c`` (fp64, threaded over (b,h) chains): the per-token
  recurrence the chunked method reaches exactly, with its own reverse-time
  matrix-form adjoint. It is the reference every GPU result is compared with.
* ``chunk_form.py`` (numpy fp64): the chunkwise block form of the same
  computation at any chunk length l, written from the equations with the chunks
  as an array axis, and its adjoint with three forms of the decay gradient. It
  exists to pin the oracle: chunk-length invariance (including the oracle's
  checkpointed backward over several 256-token segments) and the d_da identity.

* ``rotation_seq.py`` (numpy fp64): the rotation-sequence producer upstream of
  the moments path (inclusive angle sums; left-to-right renormalised Hamilton
  products of quaternion increments) and its reverse-mode VJP, pinned in
  ``tests/test_rotation_seq.py`` (scipy rotation composition, matrix products,
  a coaxial closed form, finite differences, scale invariance, and the moments
  gradient with respect to the increments).

Parity pins (see ``tests/test_oracle_pins.py``): finite differences, torch
float64 autograd, chunk-length invariance, the rotation-orthogonality trace
identity, closed forms, zero gradients past valid_len, d_m2 antisymmetric
invariance and an adjoint (dot-product) test. No function here is
"parity unpinned".
"""
from .oracle import (  # noqa: F401
    ROT_NONE, ROT_PAIRWISE, ROT_HALF, ROT_QUAT, build, library_path, oracle_fwd, oracle_bwd,
)
