"""CPU oracle for the Mamba-3 physical-frame state moments (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``mamba_ssm_chunkwise_amd``)
never imports it, and it imports nothing from the product path.

Two independent CPU implementations live here:

* ``moments_oracle.c`` (fp64, threaded over (b,h) chains): the per-token
  recurrence the chunked method reaches exactly, with its own reverse-time
  matrix-form adjoint. It is the reference every GPU result is compared with.
* ``pages_form.py`` (numpy fp64): a loop transcription of the pages' chunkwise
  algebra (chunk decay, triangular chunk states, boundary carries, the reverse
  chunk loop with G, d_W = L^T G and the rev-cumsum d_da identity). It exists to
  pin the oracle: chunk-length invariance and the d_da identity.

Parity pins (see ``tests/test_oracle_pins.py``): finite differences, torch
float64 autograd, chunk-length invariance, the rotation-orthogonality trace
identity, closed forms, zero gradients past valid_len, d_m2 antisymmetric
invariance and an adjoint (dot-product) test. No function here is
"parity unpinned".
"""
from .oracle import (  # noqa: F401
    ROT_NONE, ROT_PAIRWISE, ROT_HALF, ROT_QUAT, build, library_path, oracle_fwd, oracle_bwd,
)
