"""CPU oracle for the sampled-softmax cross-entropy step -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from here. The HIP library never calls it, and the oracle shares
no code with the HIP sources: the two meet only through the seeded input
generator, which holds none of the method's arithmetic.

* ``candidates``: the candidate build, sequential plain C (``candidates.c``).
* ``ce_c``: loss and gradients in plain C with float64 accumulation and OpenMP over
  token blocks (``ce.c``): the oracle the GPU parity tests and the benchmark's CPU
  baseline use, dense or for chosen rows and columns at full size.
* ``ce``: the same definition in float64 numpy, written independently; the tests pin
  the C oracle to it (and both to PyTorch, finite differences and closed forms).
* ``fp8``: the e4m3-operand variant of the step (e4m3 codec, power-of-two
  per-tensor scales, bf16 logits) in float64 numpy.

Every function states the passage of the pages it follows. Parity pins live in
``tests/test_oracle_*.py``; functions without an independent pin say so.
"""
from .candidates import build_candidates, OracleError  # noqa: F401
from . import ce  # noqa: F401
from . import ce_c  # noqa: F401
from . import fp8  # noqa: F401
