"""CPU oracle for the per-token mixed-precision KV transfer path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the package's
smoke check and the benchmark's CPU-baseline leg may import anything from
here.  The GPU library never calls it, and it shares no code with the GPU
library: no kernels, headers, helpers, tables or constants.  The only code
both sides use is the seeded input generator package ``workloads``, which
holds none of the method's arithmetic.

Every function is the plain, slow definition of one step, written from the
SpectrumKV paper (arXiv 2606.08635) and cited by section / equation /
algorithm:

* :mod:`oracle.plan`   - budget -> tier counts, payload byte count and layout
* :mod:`oracle.score`  - token importance A_j (causal softmax column sums), fp64
* :mod:`oracle.assign` - sink pinning + importance-sorted tier assignment
* :mod:`oracle.quant`  - symmetric absmax quantizer, pack and unpack

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force, library routines or hand-worked
examples (``tests/golden``).  Downstream model quality (perplexity, NIAH) is
outside this oracle and parity unpinned.
"""

from . import plan, score, assign, quant  # noqa: F401
