"""Plain, slow CPU oracle for the chunked fast-weight scan (numpy, fp64).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this package. The library's product path never calls it: when the
HIP library is missing, the product path raises instead of falling back to anything here.

The oracle shares no code with the HIP path and does not import the input generators. Every
function takes plain arrays, widens them to fp64 and follows the source pages' statement of the
method, citing the passage it implements:

* ``inplace``     In-Place TTT: apply the pre-update W_down to chunk i, then add
                  eta * V_hat_i^T Z_i (In-Place TTT page, sections 2, 3, 4 and 6).
* ``ttt_linear``  TTT-Linear: one mini-batch gradient step of the reconstruction loss per
                  mini-batch, output in dual form (TTT layers page; DeltaNet equivalence).
* ``route``       SR-TTT surprisal filter, EMA-smoothed 95th-percentile threshold, chunk-mean
                  condition and a fixed-capacity residual cache (SR-TTT page, section 2.1 and 5).

Parity pins (tests marked ``not gpu``) tie each function to closed forms, invariants, brute
force on tiny inputs and library routines, never to itself.
"""
from . import inplace, ttt_linear, route  # noqa: F401
