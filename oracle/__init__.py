"""CPU oracle for one QSA layer -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP product path never does.
"""
