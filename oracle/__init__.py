"""CPU oracle for the ParisKV decode path -- test infrastructure only.

Plain, slow, float64/fp32-spec reference code used by the tests, the smoke
check and the bench's CPU-baseline leg.  The HIP library never imports it and
must not fall back to it.
"""
