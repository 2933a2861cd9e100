"""fp64 CPU oracle for the KDA recurrent-state path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP library never does.
"""
