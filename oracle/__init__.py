"""fp64 CPU oracle for decode attention -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline
leg may import anything from here; the GPU library never does.
"""
