"""fp64 CPU oracle of the pi0 action-expert denoise loop.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product package never imports it.
"""
