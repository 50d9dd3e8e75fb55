"""CPU oracle for the batched speculative-sampling verify step (test infrastructure).

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product library never does.
"""
