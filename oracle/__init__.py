"""CPU oracle for paged-KV attention: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does.
"""
