"""CPU oracle for MLA chunked prefill and absorbed decode.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does. It shares no code
with the HIP path and imports nothing from it.
"""
