"""CPU oracle of the Echo rank pipeline -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP library.
"""
