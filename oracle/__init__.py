"""fp64 CPU oracle for paged decode attention and its block bookkeeping.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product
package never imports it and shares no code with it.
"""
