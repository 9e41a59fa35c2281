"""CPU fp64 oracle for KDA.  Test infrastructure: only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import anything from here."""
