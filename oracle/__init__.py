"""CPU oracle for SubMConv3d. TEST INFRASTRUCTURE: imported only by the tests,
the smoke check and the benchmark's CPU-baseline leg; never by the library."""
