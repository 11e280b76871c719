"""fp64 CPU oracle for paged-attention decode.  Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU baseline, never
by the library."""
