"""CPU oracle for the routed MoE feed-forward layer (test infrastructure only:
used by the tests, the smoke check and the benchmark's CPU-baseline leg)."""
