"""CPU oracle of the dropless top-k MoE layer. TEST INFRASTRUCTURE ONLY:
imported by tests, the smoke check and the benchmark's CPU-baseline leg."""
