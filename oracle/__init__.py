"""Plain fp64 CPU oracle for the MoE layer forward pass (test infrastructure:
only tests, the smoke check and the benchmark's CPU-baseline leg use it)."""
