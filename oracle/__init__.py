"""Plain single-threaded fp64 CPU oracle of the MoE-layer forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU product path.
"""
