"""CPU oracle for the DeepSeekMoE layer forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP library never does.
"""
