"""CPU oracle for the deterministic attention backward: test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never calls it and shares no code with it.

Contents
--------
attention : fp64 textbook attention forward and backward (numpy).
schedule  : the DASH reference schedules, the DAG critical-path simulator and a
            table validator (pure Python).

Sources: "DASH: Deterministic Attention Scheduling for High-throughput
Reproducible LLM Training" (arXiv 2601.21824), sections 2.1 and 3; "Writing an
Attention Kernel: FlashAttention and Decode in Triton" (vidyal.ai), Step 1 and
"In the real world".
"""
