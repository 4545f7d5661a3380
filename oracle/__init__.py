"""Plain CPU oracle for MSA decode (test infrastructure only).

Imported by the tests, the smoke entry and the benchmark's CPU-baseline leg;
never by the GPU library.  See ``oracle.py`` and ``msa_oracle.c``.
"""
from .oracle import (OracleProblem, attention, bf16_to_double, build, decode,  # noqa: F401
                     e2m1_to_double, e4m3_to_double, f32_to_e2m1, f32_to_e4m3, index_scores,
                     insert, num_threads, page_table, select, set_num_threads)
