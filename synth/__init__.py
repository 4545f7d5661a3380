"""Seeded synthetic workloads for MSA decode (inputs only; no method arithmetic)."""
from .generate import (BLOCK, CONFIG_ORDER, CONFIGS, EXTRA_CONFIGS, HEAD_DIM, IDX_DIM,  # noqa: F401
                       PAGE,
                       MSAConfig, Workload, encode_e2m1, encode_fp8_per_token,
                       encode_nvfp4, host_arrays, layout, make_workload, rand32,
                       small_config, write_spec)
