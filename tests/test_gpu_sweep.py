"""Seeded sweep of small configurations: stage-wise and fused paths against
the oracle.

The shapes are drawn once from a fixed seed (listed in the test ids): 1-5
requests, 1-16 rows per request, GQA groups of 1-16 query heads, 1-4 KV and
index heads, every KV and index-key format, topk 1-16, ragged contexts down
to the row count, planted blocks or none, permuted pools or not.  This
crosses the paths (VALU and matrix-core scans, threshold and list
selection, split and unsplit attention) in combinations the hand-picked
shapes do not.  Same bar as the other parity tests: scores, selections and
page tables bit for bit, outputs within 2e-3 (bf16 KV) or 1e-2.
"""
import os

import numpy as np
import pytest
import torch

from synth import make_workload, small_config
from tests.msa_gpu import (TOL, check_invariants, compare_rows, oracle_rows, run_fused,
                           run_stages)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _draw(n, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([1, 1, 2, 3, 4, 5, 8, 16]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hidx = int(rng.choice([1, 2, 4]))
        kv = str(rng.choice(["bf16", "fp8", "nvfp4"]))
        idx = str(rng.choice(["bf16", "fp8", "nvfp4"]))
        topk = int(rng.choice([1, 2, 8, 16, 16, 16]))
        B = int(rng.integers(1, 6))
        hi = int(rng.integers(max(T, 200), 12000))
        lo = int(rng.integers(T, hi + 1))
        out.append(dict(batch=B, query_len=T, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                        num_idx_heads=Hidx, kv_dtype=kv, idx_dtype=idx, topk=topk,
                        ctx_lo=lo, ctx_hi=hi, n_plant=int(rng.integers(0, 5)),
                        permute=bool(rng.integers(0, 2)), seed=5000 + i))
    return out


# MSA_SWEEP_CASES / MSA_SWEEP_SEED widen the sweep for a longer run, e.g.
# MSA_SWEEP_CASES=600 MSA_SWEEP_SEED=4242 python -m pytest tests/test_gpu_sweep.py
CASES = _draw(int(os.environ.get("MSA_SWEEP_CASES", "24")),
              seed=int(os.environ.get("MSA_SWEEP_SEED", "20261202")))


def _id(kw):
    return (f"B{kw['batch']}T{kw['query_len']}q{kw['num_q_heads']}kv{kw['num_kv_heads']}"
            f"i{kw['num_idx_heads']}-{kw['kv_dtype']}-{kw['idx_dtype']}-k{kw['topk']}"
            f"-L{kw['ctx_lo']}_{kw['ctx_hi']}")


@pytest.mark.parametrize("kw", CASES, ids=[_id(k) for k in CASES])
def test_random_configuration(kw):
    cfg = small_config(**kw)
    print(f"sweep case {_id(kw)}", flush=True)
    w = make_workload(cfg, DEV)
    rows = list(range(cfg.rows))
    ref = oracle_rows(w, rows)
    got = run_stages(w)
    err = compare_rows(w, got, rows, ref)
    fused = run_fused(w)
    for k in ("selected", "page_table", "out"):
        assert torch.equal(fused[k], got[k]), f"fused {k} differs from stage-wise"
    check_invariants(w, fused)
    assert err <= TOL[cfg.kv_dtype]
