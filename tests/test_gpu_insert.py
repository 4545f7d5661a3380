"""GPU parity of the write path (msa_insert_kv) against the CPU oracle.

The pools after the insert must equal the oracle's, byte for byte (the
quantised codes and scales are integers decided in fp32 on both sides);
then the decode step that follows, run on the updated pools, must match
the oracle on the same pools.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_10_amd as msa
import oracle
from synth import make_workload, small_config
from tests.msa_gpu import compare_rows, oracle_rows, run_fused
from tests.refs import problem_of

pytestmark = pytest.mark.gpu

DEV = "cuda"
POOLS = ("k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool", "idx_k_scale")


def _host(x):
    x = x.detach().to("cpu")
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


@pytest.mark.parametrize("kv,idx,T,seed", [
    ("bf16", "bf16", 1, 51),
    ("fp8", "fp8", 3, 52),
    ("nvfp4", "nvfp4", 1, 53),
    ("bf16", "nvfp4", 2, 54),
    ("nvfp4", "fp8", 4, 55),
    ("fp8", "bf16", 1, 56),
])
def test_insert_matches_oracle_then_decode(kv, idx, T, seed):
    cfg = small_config(batch=3, query_len=T, ctx_lo=200, ctx_hi=5000, kv_dtype=kv,
                       idx_dtype=idx, num_q_heads=8, num_kv_heads=2, num_idx_heads=2,
                       seed=seed)
    print(f"insert {kv}/{idx} T={T}", flush=True)
    w = make_workload(cfg, DEV)
    t = w.tensors
    R = cfg.rows
    rng = np.random.default_rng(seed)
    k_new = torch.from_numpy(rng.standard_normal((R, 2, 128)).astype(np.float32) * 3)
    v_new = torch.from_numpy(rng.standard_normal((R, 2, 128)).astype(np.float32))
    i_new = torch.from_numpy(rng.integers(-8, 9, (R, 2, 64)).astype(np.float32))
    k_new[0, 0, :16] = 0.0          # an all-zero 4-bit group and fp8 row part
    v_new[-1, 1, 5] = -1e-6         # rounds to zero: stored as +0 in 4-bit
    new = [x.to(torch.bfloat16) for x in (k_new, v_new, i_new)]
    ref = {n: (None if t[n] is None else _host(t[n]).copy()) for n in POOLS}
    oracle.insert(problem_of(cfg), *(_host(x) for x in new), _host(t["block_table"]),
                  _host(t["ctx_lens"]), ref)

    p = msa.describe(t["q"], t["idx_q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"],
                     t["idx_k_pool"], t["block_table"], t["ctx_lens"], decode_query_len=T,
                     topk=cfg.topk, idx_k_scale=t.get("idx_k_scale"))[0]
    pl = msa.pools(*(t[n] for n in POOLS))
    dn = [x.to(DEV) for x in new]
    msa.msa_insert_kv(p, pl, t["block_table"], t["ctx_lens"], *dn)
    torch.cuda.synchronize()
    assert msa.msa_last_dispatch().startswith("insert<")
    for n in POOLS:
        if t[n] is None:
            continue
        got = _host(t[n])
        assert np.array_equal(got, ref[n]), f"{n} differs after insert"

    # the decode step that follows sees the new tokens
    got = run_fused(w)
    rows = list(range(R))
    err = compare_rows(w, got, rows, oracle_rows(w, rows))
    print(f"  decode after insert: max abs err {err:.3g}", flush=True)
