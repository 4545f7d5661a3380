"""msa_decode_noalloc: msa_decode with the workspace taken from the array the
library holds on each device, for callers that cannot allocate.  Checked
through the C ABI against msa_decode on a caller workspace, on calls in a
row whose second input is smaller (the array keeps the previous call's
contents), and against the oracle."""
import pytest
import torch

import block_sparse_attention_10_amd as msa
from synth import make_workload, small_config
from tests.msa_gpu import TOL, compare_rows, problem_for, run_fused, tensors_for

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(w):
    c = w.cfg
    p = problem_for(w)
    t = tensors_for(w)
    o = {"selected": torch.full((c.rows, c.topk), -7, dtype=torch.int32, device=DEV),
         "page_table": torch.full((c.rows, c.topk * 8), -7, dtype=torch.int32, device=DEV),
         "out": torch.full((c.rows, c.num_q_heads, 128), float("nan"), device=DEV)}
    msa.msa_decode_noalloc(p, t, o["selected"], o["page_table"], o["out"])
    torch.cuda.synchronize()
    return o, msa.msa_last_dispatch()


# (first call, second call with a smaller input): single-row requests whose
# rows split over several workgroups (partials and the merge in the
# scratch), and multi-row requests (selection launch, tables in the scratch)
CASES = [
    (dict(batch=4, query_len=1, ctx_lo=20000, ctx_hi=40000, num_q_heads=16, num_kv_heads=2,
          num_idx_heads=2, n_plant=4, seed=41),
     dict(batch=2, query_len=1, ctx_lo=3000, ctx_hi=9000, num_q_heads=16, num_kv_heads=2,
          num_idx_heads=2, n_plant=2, seed=42)),
    (dict(batch=6, query_len=4, ctx_lo=8192, ctx_hi=16384, kv_dtype="fp8", idx_dtype="fp8",
          seed=43),
     dict(batch=3, query_len=2, ctx_lo=1000, ctx_hi=5000, kv_dtype="fp8", idx_dtype="fp8",
          seed=44)),
]


@pytest.mark.parametrize("first,second", CASES, ids=["single_row_split", "multi_row"])
def test_noalloc_matches_msa_decode_on_calls_in_a_row(first, second):
    for kw in (first, second):
        cfg = small_config(**kw)
        print(f"msa_decode_noalloc: {kw}", flush=True)
        w = make_workload(cfg, DEV)
        want = run_fused(w)
        got, rec = _noalloc(w)
        for k in ("selected", "page_table", "out"):
            assert torch.equal(got[k], want[k]), f"{k} differs from msa_decode"
        err = compare_rows(w, got, list(range(cfg.rows)))
        assert err <= TOL[cfg.kv_dtype]
        assert "index_scan" in rec and "sparse_attn" in rec, rec


def test_noalloc_without_exported_tables_and_repeats():
    cfg = small_config(batch=3, query_len=1, ctx_lo=5000, ctx_hi=30000, seed=45)
    w = make_workload(cfg, DEV)
    want = run_fused(w, export=False)
    p = problem_for(w)
    t = tensors_for(w)
    out = torch.empty_like(want["out"])
    for _ in range(3):
        out.fill_(float("nan"))
        msa.msa_decode_noalloc(p, t, None, None, out)
        torch.cuda.synchronize()
        assert torch.equal(out, want["out"])


@pytest.mark.parametrize("kw", [
    dict(batch=3, query_len=1, ctx_lo=1500, ctx_hi=9000, seed=46),
    dict(batch=2, query_len=4, ctx_lo=3000, ctx_hi=20000, kv_dtype="fp8", idx_dtype="fp8",
         seed=47),
], ids=["bf16_T1_split", "fp8_T4"])
def test_noalloc_captured_into_a_graph(kw):
    """The case it exists for: captured once into a HIP graph (no allocation
    inside the capture), replayed with the queries changed in place, each
    replay equal bit for bit to msa_decode on a caller workspace."""
    cfg = small_config(**kw)
    w = make_workload(cfg, DEV)
    t = w.tensors
    p = problem_for(w)
    tt = tensors_for(w)
    R = cfg.rows
    sel = torch.empty((R, cfg.topk), dtype=torch.int32, device=DEV)
    pt = torch.empty((R, cfg.topk * 8), dtype=torch.int32, device=DEV)
    out = torch.empty((R, cfg.num_q_heads, 128), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        msa.msa_decode_noalloc(p, tt, sel, pt, out)  # first call on the device: set-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        msa.msa_decode_noalloc(p, tt, sel, pt, out)
    q0 = t["q"].clone()
    iq0 = t["idx_q"].clone()
    for step in range(3):
        if step:
            t["q"].copy_(q0.roll(step, dims=1))
            t["idx_q"].copy_(iq0 * (step + 1))
        out.fill_(float("nan"))
        sel.fill_(-7)
        pt.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = run_fused(w)
        assert torch.equal(sel, want["selected"]), step
        assert torch.equal(pt, want["page_table"]), step
        assert torch.equal(out, want["out"]), step
