"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Block scores, selections and page tables must match bit for bit (index
queries and keys are small integers, so every score is exact); attention
outputs must be within max-abs 2e-3 of the fp64 oracle for bf16 KV and 1e-2
for fp8 / 4-bit KV.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_10_amd as msa
import oracle
from synth import CONFIG_ORDER, CONFIGS, EXTRA_CONFIGS, make_workload, small_config
from tests.msa_gpu import (TOL, alloc_outputs, check_invariants, compare_rows,
                           oracle_attention_rows, oracle_rows, problem_for, run_fused,
                           run_stages, tensors_for)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def test_device_decoders_match_oracle():
    out = torch.empty(832, dtype=torch.float32, device=DEV)
    msa.msa_selftest_decoders(out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    e4 = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    e2 = np.array([oracle.e2m1_to_double(c) for c in range(16)])
    for base in (0, 288, 576):
        got = o[base:base + 256]
        nan = np.isnan(e4)
        assert np.array_equal(np.isnan(got), nan), f"NaN codes differ (base {base})"
        assert np.array_equal(got[~nan], e4[~nan]), f"e4m3 decode differs (base {base})"
    for base in (256, 272, 544, 560):
        assert np.array_equal(o[base:base + 16], e2), f"e2m1 decode differs (base {base})"


SMALL = [
    dict(),
    dict(batch=3, query_len=1, ctx_lo=1, ctx_hi=700, seed=2),
    dict(batch=4, query_len=3, ctx_lo=2000, ctx_hi=9000, num_q_heads=16, num_kv_heads=2,
         num_idx_heads=2, seed=3),
    dict(batch=5, query_len=2, ctx_lo=2, ctx_hi=5000, kv_dtype="fp8", idx_dtype="fp8", seed=4),
    dict(batch=2, query_len=4, ctx_lo=4000, ctx_hi=20000, kv_dtype="fp8", idx_dtype="fp8",
         seed=5),
    dict(batch=3, query_len=1, ctx_lo=3000, ctx_hi=40000, kv_dtype="nvfp4", idx_dtype="fp8",
         num_q_heads=64, num_kv_heads=4, num_idx_heads=4, n_plant=16, seed=6),
    dict(batch=2, query_len=5, ctx_lo=5, ctx_hi=3000, num_q_heads=4, num_kv_heads=4, seed=7),
    dict(batch=2, query_len=1, ctx_list=(128, 2049), topk=4, seed=8),
    dict(batch=3, query_len=2, ctx_list=(2, 256, 1280), topk=1, seed=9),
    dict(batch=1, query_len=16, ctx_list=(4096,), num_q_heads=16, num_kv_heads=1,
         num_idx_heads=16, seed=10),
    # 4-bit index keys, 1 / 2 / 4 rows per scan pass, ragged contexts
    dict(batch=3, query_len=1, ctx_lo=1, ctx_hi=9000, idx_dtype="nvfp4", num_idx_heads=4,
         n_plant=4, seed=23),
    dict(batch=2, query_len=2, ctx_lo=2000, ctx_hi=12000, idx_dtype="nvfp4", num_idx_heads=2,
         num_q_heads=16, num_kv_heads=2, seed=24),
    dict(batch=2, query_len=5, ctx_lo=300, ctx_hi=6000, idx_dtype="nvfp4", kv_dtype="fp8",
         seed=25),
    # single rows around the take-every-block edge (16 blocks = 2048 tokens),
    # where msa_decode selects inside the attention launch
    dict(batch=8, query_len=1, ctx_list=(1, 127, 128, 129, 2047, 2048, 2049, 2177),
         num_q_heads=16, num_kv_heads=2, seed=26),
    # a single row of 9,375 blocks: the in-attention selection reads
    # candidates past its first batch of 8,192
    dict(batch=1, query_len=1, ctx_list=(1200000,), n_plant=6, seed=27),
    # block edges and the 32-token quarters of the four-wave scan (single
    # rows, several index heads)
    dict(batch=8, query_len=1, ctx_list=(1, 33, 64, 95, 127, 128, 129, 2177),
         num_q_heads=8, num_kv_heads=2, num_idx_heads=4, seed=28),
    dict(batch=8, query_len=1, ctx_list=(31, 32, 96, 97, 128, 129, 2048, 2049),
         num_idx_heads=4, idx_dtype="fp8", kv_dtype="fp8", seed=29),
]


# Every scan path (index_scan.hip: VALU passes of 1 / 2 / 4 rows, four waves
# per block for single rows with several heads, the matrix-core scan for one
# index head and for several), with the dispatch that must run.
SCAN_PATHS = [
    ("bf16", 1, 1, "rows1"), ("bf16", 1, 2, "rows1"), ("bf16", 1, 3, "quarters"),
    ("bf16", 1, 5, "quarters"), ("bf16", 1, 16, "quarters"),
    ("bf16", 2, 2, "rows2"), ("bf16", 4, 1, "rows4"),
    ("bf16", 5, 1, "mfma1"), ("bf16", 6, 3, "mfma"),
    ("fp8", 1, 1, "rows1"), ("fp8", 1, 3, "rows1"), ("fp8", 1, 4, "quarters"),
    ("fp8", 1, 6, "quarters"), ("fp8", 1, 8, "quarters"), ("fp8", 2, 1, "mfma1"),
    ("fp8", 3, 2, "mfma"),
    ("nvfp4", 1, 4, "rows1"), ("nvfp4", 3, 2, "rows4"),
]


@pytest.mark.parametrize("idx_dtype,T,hidx,path", SCAN_PATHS,
                         ids=[f"{d}-T{t}-H{h}" for d, t, h, _ in SCAN_PATHS])
def test_index_scan_paths(idx_dtype, T, hidx, path):
    cfg = small_config(batch=3, query_len=T, ctx_lo=100, ctx_hi=7000, idx_dtype=idx_dtype,
                       num_idx_heads=hidx, seed=60 + T + 7 * hidx)
    _say(f"scan path {idx_dtype} T={T} Hidx={hidx} (expect {path})")
    w = make_workload(cfg, DEV)
    p = problem_for(w)
    scores = torch.full((cfg.rows, cfg.max_blocks), 7.0, dtype=torch.float32, device=DEV)
    msa.msa_index_score(p, tensors_for(w), scores)
    torch.cuda.synchronize()
    assert f"index_scan<{idx_dtype},{path}>" in msa.msa_last_dispatch()
    rows = list(range(cfg.rows))
    ref = oracle_rows(w, rows)
    got = scores.cpu().numpy()
    for r in rows:
        nb = ref[r]["scores"].shape[0]
        assert np.array_equal(got[r][:nb].astype(np.float64), ref[r]["scores"]), f"row {r}"
        assert np.all(np.isneginf(got[r][nb:])), f"tail of row {r}"


@pytest.mark.parametrize("kw", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_small_shapes_stagewise_and_fused(kw):
    cfg = small_config(**kw)
    _say(f"small shape {kw}")
    w = make_workload(cfg, DEV)
    rows = list(range(cfg.rows))
    ref = oracle_rows(w, rows)
    got = run_stages(w)
    err = compare_rows(w, got, rows, ref)
    fused = run_fused(w)
    for k in ("selected", "page_table", "out"):
        assert torch.equal(fused[k], got[k]), f"fused {k} differs from stage-wise"
    check_invariants(w, fused)
    _say(f"  max abs err {err:.3g} (tol {TOL[cfg.kv_dtype]})")


@pytest.mark.parametrize("T", [1, 2])
def test_fused_without_exported_tables(T):
    cfg = small_config(batch=3, query_len=T, ctx_lo=3000, ctx_hi=9000, seed=12)
    w = make_workload(cfg, DEV)
    a = run_fused(w, export=True)
    b = run_fused(w, export=False)
    assert torch.equal(a["out"], b["out"])


def test_non_default_stream_and_determinism():
    cfg = small_config(batch=4, query_len=2, ctx_lo=3000, ctx_hi=12000, num_q_heads=16,
                       num_kv_heads=2, seed=13)
    w = make_workload(cfg, DEV)
    base = run_fused(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        again = run_fused(w, stream=s)
    s.synchronize()
    for k in ("selected", "page_table", "out"):
        assert torch.equal(base[k], again[k])
    for _ in range(5):
        rep = run_fused(w)
        assert torch.equal(rep["out"], base["out"])


def test_concurrent_streams_with_own_workspaces():
    """Two msa_decode calls in flight at once, on two streams with their
    own workspaces and outputs (a single-row layer and an fp8 verify layer),
    give the bits the same calls give one after the other: the library
    keeps no state between calls on one device beyond what the caller
    passes."""
    wa = make_workload(small_config(batch=6, query_len=1, ctx_lo=20000, ctx_hi=60000,
                                    num_q_heads=16, num_kv_heads=2, num_idx_heads=2, seed=61), DEV)
    wb = make_workload(small_config(batch=8, query_len=4, ctx_lo=3000, ctx_hi=12000,
                                    kv_dtype="fp8", idx_dtype="fp8", seed=62), DEV)
    ref = [run_fused(wa), run_fused(wb)]
    jobs = []
    for w in (wa, wb):
        p = problem_for(w)
        jobs.append((p, tensors_for(w), alloc_outputs(w, p), torch.cuda.Stream()))
    torch.cuda.synchronize()
    for _ in range(3):
        for p, t, o, s in jobs:
            with torch.cuda.stream(s):
                msa.msa_decode(p, t, o["selected"], o["page_table"], o["out"], o["workspace"], s)
    torch.cuda.synchronize()
    for (p, t, o, s), r in zip(jobs, ref):
        for k in ("selected", "page_table", "out"):
            assert torch.equal(o[k], r[k]), k


def test_dispatch_record_names_kernels():
    cfg = small_config(batch=2, ctx_lo=3000, ctx_hi=5000, seed=14)
    w = make_workload(cfg, DEV)
    run_fused(w)
    rec = msa.msa_last_dispatch()
    for name in ("index_scan<bf16", "select_topk", "sparse_attn<bf16>"):
        assert name in rec, rec
    p = problem_for(w)
    t = tensors_for(w)
    scores = torch.empty((cfg.rows, cfg.max_blocks), dtype=torch.float32, device=DEV)
    msa.msa_index_score(p, t, scores)
    assert msa.msa_last_dispatch().startswith("index_scan<bf16")


@pytest.mark.parametrize("kw", [
    dict(batch=3, query_len=2, ctx_lo=3000, ctx_hi=9000, seed=16),
    dict(batch=1, query_len=1, ctx_list=(70000,), num_q_heads=16, num_kv_heads=4,
         num_idx_heads=2, seed=17),
])
def test_workspace_reuse_across_calls_and_entry_points(kw):
    """One workspace, never cleared, serves many calls, alternating the fused
    and the stage-wise attention entry points."""
    cfg = small_config(**kw)
    w = make_workload(cfg, DEV)
    ref = run_stages(w)
    p = problem_for(w)
    t = tensors_for(w)
    ws = torch.full((msa.msa_workspace_bytes(p),), 0xA5, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(ref["out"])
    sel = torch.empty_like(ref["selected"])
    pt = torch.empty_like(ref["page_table"])
    for i in range(6):
        out.zero_()
        if i % 2 == 0:
            msa.msa_decode(p, t, sel, pt, out, ws)
        else:
            msa.msa_sparse_decode(p, t, ref["page_table"], out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref["out"]), f"call {i}"
        if i % 2 == 0:
            assert torch.equal(sel, ref["selected"]) and torch.equal(pt, ref["page_table"])


@pytest.mark.parametrize("kw", [
    dict(batch=3, query_len=2, ctx_lo=3000, ctx_hi=20000, num_q_heads=16, num_kv_heads=2,
         num_idx_heads=2, seed=21),
    dict(batch=2, query_len=1, ctx_lo=5000, ctx_hi=30000, kv_dtype="fp8", idx_dtype="fp8",
         seed=22),
])
def test_cross_layer_reuse_of_the_selection(kw):
    """Index sharing across adjacent sparse layers: layer 0 selects, layer 1
    attends over layer 0's page table through msa_sparse_decode (no scan, no
    selection of its own).  The block table is shared by the layers."""
    cfg = small_config(**kw)
    w0 = make_workload(cfg, DEV)
    w1 = make_workload(cfg, DEV, layer=1)
    assert torch.equal(w0.tensors["block_table"], w1.tensors["block_table"])
    rows = list(range(cfg.rows))
    ref0 = oracle_rows(w0, rows)
    a = run_fused(w0)
    compare_rows(w0, a, rows, ref0)
    p1 = problem_for(w1)
    t1 = tensors_for(w1)
    out1 = torch.empty_like(a["out"])
    ws = torch.empty((msa.msa_workspace_bytes(p1),), dtype=torch.uint8, device=DEV)
    msa.msa_sparse_decode(p1, t1, a["page_table"], out1, ws)
    torch.cuda.synchronize()
    ref1 = oracle_attention_rows(w1, rows, {r: ref0[r]["selected"] for r in rows})
    got = out1.cpu().numpy().astype(np.float64)
    err = max(float(np.max(np.abs(got[r] - ref1[r]))) for r in rows)
    assert err <= TOL[cfg.kv_dtype], err
    # reuse is a real change of work: layer 1 would have selected differently
    own = oracle_rows(w1, rows)
    assert any(not np.array_equal(own[r]["selected"], ref0[r]["selected"]) for r in rows)
    _say(f"  reuse max abs err {err:.3g}")


def test_workspace_too_small_is_rejected():
    cfg = small_config(batch=2, ctx_lo=3000, ctx_hi=5000, seed=15)
    w = make_workload(cfg, DEV)
    p = problem_for(w)
    t = tensors_for(w)
    need = msa.msa_workspace_bytes(p)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.rows, cfg.num_q_heads, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(msa.MSAError) as ei:
        msa.msa_decode(p, t, None, None, out, ws)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE


@pytest.mark.parametrize("kw,union", [
    (dict(batch=3, query_len=4, ctx_lo=3000, ctx_hi=12000, kv_dtype="fp8", idx_dtype="fp8",
          seed=51), True),
    (dict(batch=2, query_len=2, ctx_lo=2100, ctx_hi=9000, num_q_heads=16, num_kv_heads=1,
          num_idx_heads=2, seed=52), True),
    (dict(batch=3, query_len=3, ctx_lo=3, ctx_hi=6000, num_q_heads=20, num_kv_heads=2,
          kv_dtype="nvfp4", idx_dtype="fp8", seed=53), True),
    (dict(batch=2, query_len=4, ctx_list=(4, 2051), num_q_heads=4, num_kv_heads=1, topk=3,
          seed=54), True),
    (dict(batch=2, query_len=3, ctx_lo=3000, ctx_hi=9000, num_q_heads=16, num_kv_heads=1,
          seed=55), False),
    (dict(batch=2, query_len=5, ctx_lo=3000, ctx_hi=9000, kv_dtype="fp8", idx_dtype="fp8",
          seed=56), False),
    # rows of more than 1,024 blocks: the in-attention selection of the
    # union workgroup reads its candidates past the first batch
    (dict(batch=2, query_len=3, ctx_lo=140000, ctx_hi=200000, seed=57), True),
    (dict(batch=2, query_len=4, ctx_lo=130000, ctx_hi=170000, kv_dtype="fp8", idx_dtype="fp8",
          n_plant=4, seed=58), True),
    # fp8 (raw-V slots) with two KV heads: a ragged second tile (18 columns)
    # and a single tile (10 columns)
    (dict(batch=3, query_len=3, ctx_lo=5000, ctx_hi=15000, num_q_heads=12, num_kv_heads=2,
          kv_dtype="fp8", idx_dtype="fp8", seed=59), True),
    (dict(batch=4, query_len=2, ctx_lo=1, ctx_hi=7000, num_q_heads=10, num_kv_heads=2,
          kv_dtype="fp8", idx_dtype="bf16", seed=60), True),
], ids=["T4G8-fp8", "T2G16", "T3G10-nvfp4", "T4G4-topk3", "T3G16-rows", "T5G8-rows",
        "T3G8-long", "T4G8-fp8-long", "T3G6-fp8-2kv", "T2G5-fp8-2kv"])
def test_multi_row_union_attention(kw, union):
    """Multi-row requests whose (row, query head) pairs fit two 16-column
    tiles (T <= 4) walk the union of their rows' blocks in one workgroup;
    the others keep one workgroup per row.  Both match the oracle."""
    cfg = small_config(**kw)
    _say(f"multi-row attention {kw}")
    w = make_workload(cfg, DEV)
    rows = list(range(cfg.rows))
    got = run_stages(w)
    rec = msa.msa_last_dispatch()
    assert ("sparse_attn_union<" in rec) == union, rec
    err = compare_rows(w, got, rows)
    fused = run_fused(w)
    for k in ("selected", "page_table", "out"):
        assert torch.equal(fused[k], got[k]), f"fused {k} differs from stage-wise"
    _say(f"  max abs err {err:.3g} (tol {TOL[cfg.kv_dtype]})")


# --------------------------------------------------------- full workloads
@pytest.mark.parametrize("name", CONFIG_ORDER + EXTRA_CONFIGS)
def test_full_workload_parity(name):
    """Every row of every full-size workload against the oracle: block
    scores, selections, counts and page tables bit for bit, outputs within
    the tolerance (the 16-block / 2,048-key selection holds for every query,
    aisoku.org article, section "MSAの仕組み")."""
    cfg = CONFIGS[name]
    _say(f"full workload {name}: generating")
    w = make_workload(cfg, DEV)
    torch.cuda.synchronize()
    _say(f"full workload {name}: running fused path")
    got = run_fused(w)
    stages = run_stages(w)
    for k in ("selected", "page_table", "out"):
        assert torch.equal(got[k], stages[k]), f"{name}: fused {k} differs from stage-wise"
    got["scores"] = stages["scores"]
    got["n_selected"] = stages["n_selected"]
    del stages
    check_invariants(w, got)
    rows = list(range(cfg.rows))
    _say(f"full workload {name}: oracle on all {len(rows)} rows")
    err = compare_rows(w, got, rows)
    # planted blocks are kept for every row 0 of a request
    if cfg.n_plant and cfg.query_len == 1:
        sel = got["selected"].cpu().numpy()
        for b in range(cfg.batch):
            if len(w.planted[b]) <= cfg.topk - 1:
                assert set(w.planted[b]) <= set(sel[b].tolist()), f"request {b}"
            else:
                assert len(set(w.planted[b]) & set(sel[b].tolist())) == cfg.topk - 1
    _say(f"full workload {name}: {len(rows)} rows match, max abs err {err:.3g} "
         f"(tol {TOL[cfg.kv_dtype]})")
    del w, got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("maxb,fused", [(16384, True), (16385, False)])
def test_selection_inside_attention_up_to_16384_blocks(maxb, fused):
    """msa_decode selects inside the attention launch for single-row requests
    whose block table is at most 16384 blocks wide, and in a launch of its own
    beyond.  The table is widened (valid ids past the contexts) to either
    side of that edge; both must give the stage-wise entry points' results on
    the unwidened table bit for bit.  Two KV heads and split rows: every
    (KV head, split) workgroup of a row selects, one of them exports."""
    cfg = small_config(batch=3, query_len=1, ctx_lo=9000, ctx_hi=30000, num_q_heads=16,
                       num_kv_heads=2, num_idx_heads=2, n_plant=4, seed=31)
    print(f"fused-selection edge: table width {maxb}", flush=True)
    w = make_workload(cfg, DEV)
    ref = run_stages(w)
    t = w.tensors
    wide = torch.zeros((cfg.batch, maxb), dtype=torch.int32, device=DEV)
    wide[:, :t["block_table"].shape[1]] = t["block_table"]
    p, tt = msa.describe(t["q"], t["idx_q"], t["k_pool"], t["v_pool"], t["k_scale"],
                         t["v_scale"], t["idx_k_pool"], wide, t["ctx_lens"],
                         decode_query_len=1, topk=cfg.topk, idx_k_scale=t.get("idx_k_scale"))
    sel = torch.empty_like(ref["selected"])
    pt = torch.empty_like(ref["page_table"])
    out = torch.empty_like(ref["out"])
    ws = torch.empty((msa.msa_workspace_bytes(p),), dtype=torch.uint8, device=DEV)
    msa.msa_decode(p, tt, sel, pt, out, ws)
    torch.cuda.synchronize()
    rec = msa.msa_last_dispatch()
    assert ("sparse_attn<bf16>+select_topk" in rec) == fused, rec
    assert (" select_topk[" in rec) != fused, rec
    assert torch.equal(sel, ref["selected"])
    assert torch.equal(pt, ref["page_table"])
    assert torch.equal(out, ref["out"])
    assert compare_rows(w, ref, list(range(cfg.rows))) <= TOL[cfg.kv_dtype]
