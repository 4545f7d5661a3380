"""Debug checks of the data-dependent inputs (MSA_FLAG_DEBUG_CHECKS).

Every bad input here is chosen so that, even if a check missed it, the
kernels would stay inside allocated memory: the bad request is the middle one
of three (a context one past its table row reads the next row's first entry,
a negative position resolves inside the row before), and the pools carry one
spare block on each side, so table entries -1 and NB address real memory.
The attention clamps page ids to the pools by itself.
"""
import pytest
import torch

import block_sparse_attention_10_amd as msa
from synth import make_workload, small_config

pytestmark = pytest.mark.gpu

DEV = "cuda"
BAD = 1  # the request whose inputs are broken


def padded_workload(query_len=2, **kw):
    cfg = small_config(batch=3, query_len=query_len, ctx_lo=1500, ctx_hi=3000, seed=31, **kw)
    w = make_workload(cfg, DEV)
    keep = {}
    t = dict(w.tensors)
    for name in ("k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool", "idx_k_scale"):
        x = t.get(name)
        if x is None:
            continue
        full = torch.cat([x[:1], x, x[-1:]])  # blocks -1 and NB exist
        keep[name] = full
        t[name] = full[1:-1]
    return w, t, keep


def describe(w, t, ctx=None, table=None, flags=msa.MSA_FLAG_DEBUG_CHECKS):
    return msa.describe(t["q"], t["idx_q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"],
                        t["idx_k_pool"], t["block_table"] if table is None else table,
                        t["ctx_lens"] if ctx is None else ctx,
                        decode_query_len=w.cfg.query_len, topk=w.cfg.topk,
                        idx_k_scale=t.get("idx_k_scale"), flags=flags)


def outputs(w, p):
    c = w.cfg
    R = c.rows
    return dict(
        scores=torch.full((R, c.max_blocks), 7.0, device=DEV),
        selected=torch.full((R, c.topk), 7, dtype=torch.int32, device=DEV),
        n_selected=torch.full((R,), 7, dtype=torch.int32, device=DEV),
        page_table=torch.full((R, c.topk * 8), 7, dtype=torch.int32, device=DEV),
        out=torch.full((R, c.num_q_heads, 128), 7.0, device=DEV),
        workspace=torch.zeros((msa.msa_workspace_bytes(p),), dtype=torch.uint8, device=DEV),
    )


def expect_bad(call, *want):
    with pytest.raises(msa.MSAError) as e:
        call()
    assert e.value.status == msa.MSA_ERR_BAD_DATA
    msg = msa.msa_last_check_failure()
    for s in want:
        assert s in msg, (s, msg)
    return msg


def untouched(o, *names):
    for n in names:
        x = o[n]
        assert bool((x == 7).all()), f"{n} was written after a failed check"


# one row per request: msa_decode selects inside its attention launch; two:
# in a selection launch of its own
@pytest.mark.parametrize("T", [1, 2])
def test_valid_inputs_pass_and_give_the_same_results(T):
    w, t, keep = padded_workload(query_len=T)
    res = {}
    for flags in (0, msa.MSA_FLAG_DEBUG_CHECKS):
        p, tt = describe(w, t, flags=flags)
        o = outputs(w, p)
        msa.msa_index_score(p, tt, o["scores"])
        if flags:
            assert msa.msa_last_dispatch().startswith("input_checks[1x1024] index_scan")
        msa.msa_select_blocks(p, o["scores"], t["ctx_lens"], o["selected"], o["n_selected"])
        msa.msa_build_page_table(p, o["selected"], t["block_table"], o["page_table"])
        msa.msa_sparse_decode(p, tt, o["page_table"], o["out"], o["workspace"])
        fused = torch.empty_like(o["out"])
        msa.msa_decode(p, tt, None, None, fused, o["workspace"])
        torch.cuda.synchronize()
        res[flags] = (o, fused)
    (a, fa), (b, fb) = res[0], res[msa.MSA_FLAG_DEBUG_CHECKS]
    for n in ("scores", "selected", "n_selected", "page_table", "out"):
        assert torch.equal(a[n], b[n]), n
    assert torch.equal(fa, fb)
    assert torch.equal(a["out"], fa)


@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.parametrize("bad_len", ["short", "long"])
def test_bad_context_length_is_reported_before_any_launch(bad_len, T):
    w, t, keep = padded_workload(query_len=T)
    c = w.cfg
    ctx = t["ctx_lens"].clone()
    ctx[BAD] = c.query_len - 1 if bad_len == "short" else c.max_blocks * 128 + 1
    p, tt = describe(w, t, ctx=ctx)
    o = outputs(w, p)
    want = f"ctx_lens[{BAD}] = {int(ctx[BAD])}"
    expect_bad(lambda: msa.msa_index_score(p, tt, o["scores"]), want)
    expect_bad(lambda: msa.msa_select_blocks(p, o["scores"], ctx, o["selected"],
                                             o["n_selected"]), want)
    expect_bad(lambda: msa.msa_decode(p, tt, o["selected"], o["page_table"], o["out"],
                                      o["workspace"]), want)
    torch.cuda.synchronize()
    untouched(o, "scores", "selected", "n_selected", "page_table", "out")


@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.parametrize("value", ["minus_one", "nb"])
def test_bad_table_entry_inside_the_context_is_reported(value, T):
    w, t, keep = padded_workload(query_len=T)
    c = w.cfg
    L = int(t["ctx_lens"][BAD])
    col = (L - 1) // 128 // 2  # an older block of the context
    table = t["block_table"].clone()
    v = -1 if value == "minus_one" else w.num_phys_blocks
    table[BAD, col] = v
    p, tt = describe(w, t, table=table)
    o = outputs(w, p)
    want = f"block_table[{BAD}][{col}] = {v}"
    expect_bad(lambda: msa.msa_index_score(p, tt, o["scores"]), want)
    expect_bad(lambda: msa.msa_decode(p, tt, None, None, o["out"], o["workspace"]), want)
    torch.cuda.synchronize()
    untouched(o, "scores", "out")


@pytest.mark.parametrize("T", [1, 2])
def test_table_entries_past_the_context_are_not_checked(T):
    w, t, keep = padded_workload(query_len=T)
    c = w.cfg
    L = int(t["ctx_lens"][BAD])
    last = (L - 1) // 128
    assert last + 1 < c.max_blocks
    table = t["block_table"].clone()
    table[BAD, last + 1:] = w.num_phys_blocks  # never read: past the context
    p, tt = describe(w, t)
    p2, tt2 = describe(w, t, table=table)
    o, o2 = outputs(w, p), outputs(w, p2)
    msa.msa_decode(p, tt, o["selected"], o["page_table"], o["out"], o["workspace"])
    msa.msa_decode(p2, tt2, o2["selected"], o2["page_table"], o2["out"], o2["workspace"])
    torch.cuda.synchronize()
    for n in ("selected", "page_table", "out"):
        assert torch.equal(o[n], o2[n]), n


@pytest.mark.parametrize("case", ["past_table", "negative", "bad_entry"])
def test_bad_selection_for_the_page_table_is_reported(case):
    w, t, keep = padded_workload()
    c = w.cfg
    p, tt = describe(w, t)
    o = outputs(w, p)
    msa.msa_decode(p, tt, o["selected"], o["page_table"], o["out"], o["workspace"])
    torch.cuda.synchronize()
    sel = o["selected"].clone()
    table = t["block_table"]
    r = BAD * c.query_len
    if case == "past_table":
        sel[r, 0] = c.max_blocks
        want = f"selected[{r}][0] = {c.max_blocks}: neither -1"
    elif case == "negative":
        sel[r, 0] = -2
        want = f"selected[{r}][0] = -2: neither -1"
    else:
        table = table.clone()
        table[BAD, int(sel[r, 0])] = w.num_phys_blocks
        want = f"selected[{r}][0] = {int(sel[r, 0])} maps to block_table entry {w.num_phys_blocks}"
    pt = torch.full_like(o["page_table"], 7)
    expect_bad(lambda: msa.msa_build_page_table(p, sel, table, pt), want)
    torch.cuda.synchronize()
    assert bool((pt == 7).all())
    # the selection msa_decode exported passes
    msa.msa_build_page_table(p, o["selected"], t["block_table"], pt)
    torch.cuda.synchronize()
    assert torch.equal(pt, o["page_table"])


@pytest.mark.parametrize("case", ["page_past_pools", "not_consecutive", "block_after_padding",
                                  "no_block"])
def test_bad_page_table_is_reported(case):
    w, t, keep = padded_workload()
    c = w.cfg
    p, tt = describe(w, t)
    o = outputs(w, p)
    msa.msa_decode(p, tt, o["selected"], o["page_table"], o["out"], o["workspace"])
    torch.cuda.synchronize()
    pt = o["page_table"].clone()
    r = BAD * c.query_len
    n = int((pt[r] >= 0).sum()) // 8
    assert n >= 2
    if case == "page_past_pools":
        pt[r, 0:8] = torch.arange(8, dtype=torch.int32, device=DEV) + 8 * w.num_phys_blocks
        want = f"page_table[{r}][0..+7]"
    elif case == "not_consecutive":
        pt[r, 8 + 3] = pt[r, 8 + 4]
        want = f"page_table[{r}][8..+7]"
    elif case == "block_after_padding":
        pt[r, 0:8] = -1
        want = f"page_table[{r}][8..+7]"
    else:
        pt[r, :] = -1
        want = f"page_table[{r}][0..+7]"
    out = torch.full_like(o["out"], 7.0)
    msg = expect_bad(lambda: msa.msa_sparse_decode(p, tt, pt, out, o["workspace"]), want)
    assert msg
    torch.cuda.synchronize()
    assert bool((out == 7).all())
    # the exported table passes and reproduces msa_decode's output
    msa.msa_sparse_decode(p, tt, o["page_table"], out, o["workspace"])
    torch.cuda.synchronize()
    assert torch.equal(out, o["out"])


def test_insert_checks_only_the_new_tokens_blocks():
    w, t, keep = padded_workload()
    c = w.cfg
    R = c.rows
    g = torch.Generator(device="cpu").manual_seed(5)
    k_new = (torch.randint(-8, 9, (R, c.num_kv_heads, 128), generator=g)).to(DEV, torch.bfloat16)
    v_new = (torch.randint(-8, 9, (R, c.num_kv_heads, 128), generator=g)).to(DEV, torch.bfloat16)
    i_new = (torch.randint(-8, 9, (R, c.num_idx_heads, 64), generator=g)).to(DEV, torch.bfloat16)
    p, _ = describe(w, t)
    pools = msa.pools(t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["idx_k_pool"],
                      t.get("idx_k_scale"))
    L = int(t["ctx_lens"][BAD])
    new_col = (L - 1) // 128
    before = {n: keep[n].clone() for n in keep}
    # a bad entry in an older block is not read by the write path
    table = t["block_table"].clone()
    table[BAD, 0] = -1
    if new_col > 0:
        msa.msa_insert_kv(p, pools, table, t["ctx_lens"], k_new, v_new, i_new)
        torch.cuda.synchronize()
        assert msa.msa_last_dispatch().startswith("input_checks[1x1024] insert")
        for n in keep:
            keep[n].copy_(before[n])
    # a bad entry in the new token's block is reported and nothing is written
    table = t["block_table"].clone()
    table[BAD, new_col] = w.num_phys_blocks
    expect_bad(lambda: msa.msa_insert_kv(p, pools, table, t["ctx_lens"], k_new, v_new, i_new),
               f"block_table[{BAD}][{new_col}] = {w.num_phys_blocks}")
    torch.cuda.synchronize()
    for n in keep:
        assert torch.equal(keep[n], before[n]), n
