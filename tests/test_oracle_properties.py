"""Property tests of the oracle's selection and page table on generated
block scores (hypothesis, derandomised so a run is reproducible).

The selection rule (MSA pages: the query's own block always kept, the best
of the other blocks up to 16 in all, equal scores to the lower block id; NaN
read as -inf) is checked here against an independent statement of it: one
stable sort of the candidates by (-score, id).  Scores come from a small
pool with many exact ties, signed zeros, infinities and NaN, or from wide
floats; contexts are ragged and include rows whose whole context fits in
topk blocks.
"""
import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

POOL = [-math.inf, -2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0, math.inf, math.nan]


def sort_select(scores, local, topk):
    """Ascending kept ids of one row: all blocks up to the local one when
    they fit, else the local block and the topk - 1 first candidates of a
    sort by (-score, id) with NaN as -inf."""
    if local + 1 <= topk:
        return list(range(local + 1))
    key = [(-(-math.inf if math.isnan(s) else s), c) for c, s in enumerate(scores[:local])]
    return sorted([c for _, c in sorted(key)[:topk - 1]] + [local])


@st.composite
def problems(draw):
    B = draw(st.integers(1, 3))
    T = draw(st.integers(1, 4))
    topk = draw(st.integers(1, 16))
    MAXB = draw(st.integers(1, 40))
    ctx = [draw(st.integers(T, MAXB * 128)) for _ in range(B)]
    values = st.sampled_from(POOL) if draw(st.booleans()) else \
        st.floats(allow_nan=True, allow_infinity=True, width=32)
    scores = np.array([[draw(values) for _ in range(MAXB)] for _ in range(B * T)],
                      dtype=np.float64)
    return B, T, topk, MAXB, np.array(ctx, dtype=np.int32), scores


@settings(max_examples=300, deadline=None, derandomize=True)
@given(problems())
def test_selection_equals_a_sort_by_score_then_id(case):
    B, T, topk, MAXB, ctx, scores = case
    prob = oracle.OracleProblem(B, T, 8, 1, 1, MAXB, "bf16", "bf16", topk=topk)
    sel, nsel = oracle.select(prob, scores, ctx)
    for r in range(B * T):
        b, t = divmod(r, T)
        pos = int(ctx[b]) - T + t
        local = pos // 128
        want = sort_select(list(scores[r]), local, topk)
        assert nsel[r] == len(want) == min(topk, local + 1)
        assert list(sel[r, :nsel[r]]) == want, (r, local, scores[r, :local + 1])
        assert (sel[r, nsel[r]:] == -1).all()


@settings(max_examples=100, deadline=None, derandomize=True)
@given(problems(), st.integers(0, 10**6))
def test_page_table_expands_each_kept_block(case, seed):
    B, T, topk, MAXB, ctx, scores = case
    prob = oracle.OracleProblem(B, T, 8, 1, 1, MAXB, "bf16", "bf16", topk=topk)
    sel, nsel = oracle.select(prob, scores, ctx)
    table = np.random.default_rng(seed).permutation(B * MAXB).reshape(B, MAXB).astype(np.int32)
    pt = oracle.page_table(prob, sel, table)
    assert pt.shape == (B * T, topk * 8)
    for r in range(B * T):
        n = nsel[r]
        for k in range(topk):
            group = pt[r, 8 * k:8 * k + 8]
            if k < n:
                phys = table[r // T, sel[r, k]]
                assert list(group) == [8 * phys + j for j in range(8)]
            else:
                assert (group == -1).all()
