"""Selection on crafted block scores: msa_select_blocks against the oracle.

The scores are inputs of the selection entry point, so these tests drive it
with score patterns the index scan would rarely produce: heavy ties, equal
scores, -0 / +0, NaN and infinities, and layouts that defeat the threshold
fast path (a few lanes holding most of the best keys), which sends a row to
the list path.  Rows cover take-all contexts (local block < topk), moderate
and long contexts (past the candidates a lane keeps in registers), and 1 to
5 rows per request (1, 2 or 4 waves per row).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_10_amd as msa
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def parts_for(T, MAXB):
    """Waves per row: 8 for single-row requests of 2048 blocks or more, else 4
    / T (1 from 3 rows on), as the selection kernel splits a row."""
    if T == 1:
        return 8 if MAXB >= 2048 else 4
    return 2 if T == 2 else 1


def lane_of(c, T, MAXB):
    """(wave part, lane) that reads candidate c for T rows per request."""
    stride = parts_for(T, MAXB) * 64
    return (c % stride) // 64, c % 64


def make_scores(pattern, R, MAXB, T, rng):
    c = np.arange(MAXB)
    if pattern == "iid":
        s = rng.standard_normal((R, MAXB))
    elif pattern == "integer_ties":
        s = rng.integers(-3, 4, (R, MAXB)).astype(np.float64)
    elif pattern == "equal":
        s = np.zeros((R, MAXB))
        s[:, ::3] = -0.0
    elif pattern == "special":
        s = rng.standard_normal((R, MAXB))
        pick = rng.random((R, MAXB))
        s[pick < 0.02] = np.nan
        s[(pick >= 0.02) & (pick < 0.04)] = -np.inf
        s[(pick >= 0.04) & (pick < 0.045)] = np.inf
    elif pattern == "descending":
        s = np.tile(-c.astype(np.float64), (R, 1))
    elif pattern == "lane_clustered":
        # lanes 0..14 of the first wave hold every key above the rest, each
        # lane's keys above the previous lane's: the wave bound is lane 0's
        # maximum and almost all of lanes 1..14's keys reach it
        part, lane = lane_of(c, T, MAXB)
        s = rng.standard_normal((R, MAXB))
        hot = (part == 0) & (lane < 15)
        s[:, hot] = 1000.0 + 100.0 * lane[hot] + (c[hot] // 256) % 32
    else:
        raise ValueError(pattern)
    return s.astype(np.float32)


CASES = [
    # (T, topk, context lengths in tokens; a row's candidates are its blocks
    # before the local one, about L / 128).  A lane keeps two batches of 16
    # candidates in registers: 8192 blocks at T = 1, 4096 at T = 2 and 2048
    # at T >= 3; the longer rows here read past them.
    (1, 16, (700, 2100, 9000, 131072)),
    (1, 16, (1500, 1_100_000, 1_250_000)),
    (2, 16, (3000, 40000, 600_000)),
    (3, 16, (2048, 2049, 300_000)),
    (4, 16, (8192, 16384, 300_000)),
    (5, 16, (5000, 280_000)),
    (1, 8, (9000, 1_100_000)),
    (4, 2, (5000, 9000)),
    (2, 1, (3000, 6000)),
]
PATTERNS = ["iid", "integer_ties", "equal", "special", "descending", "lane_clustered"]


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_selection_matches_oracle_on_crafted_scores(case, pattern):
    T, topk, ctx = CASES[case]
    B = len(ctx)
    MAXB = -(-max(ctx) // 128)
    R = B * T
    rng = np.random.default_rng(1000 + 17 * case + PATTERNS.index(pattern))
    scores = make_scores(pattern, R, MAXB, T, rng)
    ctx_lens = np.array(ctx, dtype=np.int32)

    p = msa.problem(B, T, 8, 1, 1, MAXB, 1, topk=topk)
    s_dev = torch.from_numpy(scores).to(DEV)
    ctx_dev = torch.from_numpy(ctx_lens).to(DEV)
    sel = torch.full((R, topk), 7, dtype=torch.int32, device=DEV)
    nsel = torch.full((R,), 7, dtype=torch.int32, device=DEV)
    msa.msa_select_blocks(p, s_dev, ctx_dev, sel, nsel)
    torch.cuda.synchronize()

    prob = oracle.OracleProblem(B, T, 8, 1, 1, MAXB, "bf16", "bf16", topk=topk)
    want_sel, want_n = oracle.select(prob, scores.astype(np.float64), ctx_lens)
    got_sel = sel.cpu().numpy()
    got_n = nsel.cpu().numpy()
    for r in range(R):
        assert got_n[r] == want_n[r], (r, got_n[r], want_n[r])
        assert np.array_equal(got_sel[r], want_sel[r]), (r, got_sel[r], want_sel[r])


def test_lane_clustered_rows_take_the_list_path_and_iid_rows_do_not():
    # The survivors of the threshold for one long single-row request (8
    # waves) and a two-row request (2 of the 4 waves per row): the clustered
    # layout leaves far more than a row
    # can rank by counting (128), iid scores a few dozen.  Counted here on
    # the host from the same rule the kernel applies.
    rng = np.random.default_rng(3)
    for (T, L), pattern, many in (((1, 1_100_000), "lane_clustered", True),
                                  ((1, 1_100_000), "iid", False),
                                  ((2, 600_000), "lane_clustered", True),
                                  ((2, 600_000), "iid", False)):
        MAXB = -(-L // 128)
        local = (L - 1) >> 7
        s = make_scores(pattern, 1, MAXB, T, rng)[0]
        keys = [(float(s[c]), -c) for c in range(local)]
        lanes = {}
        for c in range(local):
            part, lane = lane_of(c, T, MAXB)
            lanes.setdefault((part, lane), []).append(keys[c])
        # a wave's bound: the 15th largest score among its lane maxima (every
        # key of that score or above survives, whatever its id)
        bound = None
        for part in range(parts_for(T, MAXB)):
            maxima = sorted((max(v) for (pt, _), v in lanes.items() if pt == part), reverse=True)
            if len(maxima) >= 15:
                b = maxima[14][0]
                bound = b if bound is None or b > bound else bound
        survivors = sum(1 for k in keys if k[0] >= bound)
        assert (survivors > 128) == many, (pattern, survivors)
