"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: torch's own
format conversions, the OCP format tables, brute force on tiny inputs, dense
softmax attention (a library routine) in the cases where MSA reduces to it,
invariants the pages state (local block kept, 2,048-key cap, positive scale
invariance, KV read in place through a page view) and the page figures in
tests/golden/page_figures.json.
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, host_arrays, make_workload, small_config
from tests.refs import (E2M1_TABLE, brute_force_select, decode_bf16, decode_e4m3,
                        dense_attention, problem_of, token_scores)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def run_oracle(cfg, h, sm_scale=0.0, rows=None):
    P = problem_of(cfg, sm_scale)
    return oracle.decode(P, h["q"], h["idx_q"], h["k_pool"], h["v_pool"], h["k_scale"],
                         h["v_scale"], h["idx_k_pool"], h["block_table"], h["ctx_lens"], rows,
                         idx_k_scale=h.get("idx_k_scale"))


def positions(cfg, h):
    T = cfg.query_len
    for b in range(cfg.batch):
        L = int(h["ctx_lens"][b])
        for t in range(T):
            yield b, t, b * T + t, L - T + t


# ------------------------------------------------------------------ formats
def test_bf16_decoder_matches_torch_on_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    ref = decode_bf16(codes)
    got = np.array([oracle.bf16_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = decode_e4m3(codes)
    got = np.array([oracle.e4m3_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9  # smallest subnormal


def test_e2m1_decoder_matches_ocp_table():
    got = [oracle.e2m1_to_double(c) for c in range(16)]
    assert got == E2M1_TABLE
    assert [math.copysign(1, g) for g in got] == [math.copysign(1, g) for g in E2M1_TABLE]


# ------------------------------------------------------------ block scores
@pytest.mark.parametrize("kw", [
    dict(),
    dict(query_len=3, num_idx_heads=3, ctx_lo=300, ctx_hi=1100, batch=3),
    dict(idx_dtype="fp8", num_idx_heads=2, ctx_lo=129, ctx_hi=700, batch=3, query_len=2),
    dict(ctx_list=(1, 127, 128, 129), batch=4, query_len=1),
    dict(idx_dtype="nvfp4", num_idx_heads=2, ctx_lo=129, ctx_hi=900, batch=3, query_len=2,
         n_plant=2),
])
def test_block_scores_brute_force(kw):
    cfg = small_config(**kw)
    w = make_workload(cfg)
    h = host_arrays(w)
    s = oracle.index_scores(problem_of(cfg), h["idx_q"], h["idx_k_pool"], h["block_table"],
                            h["ctx_lens"], idx_k_scale=h["idx_k_scale"])
    for b, t, r, p in positions(cfg, h):
        ts = token_scores(cfg, h, b, t)
        local = p // 128
        for c in range(cfg.max_blocks):
            if c > local:
                assert s[r, c] == -np.inf
            else:
                assert s[r, c] == ts[c * 128:min(c * 128 + 128, p + 1)].max()


def test_block_score_sums_heads_before_max():
    """Two index heads whose per-head maxima sit on different tokens: the
    block score is the max of the head sum, not the sum of head maxima."""
    cfg = small_config(batch=1, ctx_list=(128,), num_idx_heads=2)
    w = make_workload(cfg)
    h = host_arrays(w)
    ik = np.zeros_like(h["idx_k_pool"])
    one = np.uint16(0x3F80)  # bf16 1.0
    ik[0, 0, 5, :] = one     # head 0 likes token 5
    ik[0, 1, 9, :] = one     # head 1 likes token 9
    iq = np.full_like(h["idx_q"], one)
    h["idx_k_pool"], h["idx_q"] = ik, iq
    s = oracle.index_scores(problem_of(cfg), h["idx_q"], h["idx_k_pool"], h["block_table"],
                            h["ctx_lens"])
    assert s[0, 0] == 64.0  # not 128


def test_fp4_index_key_closed_form():
    """4-bit index keys: E2M1 code 0x2 (1.0) times E4M3 scale 0x40 (2.0) in
    every dim, a query of ones: each token scores 64 * 2 per head; one dim
    recoded to -6 (0xF) under scale 8 (0x50) drops a token by 2 + 48."""
    cfg = small_config(batch=1, ctx_list=(128,), num_idx_heads=2, idx_dtype="nvfp4")
    w = make_workload(cfg)
    h = host_arrays(w)
    ik = np.full_like(h["idx_k_pool"], 0x22)      # two 1.0 codes per byte
    sc = np.full_like(h["idx_k_scale"], 0x40)     # 2.0
    iq = np.full_like(h["idx_q"], np.uint16(0x3F80))
    s = oracle.index_scores(problem_of(cfg), iq, ik, h["block_table"], h["ctx_lens"],
                            idx_k_scale=sc)
    assert s[0, 0] == 2 * 64 * 2.0
    phys = int(h["block_table"][0, 0])
    ik[phys, :, :, 0] = 0xF2    # dim 1 of every token and head: -6
    sc[phys, :, :, 0] = 0x50    # dims 0..15 scaled by 8
    s = oracle.index_scores(problem_of(cfg), iq, ik, h["block_table"], h["ctx_lens"],
                            idx_k_scale=sc)
    # per head: 15 dims of 1 * 8, one of -6 * 8, 48 dims of 1 * 2
    assert s[0, 0] == 2 * (15 * 8 - 48 + 48 * 2)
    with pytest.raises(ValueError):
        oracle.index_scores(problem_of(cfg), iq, ik, h["block_table"], h["ctx_lens"])


def test_fp4_index_keys_select_planted_blocks():
    cfg = small_config(batch=3, ctx_lo=6000, ctx_hi=9000, num_idx_heads=2, idx_dtype="nvfp4",
                       n_plant=6, seed=31)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b in range(cfg.batch):
        sel = set(int(x) for x in res["selected"][b] if x >= 0)
        assert set(w.planted[b]) <= sel, (b, w.planted[b], sel)


# --------------------------------------------------------------- selection
@pytest.mark.parametrize("topk", [16, 5, 1])
@pytest.mark.parametrize("seed", [3, 11])
def test_selection_brute_force_and_properties(topk, seed):
    cfg = small_config(batch=3, query_len=2, ctx_lo=1000, ctx_hi=4000, topk=topk, seed=seed,
                       num_idx_heads=2)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b, t, r, p in positions(cfg, h):
        ts = token_scores(cfg, h, b, t)
        local = p // 128
        blk = [ts[c * 128:min(c * 128 + 128, p + 1)].max() for c in range(local + 1)]
        want = brute_force_select(blk, local, topk)
        sel = res["selected"][r]
        n = res["n_selected"][r]
        assert n == min(topk, local + 1) == len(want)
        assert list(sel[:n]) == want
        assert all(sel[n:] == -1)
        assert local in list(sel[:n])                       # local block always kept
        assert list(sel[:n]) == sorted(sel[:n])             # ascending
        chosen = set(sel[:n]) - {local}
        rest = set(range(local)) - chosen
        for c in chosen:                                    # every pick beats every miss
            for d in rest:
                assert (blk[c], -c) > (blk[d], -d)


def test_selection_invariant_under_positive_score_scale():
    """Scaling every score by the same positive constant keeps the top-k
    (news.ainew.jp MI355X article, section 2): scale the index queries by 2
    and 3 (exact in bf16 for integers up to 24)."""
    cfg = small_config(batch=4, query_len=2, ctx_lo=2500, ctx_hi=6000, num_idx_heads=2, seed=5)
    w = make_workload(cfg)
    h = host_arrays(w)
    base = run_oracle(cfg, h)
    iqf = decode_bf16(h["idx_q"])
    for k in (2.0, 3.0):
        h2 = dict(h)
        h2["idx_q"] = torch.from_numpy(iqf * k).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)
        res = run_oracle(cfg, h2)
        assert np.array_equal(res["selected"], base["selected"])
        fin = np.isfinite(base["scores"])
        assert np.array_equal(res["scores"][fin], k * base["scores"][fin])


@pytest.mark.parametrize("copy_to,want", [(3, [1, 5]), (0, [0, 5])])
def test_selection_ties_go_to_lower_block(copy_to, want):
    cfg = small_config(batch=1, ctx_list=(6 * 128,), topk=2, permute=True, seed=9)
    w = make_workload(cfg)
    h = host_arrays(w)
    ik = decode_bf16(h["idx_k_pool"]).copy()
    bt = h["block_table"][0]
    iq = decode_bf16(h["idx_q"][0])
    ik[bt[1]] += 4 * np.sign(iq)[:, None, :]                # block 1 becomes the best
    ik[bt[copy_to]] = ik[bt[1]]                              # an exact tie
    h["idx_k_pool"] = torch.from_numpy(ik).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)
    res = run_oracle(cfg, h)
    s = res["scores"][0]
    assert s[1] == s[copy_to] == s[:5].max()
    assert list(res["selected"][0]) == want


@pytest.mark.parametrize("name", ["tiny_4k"])
def test_planted_blocks_recovered(name):
    cfg = CONFIGS[name]
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b in range(cfg.batch):
        check_planted(res["scores"][b], res["selected"][b], w.planted[b],
                      (w.ctx_lens[b] - 1) // 128)


def check_planted(scores, sel, planted, local):
    """Planted blocks outrank every unplanted non-local block and are all
    kept, beside the forced local block; the other slots hold the best of the
    rest."""
    sel = list(sel)
    assert local in sel and set(planted) <= set(sel)
    others = [c for c in range(local) if c not in planted]
    assert min(scores[c] for c in planted) > max(scores[c] for c in others)
    fill = sorted(others, key=lambda c: (-scores[c], c))[:len(sel) - 1 - len(planted)]
    assert sorted(sel) == sorted(planted + fill + [local])


def test_planted_blocks_recovered_multihead_permuted():
    cfg = small_config(batch=3, ctx_lo=20000, ctx_hi=40000, num_idx_heads=4, num_q_heads=16,
                       num_kv_heads=2, n_plant=8, seed=21)
    w = make_workload(cfg)
    h = host_arrays(w)
    P = problem_of(cfg)
    s = oracle.index_scores(P, h["idx_q"], h["idx_k_pool"], h["block_table"], h["ctx_lens"])
    sel, _ = oracle.select(P, s, h["ctx_lens"])
    for b in range(cfg.batch):
        check_planted(s[b], sel[b], w.planted[b], (w.ctx_lens[b] - 1) // 128)


def test_planted_overflow_drops_weakest():
    """16 planted non-local blocks compete for 15 free slots: exactly 15 are
    kept and the forced local block takes the 16th place."""
    cfg = small_config(batch=2, ctx_lo=30000, ctx_hi=30000, n_plant=16, seed=4)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b in range(cfg.batch):
        local = (w.ctx_lens[b] - 1) // 128
        sel = list(res["selected"][b])
        assert local in sel
        picked = set(sel) - {local}
        assert len(picked) == 15 and picked <= set(w.planted[b])


def test_key_cap():
    """At most 16 x 128 = 2,048 keys per query; with a long context exactly
    15 full blocks plus the causal part of the local block."""
    gold = json.load(open(GOLDEN))
    cap = gold["blocks_kept"]["value"] * gold["block_tokens"]["value"]
    assert cap == gold["max_keys_per_query"]["value"]
    cfg = small_config(batch=4, query_len=3, ctx_lo=2100, ctx_hi=9000, seed=13)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b, t, r, p in positions(cfg, h):
        sel = res["selected"][r][:res["n_selected"][r]]
        keys = sum(min(128, p + 1 - c * 128) for c in sel)
        assert keys <= cap
        if p // 128 >= 16:
            assert keys == 15 * 128 + (p % 128) + 1


# -------------------------------------------------------------- page table
def test_page_table_closed_form():
    cfg = small_config(batch=3, query_len=2, ctx_lo=200, ctx_hi=5000, seed=17)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b, t, r, p in positions(cfg, h):
        sel = res["selected"][r]
        pt = res["page_table"][r]
        n = res["n_selected"][r]
        for k in range(cfg.topk):
            for j in range(8):
                want = h["block_table"][b][sel[k]] * 8 + j if k < n else -1
                assert pt[8 * k + j] == want


@pytest.mark.parametrize("kv", ["bf16", "fp8", "nvfp4"])
def test_outputs_invariant_under_physical_permutation(kv):
    """The page table is a view over KV that stays in place: moving physical
    blocks and rewriting the block table changes nothing else."""
    cfg = small_config(batch=3, query_len=2, ctx_lo=2000, ctx_hi=4500, kv_dtype=kv,
                       num_q_heads=8, num_kv_heads=2, permute=False, seed=23)
    w = make_workload(cfg)
    h = host_arrays(w)
    base = run_oracle(cfg, h)
    NB = w.num_phys_blocks
    pi = np.random.default_rng(0).permutation(NB)
    h2 = dict(h)
    for key in ("idx_k_pool", "k_pool", "v_pool", "k_scale", "v_scale"):
        if h[key] is None:
            continue
        moved = np.empty_like(h[key])
        moved[pi] = h[key]
        h2[key] = moved
    bt = h["block_table"].copy()
    for b in range(cfg.batch):
        bt[b, :w.nblk[b]] = pi[bt[b, :w.nblk[b]]]
    h2["block_table"] = bt
    res = run_oracle(cfg, h2)
    assert np.array_equal(res["selected"], base["selected"])
    assert np.array_equal(res["scores"], base["scores"])
    assert np.array_equal(res["out"], base["out"])
    mapped = np.where(base["page_table"] >= 0,
                      pi[np.maximum(base["page_table"], 0) // 8] * 8 + base["page_table"] % 8, -1)
    assert np.array_equal(res["page_table"], mapped)


# --------------------------------------------------------------- attention
@pytest.mark.parametrize("kw", [
    dict(ctx_list=(1, 77, 128, 129, 2048), batch=5, query_len=1),
    dict(ctx_list=(3, 700, 2048), batch=3, query_len=3, num_q_heads=16, num_kv_heads=2),
    dict(ctx_list=(1000, 2048), batch=2, kv_dtype="fp8", query_len=2),
    dict(ctx_list=(300, 1999), batch=2, kv_dtype="nvfp4", num_q_heads=4, num_kv_heads=4),
])
def test_dense_equality_up_to_2048_keys(kw):
    """With at most 16 causal blocks every block is kept, so MSA equals dense
    causal attention (softmax in float64 torch)."""
    cfg = small_config(**kw)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b, t, r, p in positions(cfg, h):
        ref = dense_attention(cfg, h, b, t)
        assert np.max(np.abs(res["out"][r] - ref)) < 1e-12


@pytest.mark.parametrize("kw", [
    dict(batch=3, query_len=2, ctx_lo=2500, ctx_hi=6000, num_q_heads=16, num_kv_heads=2),
    dict(batch=2, query_len=1, ctx_lo=3000, ctx_hi=5000, topk=5, kv_dtype="fp8"),
    dict(batch=2, query_len=3, ctx_lo=2200, ctx_hi=4000, kv_dtype="nvfp4", idx_dtype="fp8",
         num_idx_heads=2),
])
def test_masked_dense_brute_force(kw):
    """Oracle output equals dense softmax attention restricted, by an explicit
    mask, to the brute-force selection."""
    cfg = small_config(seed=31, **kw)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h)
    for b, t, r, p in positions(cfg, h):
        ts = token_scores(cfg, h, b, t)
        local = p // 128
        blk = [ts[c * 128:min(c * 128 + 128, p + 1)].max() for c in range(local + 1)]
        sel = brute_force_select(blk, local, cfg.topk)
        ref = dense_attention(cfg, h, b, t, allowed_blocks=sel)
        assert np.max(np.abs(res["out"][r] - ref)) < 1e-12


def test_custom_softmax_scale():
    cfg = small_config(ctx_list=(900,), batch=1)
    w = make_workload(cfg)
    h = host_arrays(w)
    res = run_oracle(cfg, h, sm_scale=0.3)
    ref = dense_attention(cfg, h, 0, 0, sm_scale=0.3)
    assert np.max(np.abs(res["out"][0] - ref)) < 1e-12


def test_unselected_blocks_do_not_matter():
    cfg = small_config(batch=2, ctx_lo=4000, ctx_hi=6000, seed=41)
    w = make_workload(cfg)
    h = host_arrays(w)
    base = run_oracle(cfg, h)
    h2 = dict(h)
    k = h["k_pool"].copy()
    v = h["v_pool"].copy()
    for b in range(cfg.batch):
        sel = set(base["selected"][b][:base["n_selected"][b]])
        for c in range(w.nblk[b]):
            if c not in sel:
                k[h["block_table"][b][c]] ^= np.uint16(0x1234)
                v[h["block_table"][b][c]] ^= np.uint16(0x0F0F)
    h2["k_pool"], h2["v_pool"] = k, v
    res = run_oracle(cfg, h2)
    assert np.array_equal(res["out"], base["out"])


def test_row_subset_matches_full_run():
    cfg = small_config(batch=3, query_len=2, ctx_lo=1800, ctx_hi=4000, seed=43)
    w = make_workload(cfg)
    h = host_arrays(w)
    full = run_oracle(cfg, h)
    rows = np.array([5, 0, 3], dtype=np.int32)
    part = run_oracle(cfg, h, rows=rows)
    for key in ("scores", "selected", "n_selected", "page_table", "out"):
        assert np.array_equal(part[key], full[key][rows])


# ------------------------------------------------------------ page figures
def test_kv_bytes_per_token_match_page_figures():
    """The storage layouts reproduce the byte counts the pages print: 61,440
    bytes per token for fp8 K+V codes and 34,560 for the 4-bit layout (codes
    plus one e4m3 scale per 16 elements), over 60 layers of 4 KV heads."""
    gold = json.load(open(GOLDEN))
    layers = gold["model_layers"]["value"]
    hkv = gold["heads_q_kv_idx"]["value"][1]
    per_head = {}
    for kv in ("fp8", "nvfp4"):
        cfg = small_config(batch=1, ctx_list=(128,), kv_dtype=kv, num_kv_heads=1,
                           num_q_heads=1)
        t = make_workload(cfg).tensors
        tok = t["k_pool"][0, 0, 0]
        nbytes = tok.numel() * tok.element_size()
        if kv == "nvfp4":
            sc = t["k_scale"][0, 0, 0]
            nbytes += sc.numel() * sc.element_size()
        per_head[kv] = 2 * nbytes  # K and V
    assert per_head["fp8"] * hkv * layers == gold["kv_bytes_per_token_fp8"]["value"]
    assert per_head["nvfp4"] * hkv * layers == gold["kv_bytes_per_token_nvfp4"]["value"]
    assert 1 - per_head["nvfp4"] / per_head["fp8"] == pytest.approx(0.4375)


def test_config_shapes_follow_page_heads():
    gold = json.load(open(GOLDEN))
    full = CONFIGS["layer_128k"]
    rank = CONFIGS["tp8_rank_32k"]
    assert [full.num_q_heads, full.num_kv_heads, full.num_idx_heads] == \
        gold["heads_q_kv_idx"]["value"]
    assert [rank.num_q_heads, rank.num_kv_heads, rank.num_idx_heads] == \
        gold["tp8_rank_heads_q_kv_idx"]["value"]


# -------------------------------------------------------------- write path
def _f32(v):
    return np.float32(v)


def _e4m3_probe_values():
    """Every E4M3 value, the midpoints between neighbours (exact ties), one
    fp32 ulp either side of each midpoint, and random values over the whole
    exponent range, both signs (magnitudes <= 448)."""
    vals = decode_e4m3(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)  # 0 .. 448
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    down = np.nextafter(mids, np.float32(-np.inf))
    rng = np.random.default_rng(5)
    rnd = (rng.standard_normal(4000) * np.exp2(rng.integers(-12, 8, 4000))).astype(np.float32)
    rnd = np.clip(rnd, -448, 448)
    pos = np.concatenate([vals, mids, up, down, np.abs(rnd), [1e-30, 2.0 ** -10]])
    return np.concatenate([pos, -pos]).astype(np.float32)


def test_e4m3_encoder_matches_torch_rounding():
    x = _e4m3_probe_values()
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]
    assert oracle.f32_to_e4m3(1000.0) == 0x7E and oracle.f32_to_e4m3(-1000.0) == 0xFE


def test_e2m1_encoder_is_nearest_even_on_the_grid():
    grid = np.array(E2M1_TABLE[:8])
    mids = (grid[:-1] + grid[1:]) / 2
    pts = np.concatenate([grid, mids, np.nextafter(mids, 10), np.nextafter(mids, -10),
                          np.linspace(0, 8, 801)]).astype(np.float32)
    pts = np.concatenate([pts, -pts])
    for v in pts:
        a = abs(float(v))
        d = np.abs(grid - min(a, 6.0))
        best = np.flatnonzero(d == d.min())
        m = int(best[0] if len(best) == 1 else best[best % 2 == 0][0])  # tie: even code
        want = m | (8 if v < 0 and m > 0 else 0)
        assert oracle.f32_to_e2m1(float(v)) == want, (float(v), want)
    # and the generator's (independent, torch) encoder agrees
    from synth import encode_e2m1
    t = torch.from_numpy(pts)
    assert np.array_equal(encode_e2m1(t).numpy(),
                          np.array([oracle.f32_to_e2m1(float(v)) for v in pts], dtype=np.uint8))


def _insert_case(kv_dtype, idx_dtype, seed=41, T=2):
    cfg = small_config(batch=3, query_len=T, ctx_lo=200, ctx_hi=900, kv_dtype=kv_dtype,
                       idx_dtype=idx_dtype, num_q_heads=8, num_kv_heads=2, num_idx_heads=2,
                       seed=seed)
    w = make_workload(cfg)
    h = host_arrays(w)
    rng = np.random.default_rng(seed)
    R = cfg.rows
    new = {
        "k": torch.from_numpy(rng.standard_normal((R, 2, 128)).astype(np.float32) * 3),
        "v": torch.from_numpy(rng.standard_normal((R, 2, 128)).astype(np.float32)),
        "i": torch.from_numpy(rng.integers(-8, 9, (R, 2, 64)).astype(np.float32)),
    }
    bits = {k: v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for k, v in new.items()}
    pools = {k: (None if h[k] is None else h[k].copy())
             for k in ("k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool", "idx_k_scale")}
    oracle.insert(problem_of(cfg), bits["k"], bits["v"], bits["i"], h["block_table"],
                  h["ctx_lens"], pools)
    return cfg, w, h, new, pools


def _slots(cfg, h):
    T = cfg.query_len
    for r in range(cfg.rows):
        b, t = divmod(r, T)
        p = int(h["ctx_lens"][b]) - T + t
        yield r, int(h["block_table"][b, p // 128]), p % 128


@pytest.mark.parametrize("kv,idx", [("bf16", "bf16"), ("fp8", "fp8"), ("nvfp4", "nvfp4")])
def test_insert_writes_the_generators_encoding_at_each_rows_slot(kv, idx):
    from synth import encode_fp8_per_token, encode_nvfp4
    cfg, w, h, new, pools = _insert_case(kv, idx)
    touched = {}
    for r, phys, slot in _slots(cfg, h):
        kf = new["k"][r].to(torch.bfloat16).float()
        vf = new["v"][r].to(torch.bfloat16).float()
        idf = new["i"][r].to(torch.bfloat16).float()
        for name, x in (("k", kf), ("v", vf)):
            got = pools[name + "_pool"][phys, :, slot]
            if kv == "bf16":
                assert np.array_equal(got, x.to(torch.bfloat16).view(torch.int16).numpy()
                                      .view(np.uint16))
            elif kv == "fp8":
                c, s = encode_fp8_per_token(x)
                assert np.array_equal(got, c.numpy())
                assert np.array_equal(pools[name + "_scale"][phys, :, slot], s.numpy())
            else:
                c, s = encode_nvfp4(x)
                assert np.array_equal(got, c.numpy())
                assert np.array_equal(pools[name + "_scale"][phys, :, slot], s.numpy())
        got = pools["idx_k_pool"][phys, :, slot]
        if idx == "bf16":
            assert np.array_equal(got, idf.to(torch.bfloat16).view(torch.int16).numpy()
                                  .view(np.uint16))
        elif idx == "fp8":
            assert np.array_equal(got, idf.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        else:
            c, s = encode_nvfp4(idf)
            assert np.array_equal(got, c.numpy())
            assert np.array_equal(pools["idx_k_scale"][phys, :, slot], s.numpy())
        touched.setdefault(phys, set()).add(slot)
    # every other slot is untouched
    for name in pools:
        if pools[name] is None:
            continue
        a, b0 = pools[name], h[name]
        for phys in range(a.shape[0]):
            for slot in range(128):
                if slot in touched.get(phys, ()):
                    continue
                assert np.array_equal(a[phys, :, slot], b0[phys, :, slot]), (name, phys, slot)


def test_decode_after_insert_attends_the_new_token():
    """A new key along the row's own query (scaled up) takes all the softmax
    weight of the row: the output becomes the new value, dequantised."""
    cfg = small_config(batch=2, query_len=1, ctx_lo=300, ctx_hi=800, num_q_heads=2,
                       num_kv_heads=1, num_idx_heads=1, seed=43)
    w = make_workload(cfg)
    h = host_arrays(w)
    q = decode_bf16(h["q"])                                  # [R, 2, 128]
    k_new = torch.from_numpy((q.sum(axis=1, keepdims=True) * 64).astype(np.float32))
    v_new = torch.from_numpy(np.random.default_rng(3).standard_normal((2, 1, 128))
                             .astype(np.float32))
    i_new = torch.zeros((2, 1, 64))
    bits = [x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for x in (k_new, v_new, i_new)]
    pools = {k: (None if h[k] is None else h[k].copy())
             for k in ("k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool", "idx_k_scale")}
    oracle.insert(problem_of(cfg), *bits, h["block_table"], h["ctx_lens"], pools)
    h2 = dict(h, **pools)
    res = run_oracle(cfg, h2)
    want = v_new.to(torch.bfloat16).double().numpy()[:, 0]   # [R, 128]
    for r in range(2):
        for hq in range(2):
            assert np.max(np.abs(res["out"][r, hq] - want[r])) < 1e-6
