"""msa_decode (and the write path before it) captured into a HIP graph.

A serving loop replays one captured decode step per token: the kernels take
all state from device buffers and the workspace needs no initialisation, so
the captured launches are replayable.  Each replay here follows eager work
on the same stream and a synchronisation, inputs change in place between
replays, and every replay is compared bit for bit with an eager call on the
same inputs.
"""
import pytest
import torch

import block_sparse_attention_10_amd as msa
from synth import make_workload, small_config

pytestmark = pytest.mark.gpu

DEV = "cuda"


def eager_decode(p, t, R, topk, Hq, ws_bytes):
    sel = torch.empty((R, topk), dtype=torch.int32, device=DEV)
    pt = torch.empty((R, topk * 8), dtype=torch.int32, device=DEV)
    out = torch.empty((R, Hq, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=DEV)
    msa.msa_decode(p, t, sel, pt, out, ws)
    torch.cuda.synchronize()
    return sel, pt, out


@pytest.mark.parametrize("kw", [
    dict(batch=3, query_len=1, ctx_lo=1500, ctx_hi=9000, seed=41),
    dict(batch=2, query_len=4, ctx_lo=3000, ctx_hi=20000, kv_dtype="fp8", idx_dtype="fp8",
         seed=42),
], ids=["bf16_T1_split", "fp8_T4"])
def test_captured_decode_replays_match_eager(kw):
    cfg = small_config(**kw)
    w = make_workload(cfg, DEV)
    t = w.tensors
    R = cfg.rows
    p, tt = msa.describe(t["q"], t["idx_q"], t["k_pool"], t["v_pool"], t["k_scale"],
                         t["v_scale"], t["idx_k_pool"], t["block_table"], t["ctx_lens"],
                         decode_query_len=cfg.query_len, topk=cfg.topk)
    nbytes = msa.msa_workspace_bytes(p)
    sel = torch.empty((R, cfg.topk), dtype=torch.int32, device=DEV)
    pt = torch.empty((R, cfg.topk * 8), dtype=torch.int32, device=DEV)
    out = torch.empty((R, cfg.num_q_heads, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=DEV)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        msa.msa_decode(p, tt, sel, pt, out, ws)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        msa.msa_decode(p, tt, sel, pt, out, ws)
    dispatch = msa.msa_last_dispatch()
    assert "index_scan" in dispatch and "sparse_attn" in dispatch

    q0 = t["q"].clone()
    iq0 = t["idx_q"].clone()
    g = torch.Generator(device="cpu").manual_seed(7)
    for step in range(4):
        if step >= 2:
            # the next token's queries, written in place
            t["q"].copy_(q0.flip(0) if step == 2 else q0.roll(1, dims=1))
            t["idx_q"].copy_(iq0 * (step - 1))
        # unrelated eager work on the same stream, then clear the outputs
        junk = torch.randn(1 << 16, generator=g).to(DEV)
        junk.mul_(2).add_(1)
        out.fill_(7.0)
        sel.fill_(-7)
        pt.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want_sel, want_pt, want_out = eager_decode(p, tt, R, cfg.topk, cfg.num_q_heads, nbytes)
        assert torch.equal(sel, want_sel), step
        assert torch.equal(pt, want_pt), step
        assert torch.equal(out, want_out), step
