"""Helpers for the GPU tests: run the library through its C ABI on a
synthetic workload, and compute oracle results for any set of rows.

The oracle side only ever sees generator outputs (gathered on the device by
torch indexing and copied to the host) and its own selections; nothing the
GPU library produced feeds it.
"""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_10_amd as msa
import oracle
from synth import Workload
from tests.refs import problem_of

TOL = {"bf16": 2e-3, "fp8": 1e-2, "nvfp4": 1e-2}


def problem_for(w: Workload):
    return describe_workload(w)[0]


def tensors_for(w: Workload):
    return describe_workload(w)[1]


def describe_workload(w: Workload):
    t = w.tensors
    return msa.describe(t["q"], t["idx_q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"],
                        t["idx_k_pool"], t["block_table"], t["ctx_lens"],
                        decode_query_len=w.cfg.query_len, topk=w.cfg.topk,
                        idx_k_scale=t.get("idx_k_scale"))


def alloc_outputs(w: Workload, p):
    c = w.cfg
    dev = w.device
    R = c.rows
    return {
        "scores": torch.empty((R, c.max_blocks), dtype=torch.float32, device=dev),
        "selected": torch.empty((R, c.topk), dtype=torch.int32, device=dev),
        "n_selected": torch.empty((R,), dtype=torch.int32, device=dev),
        "page_table": torch.empty((R, c.topk * 8), dtype=torch.int32, device=dev),
        "out": torch.empty((R, c.num_q_heads, 128), dtype=torch.float32, device=dev),
        "workspace": torch.empty((msa.msa_workspace_bytes(p),), dtype=torch.uint8, device=dev),
    }


def run_stages(w: Workload, stream=None):
    """Each entry point on its own, chained through device buffers."""
    p = problem_for(w)
    t = tensors_for(w)
    o = alloc_outputs(w, p)
    msa.msa_index_score(p, t, o["scores"], stream)
    msa.msa_select_blocks(p, o["scores"], w.tensors["ctx_lens"], o["selected"], o["n_selected"],
                          stream)
    msa.msa_build_page_table(p, o["selected"], w.tensors["block_table"], o["page_table"], stream)
    msa.msa_sparse_decode(p, t, o["page_table"], o["out"], o["workspace"], stream)
    torch.cuda.synchronize()
    return o


def run_fused(w: Workload, stream=None, export=True):
    p = problem_for(w)
    t = tensors_for(w)
    o = alloc_outputs(w, p)
    sel = o["selected"] if export else None
    pt = o["page_table"] if export else None
    msa.msa_decode(p, t, sel, pt, o["out"], o["workspace"], stream)
    torch.cuda.synchronize()
    del o["scores"], o["n_selected"]  # internal to the fused call
    if not export:
        del o["selected"], o["page_table"]
    return o


def _host(x: torch.Tensor) -> np.ndarray:
    x = x.detach().to("cpu")
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def _compact(pool, phys):
    """Host copy of the blocks `phys` (int64 device tensor) of a pool."""
    return None if pool is None else _host(pool[phys])


def oracle_rows(w: Workload, rows):
    """Oracle results for the given rows, in one oracle call per step so that
    its OpenMP loops spread over all the rows.  The index keys of the rows'
    requests (every block of their contexts) and the K/V blocks the oracle
    selects are copied to compact host pools; the block tables are remapped
    to them, so the oracle never reads the rest of the device pools."""
    c = w.cfg
    T = c.query_len
    t = w.tensors
    rows = [int(r) for r in rows]
    reqs = sorted({r // T for r in rows})
    bt_host = _host(t["block_table"]).astype(np.int64)
    ctx = np.asarray(w.ctx_lens, dtype=np.int32)
    prob = problem_of(c)
    rows_np = np.asarray(rows, dtype=np.int32)

    # compact index-key pool: the context blocks of the rows' requests
    phys_list, bt_idx = [], np.zeros(bt_host.shape, dtype=np.int32)
    off = 0
    for b in reqs:
        n = w.nblk[b]
        phys_list.append(bt_host[b, :n])
        bt_idx[b, :n] = np.arange(off, off + n, dtype=np.int32)
        off += n
    phys = torch.from_numpy(np.concatenate(phys_list)).to(t["block_table"].device)
    ik = _compact(t["idx_k_pool"], phys)
    iks = _compact(t.get("idx_k_scale"), phys)
    del phys
    s = oracle.index_scores(prob, _host(t["idx_q"]), ik, bt_idx, ctx, rows_np, idx_k_scale=iks)
    del ik, iks
    sel, nsel = oracle.select(prob, s, ctx, rows_np)
    pt = oracle.page_table(prob, sel, bt_host.astype(np.int32), rows_np)

    # attention on a pool holding only the selected blocks (all rows at once)
    bt_kv = np.zeros(bt_host.shape, dtype=np.int32)
    used = {}
    for i, r in enumerate(rows):
        b = r // T
        for x in sel[i]:
            if x >= 0:
                key = int(bt_host[b, x])
                if key not in used:
                    used[key] = len(used)
                bt_kv[b, x] = used[key]
    order = np.empty(len(used), dtype=np.int64)
    for key, j in used.items():
        order[j] = key
    phys = torch.from_numpy(order).to(t["block_table"].device)
    kv = {name: _compact(t[name], phys) for name in ("k_pool", "v_pool", "k_scale", "v_scale")}
    out = oracle.attention(prob, _host(t["q"]), kv["k_pool"], kv["v_pool"], kv["k_scale"],
                           kv["v_scale"], bt_kv, ctx, sel, rows_np)
    return {r: {"scores": s[i][:w.nblk[r // T]], "selected": sel[i], "n_selected": int(nsel[i]),
                "page_table": pt[i], "out": out[i]} for i, r in enumerate(rows)}


def oracle_attention_rows(w: Workload, rows, selection):
    """Oracle attention output of the given rows of `w` over a given
    selection (row -> logical block ids, -1 padded), e.g. one another layer
    made; compact host pools of just those blocks, request by request."""
    c = w.cfg
    T = c.query_len
    t = w.tensors
    out = {}
    by_req = {}
    for r in rows:
        by_req.setdefault(r // T, []).append(r)
    for b, rs in by_req.items():
        nblk = w.nblk[b]
        bt_row = t["block_table"][b, :nblk].to(torch.int64)
        local_rows = np.array([r % T for r in rs], dtype=np.int32)
        sel = np.full((T, c.topk), -1, dtype=np.int32)
        for r in rs:
            sel[r % T] = selection[r]
        mini = problem_of(c)
        mini.batch = 1
        mini.max_blocks = nblk
        used = sorted({int(x) for x in sel.reshape(-1) if x >= 0})
        remap = np.zeros(nblk, dtype=np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        phys = bt_row[torch.tensor(used, dtype=torch.int64, device=bt_row.device)]
        kv = {name: None if t[name] is None else _host(t[name][phys])
              for name in ("k_pool", "v_pool", "k_scale", "v_scale")}
        o = oracle.attention(mini, _host(t["q"][b * T:(b + 1) * T]), kv["k_pool"], kv["v_pool"],
                             kv["k_scale"], kv["v_scale"], remap[None, :],
                             np.array([w.ctx_lens[b]], dtype=np.int32), sel[local_rows],
                             local_rows)
        for i, r in enumerate(rs):
            out[r] = o[i]
    return out


def compare_rows(w: Workload, got, rows, ref=None):
    """Bit-exact scores / selection / page table, tolerance on outputs."""
    c = w.cfg
    ref = ref if ref is not None else oracle_rows(w, rows)
    tol = TOL[c.kv_dtype]
    sc = got["scores"][rows].cpu().numpy() if "scores" in got else None
    sel = got["selected"][rows].cpu().numpy()
    pt = got["page_table"][rows].cpu().numpy()
    out = got["out"][rows].cpu().numpy()
    nsel = got["n_selected"][rows].cpu().numpy() if "n_selected" in got else None
    worst = 0.0
    for i, r in enumerate(rows):
        e = ref[r]
        nb = e["scores"].shape[0]
        if sc is not None:
            assert np.array_equal(sc[i][:nb].astype(np.float64), e["scores"]), f"scores row {r}"
            assert np.all(np.isneginf(sc[i][nb:])), f"scores tail row {r}"
        assert np.array_equal(sel[i], e["selected"]), f"selected row {r}"
        if nsel is not None:
            assert nsel[i] == e["n_selected"], f"n_selected row {r}"
        assert np.array_equal(pt[i], e["page_table"]), f"page_table row {r}"
        err = float(np.max(np.abs(out[i].astype(np.float64) - e["out"])))
        worst = max(worst, err)
        assert err <= tol, f"out row {r}: max abs err {err} > {tol}"
    return worst


def check_invariants(w: Workload, got):
    """Properties every row must satisfy, checked for the whole batch."""
    c = w.cfg
    T = c.query_len
    sel = got["selected"].cpu().numpy()
    pt = got["page_table"].cpu().numpy()
    bt = w.tensors["block_table"].cpu().numpy()
    for r in range(c.rows):
        b, t = divmod(r, T)
        pos = w.ctx_lens[b] - T + t
        local = pos // 128
        n = min(c.topk, local + 1)
        s = sel[r]
        assert np.all(s[n:] == -1) and np.all(s[:n] >= 0)
        assert s[n - 1] == local, f"row {r}: local block missing"
        assert np.all(np.diff(s[:n]) > 0), f"row {r}: not ascending"
        want = np.full(c.topk * 8, -1, dtype=np.int64)
        want[:n * 8] = (bt[b, s[:n]][:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
        assert np.array_equal(pt[r], want), f"row {r}: page table"
        keys = sum(min(128, pos + 1 - int(x) * 128) for x in s[:n])
        assert keys <= 2048
    out = got["out"]
    assert torch.isfinite(out).all()
