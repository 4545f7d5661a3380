"""MSA decode benchmark on one MI355X.

One step = one fused msa_decode (index scan, top-k selection, page table,
split-K sparse attention, LSE merge) over one batch of synthetic input that
is already resident in HBM.  The default workload is the full 128K-context
layer: 64 requests with contexts uniform in [8192, 131072], 64 query / 4 KV /
4 index heads, bf16 KV and index keys.

Prints one JSON line: query-tokens/s for the whole batch, the roofline of
the dominant kernel (the index-key scan) measured live with HIP events, the
CPU oracle timed on the same workload (median of 3 passes on all host
cores, plus single-core runs on the two smallest configurations), and a
compact record per other configuration (step time back to back and after a
cache flush, end-to-end and scan fractions of the HBM peak).

    python bench.py [--steps K] [--warmup W] [--workload layer_128k]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "MSA decode query-tokens/s at 128K ctx; achieved HBM GB/s vs peak"
SCAN_KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_10_amd", "csrc", f)
                    for f in ("index_scan.hip", "msa_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "msa_decode_{}_traffic.json")


def kv_elem_bytes(kv):
    return {"bf16": 2.0, "fp8": 1.0, "nvfp4": 0.5}[kv]


def algorithmic_bytes(w, selected):
    """Full index-key scan + the KV of the attended keys (each key once per
    request, even when several draft rows attend it) + metadata.  `selected`
    is the [R, topk] selection of one run."""
    c = w.cfg
    T = c.query_len
    # index key bytes per (token, head): bf16 128, fp8 64, 4-bit 32 + 4 scales
    per_tok = {"bf16": 128, "fp8": 64, "nvfp4": 36}[c.idx_dtype]
    idx = sum(w.nblk) * 128 * c.num_idx_heads * per_tok
    # per attended key and KV head: K and V rows plus their scales
    per_key = 2 * 128 * kv_elem_bytes(c.kv_dtype)
    if c.kv_dtype == "fp8":
        per_key += 2 * 4
    elif c.kv_dtype == "nvfp4":
        per_key += 2 * 8
    keys = 0
    for b in range(c.batch):
        reach = {}  # block -> number of its tokens attended by some row
        for t in range(T):
            p = w.ctx_lens[b] - T + t
            for blk in selected[b * T + t]:
                if blk < 0:
                    continue
                blk = int(blk)
                reach[blk] = max(reach.get(blk, 0), min(128, p + 1 - 128 * blk))
        keys += sum(reach.values())
    kv = keys * c.num_kv_heads * per_key
    R = c.rows
    meta = (R * c.num_q_heads * 128 * 2 + R * c.num_idx_heads * 64 * 2 + c.batch * 4 +
            c.batch * c.max_blocks * 4 + 2 * R * c.max_blocks * 4 + R * c.topk * 4 +
            R * c.topk * 8 * 4 * 2 + R * c.num_q_heads * 128 * 4)
    return {"index": idx, "kv": int(kv), "meta": int(meta), "total": int(idx + kv + meta)}


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per scan launch from committed rocprofv3 counter runs on
    this workload, if they were taken on the current scan kernel source."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get("index_scan", {})
    if rec.get("kernel_source_sha256_16") != source_hash(SCAN_KERNEL_SRCS):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, n_requests, passes=3, threads=None):
    """The oracle on `n_requests` requests of the workload (their rows only):
    scan, selection, page table and attention, `passes` times on the host
    cores (`threads` worker threads, default all), reporting the median
    pass.  Gathering the compact host pools is not timed."""
    import numpy as np
    import torch

    import oracle
    from tests.refs import problem_of

    c = w.cfg
    T = c.query_len
    t = w.tensors
    reqs = list(range(0, c.batch, max(1, c.batch // n_requests)))[:n_requests]

    def host(x):
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16)
        return x.numpy()

    # compact index-key pool of the sampled requests
    nblk = [w.nblk[b] for b in reqs]
    maxb = max(nblk)
    bt = np.zeros((len(reqs), maxb), dtype=np.int32)
    phys = []
    off = 0
    for i, b in enumerate(reqs):
        bt[i, :nblk[i]] = np.arange(off, off + nblk[i])
        phys.append(t["block_table"][b, :nblk[i]].to(torch.int64))
        off += nblk[i]
    phys = torch.cat(phys)
    P = problem_of(c)
    P.batch = len(reqs)
    P.max_blocks = maxb
    ctx = np.array([w.ctx_lens[b] for b in reqs], dtype=np.int32)
    rows_q = torch.tensor([b * T + k for b in reqs for k in range(T)], dtype=torch.int64,
                          device=t["q"].device)
    iq = host(t["idx_q"][rows_q])
    ik = host(t["idx_k_pool"][phys])
    iks = None if t.get("idx_k_scale") is None else host(t["idx_k_scale"][phys])
    q = host(t["q"][rows_q])

    def kv_of_selected(sel):
        """Compact K/V pools holding only the selected blocks, and the table
        mapping (request, logical block) into them."""
        bt_kv = np.zeros((len(reqs), maxb), dtype=np.int32)
        take = []
        for i, b in enumerate(reqs):
            blocks = sorted(set(int(x) for x in sel[i * T:(i + 1) * T].reshape(-1) if x >= 0))
            for blk in blocks:
                bt_kv[i, blk] = len(take)
                take.append(int(t["block_table"][b, blk]))
        idx = torch.tensor(take, dtype=torch.int64, device=t["q"].device)
        kv = {k: (None if t[k] is None else host(t[k][idx]))
              for k in ("k_pool", "v_pool", "k_scale", "v_scale")}
        return kv, bt_kv

    all_threads = oracle.num_threads()
    if threads is not None:
        oracle.set_num_threads(threads)
    try:
        used = oracle.num_threads()
        times, kv = [], None
        for _ in range(passes):
            t0 = time.perf_counter()
            s = oracle.index_scores(P, iq, ik, bt, ctx, idx_k_scale=iks)
            sel, _ = oracle.select(P, s, ctx)
            oracle.page_table(P, sel, bt)
            t1 = time.perf_counter()
            if kv is None:
                kv, bt_kv = kv_of_selected(sel)
            t2 = time.perf_counter()
            oracle.attention(P, q, kv["k_pool"], kv["v_pool"], kv["k_scale"], kv["v_scale"],
                             bt_kv, ctx, sel)
            times.append((t1 - t0) + (time.perf_counter() - t2))
    finally:
        oracle.set_num_threads(all_threads)
    rows = len(reqs) * T
    med = sorted(times)[len(times) // 2]
    return {"value": rows / med, "unit": "query-tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{len(reqs)} of {c.batch} requests ({rows} query rows, full contexts), "
                      f"median of {passes} passes",
            "pass_s": [round(x, 4) for x in times]}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def describe_workload(cfg):
    return (f"{cfg.name}: batch {cfg.batch}, decode_query_len {cfg.query_len}, "
            f"context U[{cfg.ctx_lo}, {cfg.ctx_hi}], heads q/kv/idx "
            f"{cfg.num_q_heads}/{cfg.num_kv_heads}/{cfg.num_idx_heads}, "
            f"KV {cfg.kv_dtype}, index keys {cfg.idx_dtype}, top-{cfg.topk} "
            f"blocks of 128 with the local block")


class Timed:
    """One workload resident on the GPU with its descriptor and buffers."""

    def __init__(self, cfg):
        import torch

        import block_sparse_attention_10_amd as msa
        from synth import make_workload

        self.msa = msa
        self.cfg = cfg
        self.w = make_workload(cfg, "cuda")
        torch.cuda.synchronize()
        wt = self.w.tensors
        self.p, self.t = msa.describe(wt["q"], wt["idx_q"], wt["k_pool"], wt["v_pool"],
                                      wt["k_scale"], wt["v_scale"], wt["idx_k_pool"],
                                      wt["block_table"], wt["ctx_lens"],
                                      decode_query_len=cfg.query_len, topk=cfg.topk,
                                      idx_k_scale=wt.get("idx_k_scale"))
        R = cfg.rows
        self.scores = torch.empty((R, cfg.max_blocks), dtype=torch.float32, device="cuda")
        self.selected = torch.empty((R, cfg.topk), dtype=torch.int32, device="cuda")
        self.out = torch.empty((R, cfg.num_q_heads, 128), dtype=torch.float32, device="cuda")
        self.ws = torch.empty((msa.msa_workspace_bytes(self.p),), dtype=torch.uint8,
                              device="cuda")
        msa.msa_decode(self.p, self.t, self.selected, None, self.out, self.ws)
        torch.cuda.synchronize()
        self.ab = algorithmic_bytes(self.w, self.selected.cpu().numpy())

    def step(self):
        self.msa.msa_decode(self.p, self.t, None, None, self.out, self.ws)

    def scan(self):
        self.msa.msa_index_score(self.p, self.t, self.scores)


def time_loop(fn, steps, warmup):
    """Mean microseconds per call of `fn`, back to back on the current stream,
    measured with HIP events on that stream."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps * 1e3


def time_cold(fn, steps):
    """Percentiles of single calls, each after a 1 GiB write that evicts the
    L2s and the 256 MB last-level cache (the write is outside the events)."""
    import torch

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    cold = []
    for _ in range(steps):
        flush.fill_(1.0)
        start.record()
        fn()
        end.record()
        torch.cuda.synchronize()
        cold.append(start.elapsed_time(end) * 1e3)
    del flush
    cold.sort()
    return {"p10": cold[len(cold) // 10], "p50": cold[len(cold) // 2],
            "p90": cold[(9 * len(cold)) // 10], "steps": len(cold)}


def workload_record(cfg, steps, warmup, cold_steps):
    """Step time (back to back and after a cache flush), the end-to-end
    fraction of the HBM peak and the scan's own fraction, for one workload."""
    import torch

    tw = Timed(cfg)
    warm_us = time_loop(tw.step, steps, warmup)
    cold = time_cold(tw.step, cold_steps)
    dispatch = tw.msa.msa_last_dispatch()
    scan_us = time_loop(tw.scan, steps, warmup)
    ab = tw.ab
    rec = {
        "workload": describe_workload(cfg),
        "rows": cfg.rows,
        "step_us": round(warm_us, 2),
        "step_us_after_cache_flush_p50": round(cold["p50"], 2),
        "query_tokens_per_s": cfg.rows / (warm_us * 1e-6),
        "query_tokens_per_s_after_cache_flush": cfg.rows / (cold["p50"] * 1e-6),
        "algorithmic_bytes_per_step": ab["total"],
        "frac_of_peak_end_to_end": ab["total"] / (warm_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "frac_of_peak_end_to_end_after_cache_flush":
            ab["total"] / (cold["p50"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "scan_us": round(scan_us, 2),
        "scan_frac_of_peak": ab["index"] / (scan_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "kernels": dispatch,
    }
    del tw
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer_128k")
    ap.add_argument("--cpu-requests", type=int, default=64,
                    help="requests the all-core CPU oracle baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-workload records of the other configurations")
    ap.add_argument("--export-spec", default=None,
                    help="write the workload's shapes, contexts and block table for the "
                         "counter driver (msa_counters.cpp) and exit")
    args = ap.parse_args()

    if args.export_spec:
        from synth import CONFIGS, write_spec
        write_spec(CONFIGS[args.workload], args.export_spec)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (across GPUs the "
              "path would shard by request, or by context with two small exchanges).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import CONFIG_ORDER, CONFIGS, EXTRA_CONFIGS

    cfg = CONFIGS[args.workload]
    tw = Timed(cfg)
    msa = tw.msa
    w, p, t, o_out, ws = tw.w, tw.p, tw.t, tw.out, tw.ws
    wt = w.tensors
    R = cfg.rows
    ab = tw.ab

    us = time_loop(tw.step, args.steps, args.warmup)
    ms = us * 1e-3
    dispatch = msa.msa_last_dispatch()
    cold_us = time_cold(tw.step, min(args.steps, 20))

    # the dominant kernel alone: index-key scan, same stream, same buffers
    scan_us = time_loop(tw.scan, args.steps, args.warmup)
    achieved = ab["index"] / (scan_us * 1e-6) / 1e9

    # a layer that reuses another layer's selection (index sharing across
    # adjacent sparse layers): attention over a page table, scan and
    # selection skipped
    pt = torch.empty((R, cfg.topk * 8), dtype=torch.int32, device="cuda")
    msa.msa_decode(p, t, None, pt, o_out, ws)
    reuse_us = time_loop(lambda: msa.msa_sparse_decode(p, t, pt, o_out, ws), args.steps,
                         args.warmup)

    # the write path of a step: the R new tokens' K, V and index keys go into
    # the pools (quantised to their formats); timed last, as it changes them
    gen = torch.Generator(device="cuda").manual_seed(7)
    new = [torch.randn((R, H, Dh), generator=gen, device="cuda").to(torch.bfloat16)
           for H, Dh in ((cfg.num_kv_heads, 128), (cfg.num_kv_heads, 128),
                         (cfg.num_idx_heads, 64))]
    pl = msa.pools(wt["k_pool"], wt["v_pool"], wt["k_scale"], wt["v_scale"], wt["idx_k_pool"],
                   wt.get("idx_k_scale"))
    insert_us = time_loop(lambda: msa.msa_insert_kv(p, pl, wt["block_table"], wt["ctx_lens"],
                                                    *new), args.steps, args.warmup)

    rec = {
        "metric": METRIC,
        "value": cfg.rows / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": describe_workload(cfg),
            "batch": cfg.batch,
            "decode_query_len": cfg.query_len,
            "mean_context": sum(w.ctx_lens) / cfg.batch,
            "algorithmic_bytes_per_step": ab,
            "achieved_GBps_end_to_end": ab["total"] / (ms * 1e-3) / 1e9,
            "frac_of_peak_end_to_end": ab["total"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "kernels": dispatch,
            "step_us_after_cache_flush": cold_us,
            "frac_of_peak_end_to_end_after_cache_flush":
                ab["total"] / (cold_us["p50"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "insert": {
                "us": insert_us,
                "rows": R,
                "note": "write path: K, V and index key of each row's new token into the pools",
            },
            "reuse_layer": {
                "us_per_layer": reuse_us,
                "query_tokens_per_s": R / (reuse_us * 1e-6),
                "kv_GBps": ab["kv"] / (reuse_us * 1e-6) / 1e9,
            },
        },
        "roofline": {
            "kernel": "index_scan",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "avg_launch_us": scan_us,
            "algorithmic_bytes_per_launch": ab["index"],
            "traffic": measured_traffic(cfg.name),
        },
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_requests)
        cpu["cpu"] = cpu_model()
        cpu["host_cpus"] = os.cpu_count()
    del tw, w, wt, p, t, o_out, ws, pt, new, pl
    torch.cuda.empty_cache()

    # the other configurations: their own step records (not the headline)
    if not args.no_other_workloads:
        others = {}
        for name in CONFIG_ORDER + EXTRA_CONFIGS:
            if name == cfg.name:
                continue
            others[name] = workload_record(CONFIGS[name], min(args.steps, 20), args.warmup,
                                           min(args.steps, 10))
            # single-core oracle baselines of the two smallest configurations
            if cpu is not None and name in ("tiny_4k", "tp8_rank_32k"):
                from synth import make_workload
                wsmall = make_workload(CONFIGS[name], "cuda")
                cpu.setdefault("single_core", {})[name] = cpu_baseline(
                    wsmall, 1 if name == "tiny_4k" else 8, threads=1)
                del wsmall
                torch.cuda.empty_cache()
        rec["other_workloads"] = others
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
