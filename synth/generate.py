"""Seeded synthetic inputs for MSA decode, shared by the oracle and the GPU path.

This module only draws random numbers and stores them in the boundary's
layouts; it holds none of the method's arithmetic (no scoring, selection,
paging or attention).  The random source is a counter-based 32-bit hash
(Chris Wellons' "triple32" integer hash, a published bijection on 32-bit
words) evaluated with exact int64 tensor arithmetic, so the same seed gives
the same integers on the CPU and on the GPU.

Layouts produced (row r = b * T + t):
  q          [R, Hq, 128]           bf16, ~N(0, 1)
  idx_q      [R, Hidx, 64]          bf16 holding integers uniform in [-8, 8]
  idx_k_pool [NB, Hidx, 128, 64]    bf16 or fp8-e4m3 codes (uint8), integers
  k_pool/v_pool
      bf16   [NB, Hkv, 128, 128]    bf16, ~N(0, 1)
      fp8    [NB, Hkv, 128, 128]    uint8 e4m3 codes; k_scale/v_scale
                                    [NB, Hkv, 128] fp32 (one per token, head)
      nvfp4  [NB, Hkv, 128, 64]     uint8, two e2m1 codes per byte (element
                                    2j in the low nibble); k_scale/v_scale
                                    [NB, Hkv, 128, 8] uint8 e4m3 codes, one
                                    per 16 consecutive elements
  block_table [B, MAXB] int32 (entries past a request's last block are 0)
  ctx_lens    [B] int32
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np
import torch

MASK32 = 0xFFFFFFFF
BLOCK = 128
PAGE = 16
HEAD_DIM = 128
IDX_DIM = 64
CHUNK = 1 << 24  # elements generated per tensor op batch (bounds temporaries)

# stream ids: one per generated quantity
_S_CTX, _S_PERM, _S_PLANT, _S_IQ, _S_IK, _S_Q, _S_K, _S_V, _S_IKS = range(1, 10)

# E4M3 codes of the 4-bit index-key scales the generator draws: 1, 2, 4, 8.
# With E2M1 codes (multiples of 0.5, at most 6) and integer queries in
# [-8, 8], every product and every fp32 partial sum of a score is exact.
IDX_FP4_SCALE_CODES = (0x38, 0x40, 0x48, 0x50)


# ---------------------------------------------------------------- hashing
def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 x in [0, 2^32), without int64 overflow."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & MASK32


def _triple32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 17)
    x = _mul32(x, 0xED5AD4BB)
    x = x ^ (x >> 11)
    x = _mul32(x, 0xAC4C1B51)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x31848BAB)
    x = x ^ (x >> 14)
    return x


def _triple32_int(x: int) -> int:
    x &= MASK32
    x ^= x >> 17
    x = (x * 0xED5AD4BB) & MASK32
    x ^= x >> 11
    x = (x * 0xAC4C1B51) & MASK32
    x ^= x >> 15
    x = (x * 0x31848BAB) & MASK32
    x ^= x >> 14
    return x


def rand32(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """32-bit random words (int64 tensor) for counters idx (< 2^40)."""
    key = _triple32_int(seed * 0x9E3779B9 + stream * 0x85EBCA6B)
    hi = idx >> 32
    lo = idx & MASK32
    mix = _triple32((hi + key) & MASK32)
    return _triple32(lo ^ mix)


def _uniform01(r: torch.Tensor) -> torch.Tensor:
    """Open-interval (0, 1) float64 from the top 24 bits of a word."""
    return ((r >> 8).to(torch.float64) + 0.5) * (1.0 / (1 << 24))


def _normal(seed: int, stream: int, start: int, n: int, device) -> torch.Tensor:
    """n standard normals (float32) by Box-Muller on counters start..start+n."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    u1 = _uniform01(rand32(seed, stream, 2 * idx))
    u2 = _uniform01(rand32(seed, stream, 2 * idx + 1))
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)
    return z.to(torch.float32)


def _small_ints(seed: int, stream: int, start: int, n: int, device, lo=-8, hi=8):
    """n integers uniform in [lo, hi] (float32); modulo bias below 2^-27."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    r = rand32(seed, stream, idx)
    return (r % (hi - lo + 1) + lo).to(torch.float32)


def _uniform_codes(seed: int, stream: int, start: int, n: int, device, count: int):
    """n integers uniform in [0, count) for a power-of-two count (float32)."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    return (rand32(seed, stream, idx) & (count - 1)).to(torch.float32)


def _randint_host(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    return rand32(seed, stream, torch.from_numpy(np.asarray(idx, dtype=np.int64))).numpy()


# ------------------------------------------------------------- encoders
def encode_fp8_per_token(x: torch.Tensor):
    """x [..., D] float32 -> (e4m3 codes uint8 [..., D], fp32 scale [...]):
    scale = amax / 448 per row, code = round-to-nearest-even(x / scale)."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def encode_e2m1(y: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even onto the e2m1 grid {0,.5,1,1.5,2,3,4,6}, saturating
    at 6; returns 4-bit codes (sign in bit 3) as uint8."""
    a = y.abs().clamp(max=6.0)
    mids = torch.tensor(_E2M1_MIDS, dtype=a.dtype, device=a.device)
    m = torch.bucketize(a, mids)  # a == mids[i] -> i (lower neighbour)
    at_mid = (m < 7) & (a == mids[m.clamp(max=6)])
    m = m + (at_mid & (m % 2 == 1)).to(m.dtype)  # tie -> even code
    sign = (y < 0) & (m > 0)
    return (m + 8 * sign.to(m.dtype)).to(torch.uint8)


def encode_nvfp4(x: torch.Tensor):
    """x [..., D] float32 -> (packed uint8 [..., D/2], e4m3 scale codes
    [..., D/16]): per 16 elements s = e4m3_rne(amax / 6); code = e2m1_rne(x/s);
    all-zero codes when s rounds to 0."""
    shp = x.shape
    g = x.reshape(*shp[:-1], shp[-1] // 16, 16)
    s_code = (g.abs().amax(dim=-1) / 6.0).to(torch.float8_e4m3fn)
    s = s_code.to(torch.float32)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    codes = encode_e2m1(g / safe.unsqueeze(-1))
    codes = torch.where((s > 0).unsqueeze(-1), codes, torch.zeros_like(codes))
    codes = codes.reshape(*shp[:-1], shp[-1])
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.to(torch.uint8), s_code.view(torch.uint8)


# --------------------------------------------------------------- configs
@dataclass(frozen=True)
class MSAConfig:
    name: str
    batch: int
    query_len: int
    num_q_heads: int
    num_kv_heads: int
    num_idx_heads: int
    ctx_lo: int
    ctx_hi: int
    kv_dtype: str = "bf16"      # bf16 | fp8 | nvfp4
    idx_dtype: str = "bf16"     # bf16 | fp8 | nvfp4
    n_plant: int = 0
    permute: bool = True
    seed: int = 1000
    topk: int = 16
    ctx_list: Optional[tuple] = None  # explicit context lengths (overrides lo/hi)

    @property
    def max_blocks(self) -> int:
        hi = max(self.ctx_list) if self.ctx_list else self.ctx_hi
        return -(-hi // BLOCK)

    @property
    def rows(self) -> int:
        return self.batch * self.query_len


# The five workloads: tiny, one TP8 rank, a full 128K-context layer,
# speculative verify with fp8 KV, and 1M context with 4-bit KV.
CONFIGS: Dict[str, MSAConfig] = {
    "tiny_4k": MSAConfig("tiny_4k", 1, 1, 8, 1, 1, 4096, 4096, n_plant=3, permute=False,
                         seed=1000),
    "tp8_rank_32k": MSAConfig("tp8_rank_32k", 32, 1, 8, 1, 1, 32768, 32768, n_plant=8,
                              seed=1001),
    "layer_128k": MSAConfig("layer_128k", 64, 1, 64, 4, 4, 8192, 131072, n_plant=8,
                            seed=1002),
    "spec_verify_fp8": MSAConfig("spec_verify_fp8", 128, 4, 8, 1, 1, 8192, 16384,
                                 kv_dtype="fp8", idx_dtype="fp8", n_plant=0, seed=1003),
    "ctx_1m_nvfp4": MSAConfig("ctx_1m_nvfp4", 4, 1, 64, 4, 4, 1048576, 1048576,
                              kv_dtype="nvfp4", idx_dtype="fp8", n_plant=16, seed=1004),
    # the 128K layer with 4-bit index keys (E2M1 + E4M3 per 16 dims): the
    # next index-cache format, 36 bytes per token and index head
    "layer_128k_nvfp4_index": MSAConfig("layer_128k_nvfp4_index", 64, 1, 64, 4, 4, 8192, 131072,
                                        idx_dtype="nvfp4", n_plant=8, seed=1005),
}
CONFIG_ORDER = ["tiny_4k", "tp8_rank_32k", "layer_128k", "spec_verify_fp8", "ctx_1m_nvfp4"]
# workloads beyond the five above (formats the path supports next)
EXTRA_CONFIGS = ["layer_128k_nvfp4_index"]


@dataclass
class Workload:
    cfg: MSAConfig
    ctx_lens: List[int]
    nblk: List[int]
    num_phys_blocks: int
    planted: List[List[int]]           # logical planted blocks per request
    tensors: Dict[str, Optional[torch.Tensor]] = field(default_factory=dict)

    @property
    def device(self):
        return self.tensors["q"].device


def _ctx_lens(cfg: MSAConfig) -> List[int]:
    if cfg.ctx_list is not None:
        assert len(cfg.ctx_list) == cfg.batch
        return [int(x) for x in cfg.ctx_list]
    if cfg.ctx_lo == cfg.ctx_hi:
        return [cfg.ctx_lo] * cfg.batch
    r = _randint_host(cfg.seed, _S_CTX, np.arange(cfg.batch))
    return [int(cfg.ctx_lo + v % (cfg.ctx_hi - cfg.ctx_lo + 1)) for v in r]


def _permutation(seed: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by the counter hash."""
    perm = np.arange(n, dtype=np.int64)
    r = _randint_host(seed, _S_PERM, np.arange(n))
    for i in range(n - 1, 0, -1):
        j = int(r[i] % (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def _fill(out: torch.Tensor, gen) -> None:
    """Fill a contiguous tensor chunk by chunk: gen(start, n) -> values."""
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        flat[s:e] = gen(s, e - s).to(flat.dtype)


def layout(cfg: MSAConfig):
    """(context lengths, blocks per request, block table [B, MAXB]) of a
    workload, without generating its tensors."""
    T, B = cfg.query_len, cfg.batch
    ctx = _ctx_lens(cfg)
    if min(ctx) < T:
        raise ValueError("every context must hold at least decode_query_len tokens")
    nblk = [-(-L // BLOCK) for L in ctx]
    NB = int(sum(nblk))
    MAXB = cfg.max_blocks
    # logical -> physical block map
    phys = _permutation(cfg.seed, NB) if cfg.permute else np.arange(NB, dtype=np.int64)
    bt = np.zeros((B, MAXB), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = phys[off:off + nblk[b]]
        off += nblk[b]
    return ctx, nblk, bt


def write_spec(cfg: MSAConfig, path: str) -> None:
    """Text description of a workload's shapes, contexts and block table for
    the counter driver: one header line, B context lengths, B*MAXB table
    entries."""
    ctx, nblk, bt = layout(cfg)
    with open(path, "w") as f:
        f.write(f"{cfg.batch} {cfg.query_len} {cfg.num_q_heads} {cfg.num_kv_heads} "
                f"{cfg.num_idx_heads} {cfg.max_blocks} {sum(nblk)} {cfg.kv_dtype} "
                f"{cfg.idx_dtype} {cfg.topk}\n")
        f.write(" ".join(str(x) for x in ctx) + "\n")
        f.write(" ".join(str(int(x)) for x in bt.reshape(-1)) + "\n")


def make_workload(cfg: MSAConfig, device="cpu", layer: int = 0) -> Workload:
    """The workload's tensors.  `layer` > 0 draws another layer of the same
    model state: same context lengths and block table (the block table is
    shared by all layers), fresh queries, keys and values."""
    device = torch.device(device)
    T, B = cfg.query_len, cfg.batch
    R = B * T
    ctx, nblk, bt = layout(cfg)
    NB = int(sum(nblk))
    MAXB = cfg.max_blocks

    seed = cfg.seed + 100003 * layer
    t = {}
    t["ctx_lens"] = torch.tensor(ctx, dtype=torch.int32, device=device)
    t["block_table"] = torch.from_numpy(bt).to(device)

    # index queries: integers in [-8, 8]
    iq = torch.empty((R, cfg.num_idx_heads, IDX_DIM), dtype=torch.float32, device=device)
    _fill(iq, lambda s, n: _small_ints(seed, _S_IQ, s, n, device))
    t["idx_q"] = iq.to(torch.bfloat16)

    # index keys, by physical element position: integers in [-8, 8] (bf16 /
    # fp8), or 4-bit E2M1 codes with an E4M3 scale per 16 dims (nvfp4)
    fp4 = cfg.idx_dtype == "nvfp4"
    ik = torch.empty((NB, cfg.num_idx_heads, BLOCK, IDX_DIM), dtype=torch.int8, device=device)
    if fp4:
        _fill(ik, lambda s, n: _uniform_codes(seed, _S_IK, s, n, device, 16))
    else:
        _fill(ik, lambda s, n: _small_ints(seed, _S_IK, s, n, device))

    # planted blocks: components aligned with sign(index q of row 0) get +4
    # (integer keys) or the E2M1 code of +-6 (4-bit keys)
    planted: List[List[int]] = []
    for b in range(B):
        local0 = (ctx[b] - T) // BLOCK
        n_p = min(cfg.n_plant, local0)
        chosen: List[int] = []
        if n_p > 0:
            cand = np.arange(local0, dtype=np.int64)
            r = _randint_host(seed + 7919 * (b + 1), _S_PLANT, np.arange(n_p))
            for i in range(n_p):  # partial Fisher-Yates
                j = i + int(r[i] % (local0 - i))
                cand[i], cand[j] = cand[j], cand[i]
            chosen = sorted(int(c) for c in cand[:n_p])
            sgn = torch.sign(iq[b * T]).to(torch.int8)  # [Hidx, 64]
            pb = torch.tensor([int(bt[b, c]) for c in chosen], dtype=torch.int64,
                              device=device)
            if fp4:
                six = torch.where(sgn > 0, 0x7, 0xF).to(torch.int8)  # +6 / -6
                blk = ik[pb]
                ik[pb] = torch.where(sgn.unsqueeze(1) != 0, six.unsqueeze(1), blk)
            else:
                ik[pb] += 4 * sgn.unsqueeze(1)
        planted.append(chosen)
    t["idx_k_scale"] = None
    if fp4:
        nib = ik.to(torch.uint8).view(NB, cfg.num_idx_heads, BLOCK, IDX_DIM // 2, 2)
        t["idx_k_pool"] = (nib[..., 0] | (nib[..., 1] << 4)).contiguous()
        sc = torch.empty((NB, cfg.num_idx_heads, BLOCK, IDX_DIM // 16), dtype=torch.int8,
                         device=device)
        _fill(sc, lambda s, n: _uniform_codes(seed, _S_IKS, s, n, device, 4))
        codes = torch.tensor(IDX_FP4_SCALE_CODES, dtype=torch.uint8, device=device)
        t["idx_k_scale"] = codes[sc.to(torch.int64)]
    elif cfg.idx_dtype == "bf16":
        t["idx_k_pool"] = ik.to(torch.bfloat16)
    else:
        t["idx_k_pool"] = ik.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    del ik

    # queries
    q = torch.empty((R, cfg.num_q_heads, HEAD_DIM), dtype=torch.bfloat16, device=device)
    _fill(q, lambda s, n: _normal(seed, _S_Q, s, n, device))
    t["q"] = q

    # keys / values
    kv_shape = (NB, cfg.num_kv_heads, BLOCK, HEAD_DIM)
    for name, stream in (("k", _S_K), ("v", _S_V)):
        if cfg.kv_dtype == "bf16":
            pool = torch.empty(kv_shape, dtype=torch.bfloat16, device=device)
            _fill(pool, lambda s, n, st=stream: _normal(seed, st, s, n, device))
            t[name + "_pool"] = pool
            t[name + "_scale"] = None
            continue
        if cfg.kv_dtype == "fp8":
            pool = torch.empty(kv_shape, dtype=torch.uint8, device=device)
            scale = torch.empty(kv_shape[:-1], dtype=torch.float32, device=device)
        else:
            pool = torch.empty(kv_shape[:-1] + (HEAD_DIM // 2,), dtype=torch.uint8,
                               device=device)
            scale = torch.empty(kv_shape[:-1] + (HEAD_DIM // 16,), dtype=torch.uint8,
                                device=device)
        rows_per = max(1, CHUNK // HEAD_DIM)
        flat_rows = NB * cfg.num_kv_heads * BLOCK
        pv = pool.view(flat_rows, -1)
        sv = scale.view(flat_rows, -1)
        for s in range(0, flat_rows, rows_per):
            e = min(flat_rows, s + rows_per)
            x = _normal(seed, stream, s * HEAD_DIM, (e - s) * HEAD_DIM, device)
            x = x.view(e - s, HEAD_DIM)
            if cfg.kv_dtype == "fp8":
                c, sc = encode_fp8_per_token(x)
                pv[s:e] = c
                sv[s:e, 0] = sc
            else:
                c, sc = encode_nvfp4(x)
                pv[s:e] = c
                sv[s:e] = sc
        t[name + "_pool"] = pool
        t[name + "_scale"] = scale
    return Workload(cfg=cfg, ctx_lens=ctx, nblk=nblk, num_phys_blocks=NB, planted=planted,
                    tensors=t)


def small_config(name="small", **kw) -> MSAConfig:
    """A quick ad-hoc configuration for tests (defaults: 2 requests, 1.5K-3K ctx)."""
    base = MSAConfig(name, batch=2, query_len=1, num_q_heads=8, num_kv_heads=1,
                     num_idx_heads=1, ctx_lo=1500, ctx_hi=3000, seed=7)
    return replace(base, **kw)


def host_arrays(w: Workload) -> Dict[str, Optional[np.ndarray]]:
    """Host numpy views of a workload in the oracle's storage types (bf16 as
    uint16 bit patterns, fp8 / 4-bit as uint8, scales as stored)."""
    out = {}
    for k, v in w.tensors.items():
        if v is None:
            out[k] = None
            continue
        v = v.detach().to("cpu")
        if v.dtype == torch.bfloat16:
            v = v.view(torch.int16).numpy().view(np.uint16)
        else:
            v = v.numpy()
        out[k] = v
    return out
