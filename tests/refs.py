"""Independent references used to pin the oracle (tests only).

Nothing here calls the oracle or the GPU library.  Decoding uses torch's own
float8 / bfloat16 conversions and the e2m1 value table of the OCP
Microscaling (MX) format definition; attention uses torch's softmax in
float64 over a dense, explicitly masked key sequence.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import OracleProblem

# OCP MX specification, FP4 E2M1 element encoding: codes 0..7 are the
# magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def problem_of(cfg, sm_scale=0.0) -> OracleProblem:
    return OracleProblem(cfg.batch, cfg.query_len, cfg.num_q_heads, cfg.num_kv_heads,
                         cfg.num_idx_heads, cfg.max_blocks, cfg.kv_dtype, cfg.idx_dtype,
                         topk=cfg.topk, sm_scale=sm_scale)


def decode_bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def decode_e4m3(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def decode_kv(kind: str, pool: np.ndarray, scale) -> np.ndarray:
    """Dense float64 values [NB, Hkv, 128, 128] of a K or V pool."""
    if kind == "bf16":
        return decode_bf16(pool)
    if kind == "fp8":
        return decode_e4m3(pool) * scale.astype(np.float64)[..., None]
    lo = pool & 0xF
    hi = pool >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*pool.shape[:-1], pool.shape[-1] * 2)
    vals = np.asarray(E2M1_TABLE, dtype=np.float64)[codes]
    s = decode_e4m3(scale)  # [..., D/16]
    return vals * np.repeat(s, 16, axis=-1)


def decode_idx(kind: str, pool: np.ndarray, scale=None) -> np.ndarray:
    """Dense float64 index keys [NB, Hidx, 128, 64]; 4-bit keys use the same
    packing and per-16 E4M3 scales as 4-bit K / V."""
    if kind == "nvfp4":
        return decode_kv("nvfp4", pool, scale)
    return decode_bf16(pool) if kind == "bf16" else decode_e4m3(pool)


def logical(pool: np.ndarray, block_table_row: np.ndarray, nblk: int, L: int) -> np.ndarray:
    """[NB, H, 128, X] pool -> [H, L, X] logical token sequence of one request."""
    blocks = pool[block_table_row[:nblk]]                 # [nblk, H, 128, X]
    seq = np.transpose(blocks, (1, 0, 2, 3)).reshape(blocks.shape[1], nblk * 128, -1)
    return seq[:, :L]


def token_scores(cfg, h, b, t) -> np.ndarray:
    """Per-token index scores of row (b, t) over its causal tokens [p + 1]."""
    L = int(h["ctx_lens"][b])
    nblk = -(-L // 128)
    T = cfg.query_len
    p = L - T + t
    ik = logical(decode_idx(cfg.idx_dtype, h["idx_k_pool"], h.get("idx_k_scale")),
                 h["block_table"][b], nblk, L)
    iq = decode_bf16(h["idx_q"][b * T + t])               # [Hidx, 64]
    s = np.einsum("hd,hld->l", iq, ik)                     # sum over heads and dims
    return s[:p + 1]


def brute_force_select(scores_blocks: np.ndarray, local: int, topk: int) -> list:
    """Selection by Python's sorted() on (-score, id)."""
    if local + 1 <= topk:
        return list(range(local + 1))
    cand = sorted(range(local), key=lambda c: (-scores_blocks[c], c))[:topk - 1]
    return sorted(cand + [local])


def dense_attention(cfg, h, b, t, allowed_blocks=None, sm_scale=None) -> np.ndarray:
    """softmax(q K^T * scale) V over the row's causal tokens (optionally only
    tokens of `allowed_blocks`), float64 torch; returns [Hq, 128]."""
    L = int(h["ctx_lens"][b])
    nblk = -(-L // 128)
    T = cfg.query_len
    p = L - T + t
    K = logical(decode_kv(cfg.kv_dtype, h["k_pool"], h["k_scale"]), h["block_table"][b], nblk, L)
    V = logical(decode_kv(cfg.kv_dtype, h["v_pool"], h["v_scale"]), h["block_table"][b], nblk, L)
    q = decode_bf16(h["q"][b * T + t])                    # [Hq, 128]
    Kt = torch.from_numpy(K)
    Vt = torch.from_numpy(V)
    qt = torch.from_numpy(q)
    group = cfg.num_q_heads // cfg.num_kv_heads
    Kh = Kt.repeat_interleave(group, dim=0)               # [Hq, L, 128]
    Vh = Vt.repeat_interleave(group, dim=0)
    scale = sm_scale if sm_scale else 1.0 / np.sqrt(128.0)
    z = torch.einsum("hd,hld->hl", qt, Kh) * scale
    mask = torch.zeros(L, dtype=torch.bool)
    mask[:p + 1] = True
    if allowed_blocks is not None:
        allow = torch.zeros(L, dtype=torch.bool)
        for c in allowed_blocks:
            allow[c * 128:(c + 1) * 128] = True
        mask &= allow
    z = z.masked_fill(~mask, float("-inf"))
    w = torch.softmax(z, dim=-1)
    return torch.einsum("hl,hld->hd", w, Vh).numpy()
