"""ctypes wrapper around the plain C oracle (``msa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke entry and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports this
module and this module never imports the GPU library.

Every function takes host numpy arrays in the layouts of the GPU boundary
(bf16 values travel as their uint16 bit patterns, fp8 / 4-bit data as uint8
codes) and returns numpy arrays.  ``rows`` selects a subset of query rows
(row r = b * T + t); the outputs are in that order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")

KV_DTYPES = {"bf16": 0, "fp8": 1, "nvfp4": 2}
IDX_DTYPES = {"bf16": 0, "fp8": 1, "nvfp4": 2}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into ``libmsa_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("query_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_idx_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("idx_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
    ]


@dataclass
class OracleProblem:
    batch: int
    query_len: int
    num_q_heads: int
    num_kv_heads: int
    num_idx_heads: int
    max_blocks: int
    kv_dtype: str = "bf16"
    idx_dtype: str = "bf16"
    head_dim: int = 128
    idx_dim: int = 64
    block_size: int = 128
    page_size: int = 16
    topk: int = 16
    sm_scale: float = 0.0

    def c(self) -> _Problem:
        return _Problem(self.batch, self.query_len, self.num_q_heads, self.num_kv_heads,
                        self.num_idx_heads, self.head_dim, self.idx_dim, self.block_size,
                        self.page_size, self.topk, self.max_blocks,
                        KV_DTYPES[self.kv_dtype], IDX_DTYPES[self.idx_dtype], self.sm_scale)


_lib = None


def lib():
    global _lib
    if _lib is None:
        # MSA_ORACLE_LIB: another build of the same source (the sanitizer test)
        path = os.environ.get("MSA_ORACLE_LIB") or (_LIB if os.path.exists(_LIB) else build())
        L = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        pp = ctypes.POINTER(_Problem)
        L.msa_oracle_bf16_to_double.restype = ctypes.c_double
        L.msa_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.msa_oracle_e4m3_to_double.restype = ctypes.c_double
        L.msa_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.msa_oracle_e2m1_to_double.restype = ctypes.c_double
        L.msa_oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
        L.msa_oracle_index_scores.argtypes = [pp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp]
        L.msa_oracle_select.argtypes = [pp, vp, vp, vp, ctypes.c_int32, vp, vp]
        L.msa_oracle_page_table.argtypes = [pp, vp, vp, vp, ctypes.c_int32, vp]
        L.msa_oracle_attention.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_int32, vp]
        L.msa_oracle_num_threads.restype = ctypes.c_int
        L.msa_oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.msa_oracle_set_num_threads.restype = None
        L.msa_oracle_f32_to_e4m3.restype = ctypes.c_uint8
        L.msa_oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.msa_oracle_f32_to_e2m1.restype = ctypes.c_uint8
        L.msa_oracle_f32_to_e2m1.argtypes = [ctypes.c_float]
        L.msa_oracle_insert.argtypes = [pp] + [vp] * 11
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _rows(prob: OracleProblem, rows):
    if rows is None:
        return None, prob.batch * prob.query_len
    rows = _c(rows, np.int32)
    return rows, int(rows.shape[0])


def bf16_to_double(bits: int) -> float:
    return lib().msa_oracle_bf16_to_double(bits)


def e4m3_to_double(code: int) -> float:
    return lib().msa_oracle_e4m3_to_double(code)


def e2m1_to_double(nibble: int) -> float:
    return lib().msa_oracle_e2m1_to_double(nibble)


def index_scores(prob, idx_q, idx_k_pool, block_table, ctx_lens, rows=None, *,
                 idx_k_scale=None):
    """Block scores [nrows, max_blocks] (float64, -inf past the local block).
    4-bit index keys (idx_dtype "nvfp4") need `idx_k_scale`, the E4M3 code of
    every group of 16 dims."""
    rows, n = _rows(prob, rows)
    idx_q = _c(idx_q, np.uint16)
    idx_k_pool = _c(idx_k_pool, np.uint16 if prob.idx_dtype == "bf16" else np.uint8)
    if prob.idx_dtype == "nvfp4":
        if idx_k_scale is None:
            raise ValueError("4-bit index keys need idx_k_scale")
        idx_k_scale = _c(idx_k_scale, np.uint8)
    else:
        idx_k_scale = None
    block_table = _c(block_table, np.int32)
    ctx_lens = _c(ctx_lens, np.int32)
    out = np.empty((n, prob.max_blocks), dtype=np.float64)
    p = prob.c()
    lib().msa_oracle_index_scores(ctypes.byref(p), _ptr(idx_q), _ptr(idx_k_pool),
                                  _ptr(idx_k_scale), _ptr(block_table), _ptr(ctx_lens),
                                  _ptr(rows), n, _ptr(out))
    return out


def select(prob, scores, ctx_lens, rows=None):
    """(selected [nrows, topk] int32 ascending, -1 padded; n_selected [nrows])."""
    rows, n = _rows(prob, rows)
    scores = _c(scores, np.float64)
    ctx_lens = _c(ctx_lens, np.int32)
    sel = np.empty((n, prob.topk), dtype=np.int32)
    nsel = np.empty((n,), dtype=np.int32)
    p = prob.c()
    lib().msa_oracle_select(ctypes.byref(p), _ptr(scores), _ptr(ctx_lens), _ptr(rows), n,
                            _ptr(sel), _ptr(nsel))
    return sel, nsel


def page_table(prob, selected, block_table, rows=None):
    """Page table [nrows, topk * block_size / page_size] int32, -1 padded."""
    rows, n = _rows(prob, rows)
    selected = _c(selected, np.int32)
    block_table = _c(block_table, np.int32)
    ppb = prob.block_size // prob.page_size
    out = np.empty((n, prob.topk * ppb), dtype=np.int32)
    p = prob.c()
    lib().msa_oracle_page_table(ctypes.byref(p), _ptr(selected), _ptr(block_table),
                                _ptr(rows), n, _ptr(out))
    return out


def attention(prob, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, selected,
              rows=None):
    """Attention output [nrows, Hq, head_dim] float64 over the selected blocks."""
    rows, n = _rows(prob, rows)
    kv_np = np.uint16 if prob.kv_dtype == "bf16" else np.uint8
    q = _c(q, np.uint16)
    k_pool = _c(k_pool, kv_np)
    v_pool = _c(v_pool, kv_np)
    sc_np = np.float32 if prob.kv_dtype == "fp8" else np.uint8
    k_scale = _c(k_scale, sc_np)
    v_scale = _c(v_scale, sc_np)
    block_table = _c(block_table, np.int32)
    ctx_lens = _c(ctx_lens, np.int32)
    selected = _c(selected, np.int32)
    out = np.empty((n, prob.num_q_heads, prob.head_dim), dtype=np.float64)
    p = prob.c()
    lib().msa_oracle_attention(ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                               _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                               _ptr(ctx_lens), _ptr(selected), _ptr(rows), n, _ptr(out))
    return out


def decode(prob, q, idx_q, k_pool, v_pool, k_scale, v_scale, idx_k_pool, block_table,
           ctx_lens, rows=None, *, idx_k_scale=None):
    """The whole path for the given rows: dict of scores, selected, n_selected,
    page_table and out."""
    s = index_scores(prob, idx_q, idx_k_pool, block_table, ctx_lens, rows,
                     idx_k_scale=idx_k_scale)
    sel, nsel = select(prob, s, ctx_lens, rows)
    pt = page_table(prob, sel, block_table, rows)
    out = attention(prob, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, sel, rows)
    return {"scores": s, "selected": sel, "n_selected": nsel, "page_table": pt, "out": out}


def f32_to_e4m3(x: float) -> int:
    return int(lib().msa_oracle_f32_to_e4m3(x))


def f32_to_e2m1(x: float) -> int:
    return int(lib().msa_oracle_f32_to_e2m1(x))


def insert(prob, k_new, v_new, idx_new, block_table, ctx_lens, pools):
    """Write the T new tokens of every request into `pools` (a dict of host
    arrays k_pool, v_pool, k_scale, v_scale, idx_k_pool, idx_k_scale in the
    attention's layouts, modified in place), quantised to the pools'
    formats.  k_new / v_new [R, Hkv, 128] and idx_new [R, Hidx, 64] are bf16
    bit patterns (uint16)."""
    for name in ("k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool", "idx_k_scale"):
        a = pools.get(name)
        if a is not None and not a.flags["C_CONTIGUOUS"]:
            raise ValueError(f"{name} must be C-contiguous (it is written in place)")
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    idx_new = _c(idx_new, np.uint16)
    block_table = _c(block_table, np.int32)
    ctx_lens = _c(ctx_lens, np.int32)
    p = prob.c()
    lib().msa_oracle_insert(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(idx_new),
                            _ptr(block_table), _ptr(ctx_lens),
                            *(_ptr(pools.get(n)) for n in ("k_pool", "v_pool", "k_scale",
                                                           "v_scale", "idx_k_pool",
                                                           "idx_k_scale")))


def num_threads() -> int:
    return int(lib().msa_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Worker threads of the oracle's parallel loops (1: a single core)."""
    lib().msa_oracle_set_num_threads(int(n))
