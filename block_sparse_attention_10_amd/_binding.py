"""ctypes binding of libmsa (include/msa.h).

Argument marshalling only: every function passes torch device pointers, sizes
and the current HIP stream straight to the C ABI, and raises MSAError on a
non-zero status.  No computation happens here, and there is no fallback: if
libmsa.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# MSA_LIBRARY: another build of the same sources (the host-sanitizer test)
_LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4
MSA_ERR_BAD_DATA = -5

MSA_FLAG_DEBUG_CHECKS = 1

DTYPES = {"bf16": 0, "fp8": 1, "nvfp4": 2}

# Every symbol include/msa.h declares.
EXPORTS = ("msa_index_score", "msa_select_blocks", "msa_build_page_table", "msa_sparse_decode",
           "msa_decode", "msa_workspace_bytes", "msa_status_string", "msa_last_hip_error",
           "msa_last_dispatch", "msa_selftest_decoders", "msa_insert_kv",
           "msa_last_check_failure", "msa_decode_noalloc")

MSA_NOALLOC_SCRATCH_BYTES = 16 << 20


class MSAError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        msg = _lib.msa_status_string(status).decode()
        if status == MSA_ERR_HIP:
            msg += f" (hip error {_lib.msa_last_hip_error()})"
        if status == MSA_ERR_BAD_DATA:
            msg += f" ({msa_last_check_failure()})"
        super().__init__(f"{fn}: {msg} [{status}]")


class Problem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("decode_query_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_idx_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("local_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_phys_blocks", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("idx_k_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class Pools(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool", "idx_k_scale")]


class Tensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "idx_q", "k_pool", "v_pool", "k_scale", "v_scale", "idx_k_pool",
                 "block_table", "ctx_lens", "idx_k_scale")]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python block_sparse_attention_10_amd/build.py")
    L = ctypes.CDLL(_LIB_PATH)
    vp, pp, tp = ctypes.c_void_p, ctypes.POINTER(Problem), ctypes.POINTER(Tensors)
    sz = ctypes.c_size_t
    for name, args in (
            ("msa_index_score", [pp, tp, vp, vp]),
            ("msa_select_blocks", [pp, vp, vp, vp, vp, vp]),
            ("msa_build_page_table", [pp, vp, vp, vp, vp]),
            ("msa_sparse_decode", [pp, tp, vp, vp, vp, sz, vp]),
            ("msa_decode", [pp, tp, vp, vp, vp, vp, sz, vp]),
            ("msa_decode_noalloc", [pp, tp, vp, vp, vp, vp]),
            ("msa_selftest_decoders", [vp, vp]),
            ("msa_insert_kv", [pp, ctypes.POINTER(Pools), vp, vp, vp, vp, vp, vp])):
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.msa_workspace_bytes.argtypes = [pp]
    L.msa_workspace_bytes.restype = sz
    L.msa_status_string.argtypes = [ctypes.c_int]
    L.msa_status_string.restype = ctypes.c_char_p
    L.msa_last_hip_error.argtypes = []
    L.msa_last_hip_error.restype = ctypes.c_int
    L.msa_last_dispatch.argtypes = [ctypes.c_char_p, sz]
    L.msa_last_dispatch.restype = ctypes.c_int
    L.msa_last_check_failure.argtypes = [ctypes.c_char_p, sz]
    L.msa_last_check_failure.restype = ctypes.c_int
    return L


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def lib():
    return _lib


def problem(batch, decode_query_len, num_q_heads, num_kv_heads, num_idx_heads,
            max_blocks_per_seq, num_phys_blocks, kv_dtype="bf16", idx_k_dtype="bf16", topk=16,
            sm_scale=0.0, head_dim=128, idx_dim=64, block_size=128, page_size=16,
            local_blocks=1, flags=0) -> Problem:
    return Problem(ctypes.sizeof(Problem), batch, decode_query_len, num_q_heads, num_kv_heads,
                   num_idx_heads, head_dim, idx_dim, block_size, page_size, topk, local_blocks,
                   max_blocks_per_seq, num_phys_blocks, DTYPES[kv_dtype], DTYPES[idx_k_dtype],
                   sm_scale, flags)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def tensors(q=None, idx_q=None, k_pool=None, v_pool=None, k_scale=None, v_scale=None,
            idx_k_pool=None, block_table=None, ctx_lens=None, idx_k_scale=None) -> Tensors:
    return Tensors(*(None if t is None else t.data_ptr() for t in
                     (q, idx_q, k_pool, v_pool, k_scale, v_scale, idx_k_pool, block_table,
                      ctx_lens, idx_k_scale)))


def describe(q, idx_q, k_pool, v_pool, k_scale, v_scale, idx_k_pool, block_table, ctx_lens,
             decode_query_len=1, topk=16, sm_scale=0.0, idx_k_scale=None, flags=0):
    """(Problem, Tensors) for device tensors in the boundary's layouts; the
    dimensions and dtypes are read from the tensor shapes (index keys with an
    idx_k_scale pool are 4-bit)."""
    B = int(ctx_lens.shape[0])
    if k_pool.dtype == torch.bfloat16:
        kv = "bf16"
    elif k_scale is not None and k_scale.dtype == torch.float32:
        kv = "fp8"
    else:
        kv = "nvfp4"
    if idx_k_pool.dtype == torch.bfloat16:
        idx = "bf16"
    else:
        idx = "nvfp4" if idx_k_scale is not None else "fp8"
    p = problem(B, decode_query_len, int(q.shape[1]), int(k_pool.shape[1]),
                int(idx_k_pool.shape[1]), int(block_table.shape[1]), int(k_pool.shape[0]),
                kv_dtype=kv, idx_k_dtype=idx, topk=topk, sm_scale=sm_scale, flags=flags)
    t = tensors(q, idx_q, k_pool, v_pool, k_scale, v_scale, idx_k_pool, block_table, ctx_lens,
                idx_k_scale)
    return p, t


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, fn: str):
    if status != MSA_OK:
        raise MSAError(status, fn)


def pools(k_pool, v_pool, k_scale, v_scale, idx_k_pool, idx_k_scale=None) -> Pools:
    return Pools(*(None if t is None else t.data_ptr() for t in
                   (k_pool, v_pool, k_scale, v_scale, idx_k_pool, idx_k_scale)))


def msa_insert_kv(p: Problem, pl: Pools, block_table, ctx_lens, k_new, v_new, idx_k_new,
                  stream=None):
    _check(_lib.msa_insert_kv(ctypes.byref(p), ctypes.byref(pl), _p(block_table), _p(ctx_lens),
                              _p(k_new), _p(v_new), _p(idx_k_new), _stream(stream)),
           "msa_insert_kv")


def msa_index_score(p: Problem, t: Tensors, block_scores, stream=None):
    _check(_lib.msa_index_score(ctypes.byref(p), ctypes.byref(t), _p(block_scores),
                                _stream(stream)), "msa_index_score")


def msa_select_blocks(p: Problem, block_scores, ctx_lens, selected, n_selected, stream=None):
    _check(_lib.msa_select_blocks(ctypes.byref(p), _p(block_scores), _p(ctx_lens), _p(selected),
                                  _p(n_selected), _stream(stream)), "msa_select_blocks")


def msa_build_page_table(p: Problem, selected, block_table, page_table, stream=None):
    _check(_lib.msa_build_page_table(ctypes.byref(p), _p(selected), _p(block_table),
                                     _p(page_table), _stream(stream)), "msa_build_page_table")


def msa_sparse_decode(p: Problem, t: Tensors, page_table, out, workspace, stream=None):
    _check(_lib.msa_sparse_decode(ctypes.byref(p), ctypes.byref(t), _p(page_table), _p(out),
                                  _p(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)), "msa_sparse_decode")


def msa_decode(p: Problem, t: Tensors, selected, page_table, out, workspace, stream=None):
    _check(_lib.msa_decode(ctypes.byref(p), ctypes.byref(t), _p(selected), _p(page_table),
                           _p(out), _p(workspace), workspace.numel() * workspace.element_size(),
                           _stream(stream)), "msa_decode")


def msa_decode_noalloc(p: Problem, t: Tensors, selected, page_table, out, stream=None):
    _check(_lib.msa_decode_noalloc(ctypes.byref(p), ctypes.byref(t), _p(selected),
                                   _p(page_table), _p(out), _stream(stream)),
           "msa_decode_noalloc")


def msa_workspace_bytes(p: Problem) -> int:
    return int(_lib.msa_workspace_bytes(ctypes.byref(p)))


def msa_status_string(status: int) -> str:
    return _lib.msa_status_string(status).decode()


def msa_last_hip_error() -> int:
    return int(_lib.msa_last_hip_error())


def msa_last_dispatch() -> str:
    n = _lib.msa_last_dispatch(None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    _lib.msa_last_dispatch(buf, n + 1)
    return buf.value.decode()


def msa_last_check_failure() -> str:
    n = _lib.msa_last_check_failure(None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    _lib.msa_last_check_failure(buf, n + 1)
    return buf.value.decode()


def msa_selftest_decoders(out, stream=None):
    _check(_lib.msa_selftest_decoders(_p(out), _stream(stream)), "msa_selftest_decoders")
