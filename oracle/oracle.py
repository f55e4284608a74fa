"""Python face of the CPU oracle (``libkpool_oracle.so``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the product path never does. It shares no code with the
HIP library. Each wrapper below calls one C function of ``kpool_oracle.c``,
whose comments cite the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        P = C.c_void_p
        i32, i64, f32 = C.c_int32, C.c_int64, C.c_float
        L.kpo_layout.argtypes = [P, i32, i32, i32, P, P]
        L.kpo_layout.restype = i32
        L.kpo_query_info.argtypes = [P, i32, P, i32, i32, P, P, P]
        L.kpo_query_info.restype = i32
        L.kpo_pool.argtypes = [P, P, P, P, i32, i32, i32, P]
        L.kpo_pool.restype = None
        L.kpo_fwht.argtypes = [P, i32]
        L.kpo_fwht.restype = None
        L.kpo_e4m3_encode.argtypes = [f32]
        L.kpo_e4m3_encode.restype = C.c_uint8
        L.kpo_e4m3_decode.argtypes = [C.c_uint8]
        L.kpo_e4m3_decode.restype = f32
        L.kpo_quant_rows.argtypes = [P, i64, i32, P, P]
        L.kpo_quant_rows.restype = None
        L.kpo_keys.argtypes = [P, P, P, P, i32, i32, i32, P, P, P]
        L.kpo_keys.restype = None
        L.kpo_queries.argtypes = [P, i32, i32, i32, P, P]
        L.kpo_queries.restype = None
        L.kpo_scores.argtypes = [P, i32, P, i32, P, i32, i32, P, P, P, P, P, P, i32, P, i32, i32, P]
        L.kpo_scores.restype = None
        L.kpo_topk.argtypes = [P, i32, P, i32, P, i32, i32, P, i32, i32, P, P]
        L.kpo_topk.restype = None
        L.kpo_sparse_mla.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, P, P, P]
        L.kpo_sparse_mla.restype = None
        L.kpo_sparse_mla_dv.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f32, P, P, P]
        L.kpo_sparse_mla_dv.restype = None
        L.kpo_sparse_mla_bwd.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f32, P, P]
        L.kpo_sparse_mla_bwd.restype = None
        L.kpo_num_threads.argtypes = []
        L.kpo_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().kpo_num_threads())


# ---------------------------------------------------------------- layout ----
def layout(cu, T: int, kpool: int):
    cu = _c(cu, np.int32)
    B = cu.shape[0] - 1
    cu_pools = np.zeros(B + 1, np.int32)
    pool_start = np.zeros(max(1, T // kpool), np.int32)
    P = lib().kpo_layout(_p(cu), B, T, kpool, _p(cu_pools), _p(pool_start))
    if P < 0:
        raise ValueError("malformed cu_seqlens")
    return cu_pools, pool_start[:P].copy()


def query_info(cu, cu_pools, kpool: int, t: int):
    cu = _c(cu, np.int32)
    cu_pools = _c(cu_pools, np.int32)
    out = np.zeros(3, np.int32)
    d = lib().kpo_query_info(_p(cu), cu.shape[0] - 1, _p(cu_pools), kpool, int(t),
                             _p(out[0:1]), _p(out[1:2]), _p(out[2:3]))
    return int(d), int(out[0]), int(out[1]), int(out[2])


# ---------------------------------------------------------- pool / rotate ---
def pool(k_idx, gate, ape, pool_start, kpool: int):
    k_idx = _c(k_idx, np.uint16)
    gate = _c(gate, np.uint16)
    ape = _c(ape, np.float32)
    pool_start = _c(pool_start, np.int32)
    d = k_idx.shape[1]
    P = pool_start.shape[0]
    out = np.zeros((P, d), np.float32)
    lib().kpo_pool(_p(k_idx), _p(gate), _p(ape), _p(pool_start), P, d, kpool, _p(out))
    return out


def fwht(x):
    """Orthonormal fp32 FWHT along the last axis (returns a new array)."""
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    n = y.shape[-1]
    flat = y.reshape(-1, n)
    for r in range(flat.shape[0]):
        lib().kpo_fwht(_p(flat[r]), n)
    return y


def e4m3_encode(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    L = lib()
    return np.array([L.kpo_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def e4m3_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    L = lib()
    return np.array([L.kpo_e4m3_decode(int(c)) for c in codes.ravel()], dtype=np.float32).reshape(codes.shape)


def quant_rows(x):
    x = _c(x, np.float32)
    n = x.shape[-1]
    rows = x.size // n
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1], np.float32)
    lib().kpo_quant_rows(_p(x), rows, n, _p(codes), _p(scales))
    return codes, scales


def keys(k_idx, gate, ape, pool_start, kpool: int):
    """Pooled, rotated, quantised keys: (codes [P,d] u8, scales [P] f32, pooled [P,d] f32)."""
    k_idx = _c(k_idx, np.uint16)
    gate = _c(gate, np.uint16)
    ape = _c(ape, np.float32)
    pool_start = _c(pool_start, np.int32)
    d = k_idx.shape[1]
    P = pool_start.shape[0]
    codes = np.zeros((P, d), np.uint8)
    scales = np.zeros(P, np.float32)
    pooled = np.zeros((P, d), np.float32)
    lib().kpo_keys(_p(k_idx), _p(gate), _p(ape), _p(pool_start), P, d, kpool,
                   _p(codes), _p(scales), _p(pooled))
    return codes, scales, pooled


def queries(q_idx):
    """Rotated, quantised indexer queries: (codes [Tq,H_I,d] u8, scales [Tq,H_I] f32)."""
    q_idx = _c(q_idx, np.uint16)
    Tq, h, d = q_idx.shape
    codes = np.zeros((Tq, h, d), np.uint8)
    scales = np.zeros((Tq, h), np.float32)
    lib().kpo_queries(_p(q_idx), Tq, h, d, _p(codes), _p(scales))
    return codes, scales


# ---------------------------------------------------------------- scores ----
def scores(cu, cu_pools, kpool, q_pos, max_pools, w, q_codes=None, q_scales=None,
           k_codes=None, k_scales=None, q_rot=None, k_rot=None):
    """Indexer scores [Tq, max_pools] (-inf where not visible). FP8 operands when
    codes are given; unquantised rotated fp32 operands (debug) when q_rot/k_rot are."""
    cu = _c(cu, np.int32)
    cu_pools = _c(cu_pools, np.int32)
    w = _c(w, np.float32)
    Tq, h = w.shape
    mode = 0 if q_codes is not None else 1
    if mode == 0:
        q_codes = _c(q_codes, np.uint8)
        q_scales = _c(q_scales, np.float32)
        k_codes = _c(k_codes, np.uint8)
        k_scales = _c(k_scales, np.float32)
        d = q_codes.shape[-1]
    else:
        q_rot = _c(q_rot, np.float32)
        k_rot = _c(k_rot, np.float32)
        d = q_rot.shape[-1]
    qp = None if q_pos is None else _c(q_pos, np.int32)
    out = np.zeros((Tq, max_pools), np.float32)
    lib().kpo_scores(_p(cu), cu.shape[0] - 1, _p(cu_pools), kpool, _p(qp), Tq, max_pools,
                     _p(q_codes), _p(q_scales), _p(k_codes), _p(k_scales), _p(q_rot), _p(k_rot),
                     mode, _p(w), h, d, _p(out))
    return out


def topk(cu, cu_pools, kpool, q_pos, scores_, topk_, row_width):
    cu = _c(cu, np.int32)
    cu_pools = _c(cu_pools, np.int32)
    scores_ = _c(scores_, np.float32)
    Tq, max_pools = scores_.shape
    qp = None if q_pos is None else _c(q_pos, np.int32)
    idx = np.zeros((Tq, row_width), np.int32)
    nv = np.zeros(Tq, np.int32)
    lib().kpo_topk(_p(cu), cu.shape[0] - 1, _p(cu_pools), kpool, _p(qp), Tq, max_pools,
                   _p(scores_), topk_, row_width, _p(idx), _p(nv))
    return idx, nv


def sparse_mla(q, kv, indices, scale: float, with_abs: bool = False):
    """(out [Tq,H,D] f32, lse [Tq,H] f32) of absorbed sparse MLA over the index rows;
    with_abs adds out_abs = sum_j softmax_j |kv_j| (the error scale of each output)."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    indices = _c(indices, np.int32)
    Tq, H, D = q.shape
    out = np.zeros((Tq, H, D), np.float32)
    lse = np.zeros((Tq, H), np.float32)
    oabs = np.zeros((Tq, H, D), np.float32) if with_abs else None
    lib().kpo_sparse_mla(_p(q), _p(kv), _p(indices), Tq, kv.shape[0], H, D, indices.shape[1],
                         float(scale), _p(out), _p(lse), _p(oabs))
    return (out, lse, oabs) if with_abs else (out, lse)


def sparse_mla_dv(q, kv, indices, scale: float, d_v: int, with_abs: bool = False):
    """Sparse MLA with values narrower than keys: keys are the kv rows (width of
    q), values their first d_v columns. (out [Tq,H,d_v] f32, lse [Tq,H] f32)."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    indices = _c(indices, np.int32)
    Tq, H, D = q.shape
    out = np.zeros((Tq, H, d_v), np.float32)
    lse = np.zeros((Tq, H), np.float32)
    oabs = np.zeros((Tq, H, d_v), np.float32) if with_abs else None
    lib().kpo_sparse_mla_dv(_p(q), _p(kv), _p(indices), Tq, kv.shape[0], H, D, d_v, indices.shape[1],
                            float(scale), _p(out), _p(lse), _p(oabs))
    return (out, lse, oabs) if with_abs else (out, lse)


def sparse_mla_bwd(q, kv, indices, d_out, scale: float):
    """Gradients of sparse_mla / sparse_mla_dv for output gradient d_out
    [Tq,H,d_v] (bf16 bits): (d_q [Tq,H,D] f32, d_kv [N,D] f32)."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    indices = _c(indices, np.int32)
    d_out = _c(d_out, np.uint16)
    Tq, H, D = q.shape
    d_v = d_out.shape[-1]
    dq = np.zeros((Tq, H, D), np.float32)
    dkv = np.zeros(kv.shape, np.float32)
    lib().kpo_sparse_mla_bwd(_p(q), _p(kv), _p(indices), _p(d_out), Tq, kv.shape[0], H, D, d_v,
                             indices.shape[1], float(scale), _p(dq), _p(dkv))
    return dq, dkv


# ------------------------------------------------------------- pipeline -----
def dsa_forward(wl, q_rows: Optional[np.ndarray] = None, with_mla: bool = True):
    """Whole forward of workload ``wl`` (a :class:`workloads.Workload`) for the
    query rows ``q_rows`` (indices into the workload's queries; all by default).
    Returns a dict of every intermediate the GPU path is compared with."""
    s = wl.s
    cu_pools, pool_start = layout(s.cu, s.T, s.kpool)
    ape = wl.ape()
    k_idx = wl.full("k_idx")
    gate = wl.full("gate")
    kc, ks, pooled = keys(k_idx, gate, ape, pool_start, s.kpool)
    qpos_all = s.query_positions()
    if q_rows is None:
        q_rows = np.arange(s.Tq)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    qpos = qpos_all[q_rows].astype(np.int32)
    q_idx = np.concatenate([wl.rows("q_idx", int(r), int(r) + 1) for r in q_rows], axis=0)
    w = np.concatenate([wl.rows("w", int(r), int(r) + 1) for r in q_rows], axis=0)
    qc, qs = queries(q_idx)
    sc = scores(s.cu, cu_pools, s.kpool, qpos, s.max_pools, w, qc, qs, kc, ks)
    idx, nv = topk(s.cu, cu_pools, s.kpool, qpos, sc, s.topk, s.row_width)
    res = dict(cu_pools=cu_pools, pool_start=pool_start, k_codes=kc, k_scales=ks, pooled=pooled,
               q_codes=qc, q_scales=qs, scores=sc, indices=idx, num_valid=nv, q_pos=qpos)
    if with_mla:
        q = np.concatenate([wl.rows("q", int(r), int(r) + 1) for r in q_rows], axis=0)
        kv = wl.full("kv")
        out, lse = sparse_mla(q, kv, idx, s.scale)
        res.update(out=out, lse=lse)
    return res
