"""ctypes binding of libkpool.so: the C ABI of include/kpool.h with torch
tensors for device memory and the current torch stream.

Argument marshalling only: each wrapper checks dtypes, devices and shapes,
allocates its outputs with ``torch.empty`` and calls one C entry point. Every
step of the computation runs in the HIP kernels. There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkpool.so")

KP_OK, KP_ERR_INVALID_ARG, KP_ERR_UNSUPPORTED, KP_ERR_HIP = 0, 1, 2, 3
_STATUS = {0: "KP_OK", 1: "KP_ERR_INVALID_ARG", 2: "KP_ERR_UNSUPPORTED", 3: "KP_ERR_HIP"}

# (name, restype, argtypes) of every exported entry point, in header order.
_P, _I, _F, _Z = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
SIGNATURES = [
    ("kp_last_error", C.c_char_p, []),
    ("kp_version", _I, []),
    ("kp_row_width", _I, [_I, _I]),
    ("kpool_build", _I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P]),
    ("kpool_build_from", _I, [_P, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    ("indexer_rotate_quant", _I, [_P, _I, _I, _I, _P, _P, _P]),
    ("kp_indexer_workspace_bytes", _Z, [_I, _I, _I, _I, _I]),
    ("indexer_score_topk", _I, [_P, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I,
                                _P, _P, _P, _P, _Z, _P]),
    ("indexer_score_topk_noalloc", _I, [_P, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I,
                                        _P, _P, _P, _P]),
    ("kpool_update_paged", _I, [_P, _I, _P, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P, _P]),
    ("kp_indexer_paged_workspace_bytes", _Z, [_I, _I, _I, _I]),
    ("indexer_score_topk_paged", _I, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I,
                                      _P, _P, _P, _P, _Z, _P]),
    ("indexer_topk_from_scores", _I, [_P, _I, _I, _P, _I, _P, _I, _P, _I, _I, _I, _P, _P, _P]),
    ("kp_mla_fwd_workspace_bytes", _Z, [_I, _I, _I, _I]),
    ("sparse_mla_fwd", _I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _Z, _P]),
    ("kp_mla_bwd_workspace_bytes", _Z, [_I, _I, _I]),
    ("sparse_mla_bwd", _I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _Z, _P]),
    ("kp_check_inputs", _I, [_P, _I, _I, _P, _I, _P]),
]


class KpoolError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libkpool.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_kpool_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != KP_OK:
        raise KpoolError(status, lib().kp_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape) -> None:
    """dtype, rank and shape of one tensor argument (``shape`` holds None for a
    dimension checked elsewhere); devices and contiguity are checked by _on."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape):
        raise ValueError(f"{name} must have {len(shape)} dims, got shape {tuple(t.shape)}")
    for got, want in zip(t.shape, shape):
        if want is not None and got != want:
            want_s = tuple("*" if w is None else w for w in shape)
            raise ValueError(f"{name} must have shape {want_s}, got {tuple(t.shape)}")


def _on(*named) -> torch.device:
    """Every (name, tensor) pair (None tensors skipped) is a contiguous tensor on
    one and the same GPU; returns that device. Runs after the shape checks, so a
    shape mismatch is reported whatever the device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return dev


# ------------------------------------------------------------------ helpers ---
def kp_row_width(kpool: int, topk_pools: int) -> int:
    return int(lib().kp_row_width(kpool, topk_pools))


def kp_version() -> int:
    return int(lib().kp_version())


def kp_indexer_workspace_bytes(num_q: int, max_pools: int, h_idx: int, d_idx: int, topk_pools: int) -> int:
    return int(lib().kp_indexer_workspace_bytes(num_q, max_pools, h_idx, d_idx, topk_pools))


def kp_indexer_paged_workspace_bytes(num_q: int, num_docs: int, h_idx: int, d_idx: int) -> int:
    return int(lib().kp_indexer_paged_workspace_bytes(num_q, num_docs, h_idx, d_idx))


# -------------------------------------------------------------- entry points --
def kpool_build(cu_seqlens: torch.Tensor, k_idx: torch.Tensor, gate: torch.Tensor, ape: torch.Tensor,
                kpool: int = 4, with_f32: bool = False):
    """Pool layout and rotated FP8 pooled keys.
    Returns (cu_pools, pool_start, pooled_k_fp8, pooled_k_scale, pooled_k_f32 or None)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    _need(k_idx, "k_idx", torch.bfloat16, (None, None))
    T, d = k_idx.shape
    _need(gate, "gate", torch.bfloat16, (T, d))
    _need(ape, "ape", torch.float32, (kpool, d))
    B = cu_seqlens.shape[0] - 1
    dev = _on(("cu_seqlens", cu_seqlens), ("k_idx", k_idx), ("gate", gate), ("ape", ape))
    cap = T // kpool
    cu_pools = torch.empty(B + 1, dtype=torch.int32, device=dev)
    pool_start = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)[:cap]
    k8 = torch.empty((max(cap, 1), d), dtype=torch.uint8, device=dev)[:cap]
    ks = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)[:cap]
    kf = torch.empty((max(cap, 1), d), dtype=torch.float32, device=dev)[:cap] if with_f32 else None
    _check(lib().kpool_build(_ptr(cu_seqlens), B, T, _ptr(k_idx), _ptr(gate), _ptr(ape), d, kpool,
                             _ptr(cu_pools), _ptr(pool_start), _ptr(k8), _ptr(ks), _ptr(kf), _stream(dev)))
    return cu_pools, pool_start, k8, ks, kf


def kpool_build_from(cu_seqlens: torch.Tensor, k_idx: torch.Tensor, gate: torch.Tensor, ape: torch.Tensor,
                     token_lo: int, out, kpool: int = 4) -> None:
    """kpool_build for the pools ending at or after token_lo, into `out` =
    (cu_pools, pool_start, pooled_k_fp8, pooled_k_scale, pooled_k_f32 or None),
    the tensors of an earlier kpool_build over the same documents (the pooled-key
    cache); the rows of pools ending before token_lo are left as they are."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    _need(k_idx, "k_idx", torch.bfloat16, (None, None))
    T, d = k_idx.shape
    _need(gate, "gate", torch.bfloat16, (T, d))
    _need(ape, "ape", torch.float32, (kpool, d))
    B = cu_seqlens.shape[0] - 1
    cap = T // kpool
    cu_pools, pool_start, k8, ks, kf = out
    _need(cu_pools, "cu_pools", torch.int32, (B + 1,))
    _need(pool_start, "pool_start", torch.int32, (cap,))
    _need(k8, "pooled_k_fp8", torch.uint8, (cap, d))
    _need(ks, "pooled_k_scale", torch.float32, (cap,))
    if kf is not None:
        _need(kf, "pooled_k_f32", torch.float32, (cap, d))
    _on(("cu_seqlens", cu_seqlens), ("k_idx", k_idx), ("gate", gate), ("ape", ape), ("cu_pools", cu_pools),
        ("pool_start", pool_start), ("pooled_k_fp8", k8), ("pooled_k_scale", ks), ("pooled_k_f32", kf))
    _check(lib().kpool_build_from(_ptr(cu_seqlens), B, T, _ptr(k_idx), _ptr(gate), _ptr(ape), d, kpool,
                                  int(token_lo), _ptr(cu_pools), _ptr(pool_start), _ptr(k8), _ptr(ks), _ptr(kf),
                                  _stream(k_idx.device)))


def indexer_rotate_quant(q_idx: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rotated FP8 indexer queries: (codes uint8 [Tq,H_I,D_I], scales f32 [Tq,H_I])."""
    _need(q_idx, "q_idx", torch.bfloat16, (None, None, None))
    _on(("q_idx", q_idx))
    Tq, h, d = q_idx.shape
    codes = torch.empty((Tq, h, d), dtype=torch.uint8, device=q_idx.device)
    scales = torch.empty((Tq, h), dtype=torch.float32, device=q_idx.device)
    _check(lib().indexer_rotate_quant(_ptr(q_idx), Tq, h, d, _ptr(codes), _ptr(scales), _stream(q_idx.device)))
    return codes, scales


def indexer_score_topk(cu_seqlens: torch.Tensor, cu_pools: torch.Tensor, pooled_k_fp8: torch.Tensor,
                       pooled_k_scale: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor,
                       num_tokens: int, kpool: int = 4, topk_pools: int = 512,
                       row_width: Optional[int] = None, q_pos: Optional[torch.Tensor] = None,
                       return_scores: bool = False, workspace: Optional[torch.Tensor] = None):
    """FP8 indexer scoring and top-k index rows.
    Returns (indices int32 [Tq,W], num_valid int32 [Tq], scores f32 [Tq,max_pools] or None)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    B = cu_seqlens.shape[0] - 1
    _need(q_idx, "q_idx", torch.bfloat16, (None, None, None))
    Tq, h, d = q_idx.shape
    max_pools = num_tokens // kpool
    _need(cu_pools, "cu_pools", torch.int32, (B + 1,))
    _need(pooled_k_fp8, "pooled_k_fp8", torch.uint8, (max_pools, d))
    _need(pooled_k_scale, "pooled_k_scale", torch.float32, (max_pools,))
    _need(w_idx, "w_idx", torch.float32, (Tq, h))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (Tq,))
    elif Tq != num_tokens:
        raise ValueError(f"without q_pos every token is a query: q_idx must have {num_tokens} rows, got {Tq}")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, (None,))
    dev = _on(("cu_seqlens", cu_seqlens), ("cu_pools", cu_pools), ("pooled_k_fp8", pooled_k_fp8),
              ("pooled_k_scale", pooled_k_scale), ("q_idx", q_idx), ("w_idx", w_idx), ("q_pos", q_pos),
              ("workspace", workspace))
    W = row_width if row_width is not None else kp_row_width(kpool, topk_pools)
    indices = torch.empty((Tq, W), dtype=torch.int32, device=dev)
    num_valid = torch.empty(Tq, dtype=torch.int32, device=dev)
    scores = torch.empty((Tq, max_pools), dtype=torch.float32, device=dev) if return_scores else None
    need = kp_indexer_workspace_bytes(Tq, max_pools, h, d, topk_pools)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().indexer_score_topk(_ptr(cu_seqlens), cu_seqlens.shape[0] - 1, num_tokens, _ptr(cu_pools),
                                    max_pools, _ptr(pooled_k_fp8), _ptr(pooled_k_scale), _ptr(q_pos), Tq,
                                    _ptr(q_idx), _ptr(w_idx), h, d, kpool, topk_pools, W, _ptr(indices),
                                    _ptr(num_valid), _ptr(scores), _ptr(workspace), workspace.numel(),
                                    _stream(dev)))
    return indices, num_valid, scores


def indexer_score_topk_noalloc(cu_seqlens: torch.Tensor, cu_pools: torch.Tensor, pooled_k_fp8: torch.Tensor,
                               pooled_k_scale: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor,
                               num_tokens: int, kpool: int = 4, topk_pools: int = 512,
                               row_width: Optional[int] = None, q_pos: Optional[torch.Tensor] = None,
                               out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                               return_scores: bool = False):
    """indexer_score_topk with the library's own device scratch as its workspace
    (no workspace argument). ``out`` = (indices, num_valid) to write into
    caller tensors (e.g. inside graph capture, where this call allocates
    nothing). Returns (indices, num_valid, scores or None)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    B = cu_seqlens.shape[0] - 1
    _need(q_idx, "q_idx", torch.bfloat16, (None, None, None))
    Tq, h, d = q_idx.shape
    max_pools = num_tokens // kpool
    _need(cu_pools, "cu_pools", torch.int32, (B + 1,))
    _need(pooled_k_fp8, "pooled_k_fp8", torch.uint8, (max_pools, d))
    _need(pooled_k_scale, "pooled_k_scale", torch.float32, (max_pools,))
    _need(w_idx, "w_idx", torch.float32, (Tq, h))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (Tq,))
    elif Tq != num_tokens:
        raise ValueError(f"without q_pos every token is a query: q_idx must have {num_tokens} rows, got {Tq}")
    W = row_width if row_width is not None else kp_row_width(kpool, topk_pools)
    if out is not None:
        _need(out[0], "indices", torch.int32, (Tq, W))
        _need(out[1], "num_valid", torch.int32, (Tq,))
    dev = _on(("cu_seqlens", cu_seqlens), ("cu_pools", cu_pools), ("pooled_k_fp8", pooled_k_fp8),
              ("pooled_k_scale", pooled_k_scale), ("q_idx", q_idx), ("w_idx", w_idx), ("q_pos", q_pos),
              ("indices", None if out is None else out[0]), ("num_valid", None if out is None else out[1]))
    if out is None:
        indices = torch.empty((Tq, W), dtype=torch.int32, device=dev)
        num_valid = torch.empty(Tq, dtype=torch.int32, device=dev)
    else:
        indices, num_valid = out
    scores = torch.empty((Tq, max_pools), dtype=torch.float32, device=dev) if return_scores else None
    _check(lib().indexer_score_topk_noalloc(_ptr(cu_seqlens), B, num_tokens, _ptr(cu_pools), max_pools,
                                            _ptr(pooled_k_fp8), _ptr(pooled_k_scale), _ptr(q_pos), Tq,
                                            _ptr(q_idx), _ptr(w_idx), h, d, kpool, topk_pools, W, _ptr(indices),
                                            _ptr(num_valid), _ptr(scores), _stream(dev)))
    return indices, num_valid, scores


def kpool_update_paged(cu_seqlens: torch.Tensor, page_table: torch.Tensor, k_idx_pages: torch.Tensor,
                       gate_pages: torch.Tensor, ape: torch.Tensor, k8_pages: torch.Tensor, sk_pages: torch.Tensor,
                       last_tokens: int, kpool: int = 4) -> None:
    """Pool, rotate and quantise into a paged cache the pools whose last token is
    among each document's last ``last_tokens`` tokens (writes k8_pages, sk_pages)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    B = cu_seqlens.shape[0] - 1
    _need(page_table, "page_table", torch.int32, (B, None))
    max_pages = page_table.shape[1]
    _need(k8_pages, "k8_pages", torch.uint8, (None, None))
    num_pages = k8_pages.shape[0] // 32
    d = k8_pages.shape[1]
    if k8_pages.shape[0] != 32 * num_pages:
        raise ValueError(f"k8_pages must have a multiple of 32 rows, got {k8_pages.shape[0]}")
    _need(sk_pages, "sk_pages", torch.float32, (32 * num_pages,))
    _need(k_idx_pages, "k_idx_pages", torch.bfloat16, (32 * kpool * num_pages, d))
    _need(gate_pages, "gate_pages", torch.bfloat16, (32 * kpool * num_pages, d))
    _need(ape, "ape", torch.float32, (kpool, d))
    dev = _on(("cu_seqlens", cu_seqlens), ("page_table", page_table), ("k_idx_pages", k_idx_pages),
              ("gate_pages", gate_pages), ("ape", ape), ("k8_pages", k8_pages), ("sk_pages", sk_pages))
    _check(lib().kpool_update_paged(_ptr(cu_seqlens), B, _ptr(page_table), max_pages, num_pages, _ptr(k_idx_pages),
                                    _ptr(gate_pages), _ptr(ape), d, kpool, last_tokens, _ptr(k8_pages),
                                    _ptr(sk_pages), _stream(dev)))


def indexer_score_topk_paged(cu_seqlens: torch.Tensor, page_table: torch.Tensor, k8_pages: torch.Tensor,
                             sk_pages: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor, num_tokens: int,
                             kpool: int = 4, topk_pools: int = 512, row_width: Optional[int] = None,
                             q_pos: Optional[torch.Tensor] = None, return_row_path: bool = False,
                             workspace: Optional[torch.Tensor] = None):
    """Fused FP8 scoring and top-k over a paged pooled-key cache. Index rows hold
    page slots. Returns (indices int32 [Tq,W], num_valid int32 [Tq], row_path
    int32 [Tq] or None)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    B = cu_seqlens.shape[0] - 1
    _need(page_table, "page_table", torch.int32, (B, None))
    max_pages = page_table.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16, (None, None, None))
    Tq, h, d = q_idx.shape
    _need(k8_pages, "k8_pages", torch.uint8, (None, d))
    num_pages = k8_pages.shape[0] // 32
    if k8_pages.shape[0] != 32 * num_pages:
        raise ValueError(f"k8_pages must have a multiple of 32 rows, got {k8_pages.shape[0]}")
    _need(sk_pages, "sk_pages", torch.float32, (32 * num_pages,))
    _need(w_idx, "w_idx", torch.float32, (Tq, h))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (Tq,))
    elif Tq != num_tokens:
        raise ValueError(f"without q_pos every token is a query: q_idx must have {num_tokens} rows, got {Tq}")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, (None,))
    dev = _on(("cu_seqlens", cu_seqlens), ("page_table", page_table), ("k8_pages", k8_pages),
              ("sk_pages", sk_pages), ("q_idx", q_idx), ("w_idx", w_idx), ("q_pos", q_pos), ("workspace", workspace))
    W = row_width if row_width is not None else kp_row_width(kpool, topk_pools)
    indices = torch.empty((Tq, W), dtype=torch.int32, device=dev)
    num_valid = torch.empty(Tq, dtype=torch.int32, device=dev)
    row_path = torch.empty(Tq, dtype=torch.int32, device=dev) if return_row_path else None
    need = kp_indexer_paged_workspace_bytes(Tq, B, h, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().indexer_score_topk_paged(_ptr(cu_seqlens), B, num_tokens, _ptr(page_table), max_pages, num_pages,
                                          _ptr(k8_pages), _ptr(sk_pages), _ptr(q_pos), Tq, _ptr(q_idx), _ptr(w_idx),
                                          h, d, kpool, topk_pools, W, _ptr(indices), _ptr(num_valid),
                                          _ptr(row_path), _ptr(workspace), workspace.numel(), _stream(dev)))
    return indices, num_valid, row_path


def indexer_topk_from_scores(cu_seqlens: torch.Tensor, cu_pools: torch.Tensor, scores: torch.Tensor,
                             num_tokens: int, kpool: int = 4, topk_pools: int = 512,
                             row_width: Optional[int] = None, q_pos: Optional[torch.Tensor] = None):
    """Top-k index rows of a given score tensor [Tq, num_tokens // kpool]."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    B = cu_seqlens.shape[0] - 1
    _need(cu_pools, "cu_pools", torch.int32, (B + 1,))
    _need(scores, "scores", torch.float32, (None, num_tokens // kpool))
    Tq, max_pools = scores.shape
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (Tq,))
    elif Tq != num_tokens:
        raise ValueError(f"without q_pos every token is a query: scores must have {num_tokens} rows, got {Tq}")
    dev = _on(("cu_seqlens", cu_seqlens), ("cu_pools", cu_pools), ("scores", scores), ("q_pos", q_pos))
    W = row_width if row_width is not None else kp_row_width(kpool, topk_pools)
    indices = torch.empty((Tq, W), dtype=torch.int32, device=dev)
    num_valid = torch.empty(Tq, dtype=torch.int32, device=dev)
    _check(lib().indexer_topk_from_scores(_ptr(cu_seqlens), cu_seqlens.shape[0] - 1, num_tokens,
                                          _ptr(cu_pools), max_pools, _ptr(q_pos), Tq, _ptr(scores), kpool,
                                          topk_pools, W, _ptr(indices), _ptr(num_valid), _stream(dev)))
    return indices, num_valid


def kp_mla_fwd_workspace_bytes(num_q: int, heads: int, d_latent: int, row_width: int) -> int:
    return int(lib().kp_mla_fwd_workspace_bytes(num_q, heads, d_latent, row_width))


def sparse_mla_fwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, softmax_scale: float,
                   return_lse: bool = True, out: Optional[torch.Tensor] = None, split: bool = True,
                   workspace: Optional[torch.Tensor] = None):
    """Absorbed sparse latent attention: (out bf16 [Tq,H,d_v], lse f32 [Tq,H] or None);
    d_v = D, except 512 for 576-wide keys (a 64-wide RoPE tail). ``split``: give
    the library a workspace, so that few-query launches split their rows."""
    _need(q, "q", torch.bfloat16, (None, None, None))
    Tq, H, D = q.shape
    d_v = 512 if D == 576 else D
    _need(kv, "kv", torch.bfloat16, (None, D))
    _need(indices, "indices", torch.int32, (Tq, None))
    if out is not None:
        _need(out, "out", torch.bfloat16, (Tq, H, d_v))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, (None,))
    dev = _on(("q", q), ("kv", kv), ("indices", indices), ("out", out), ("workspace", workspace))
    if out is None:
        out = torch.empty((Tq, H, d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Tq, H), dtype=torch.float32, device=dev) if return_lse else None
    W = indices.shape[1]
    need = kp_mla_fwd_workspace_bytes(Tq, H, D, W) if split else 0
    if need > 0 and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws = workspace if need > 0 else None
    _check(lib().sparse_mla_fwd(_ptr(q), _ptr(kv), _ptr(indices), Tq, kv.shape[0], H, D, W, float(softmax_scale),
                                _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return out, lse


def kp_mla_bwd_workspace_bytes(num_q: int, d_latent: int, row_width: int) -> int:
    return int(lib().kp_mla_bwd_workspace_bytes(num_q, d_latent, row_width))


def sparse_mla_bwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, out: torch.Tensor,
                   lse: torch.Tensor, d_out: torch.Tensor, softmax_scale: float,
                   workspace: Optional[torch.Tensor] = None):
    """Backward of sparse_mla_fwd: (d_q bf16 [Tq,H,D], d_kv f32 [N,D])."""
    _need(q, "q", torch.bfloat16, (None, None, None))
    Tq, H, D = q.shape
    _need(kv, "kv", torch.bfloat16, (None, D))
    _need(indices, "indices", torch.int32, (Tq, None))
    _need(out, "out", torch.bfloat16, (Tq, H, D))
    _need(lse, "lse", torch.float32, (Tq, H))
    _need(d_out, "d_out", torch.bfloat16, (Tq, H, D))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, (None,))
    dev = _on(("q", q), ("kv", kv), ("indices", indices), ("out", out), ("lse", lse), ("d_out", d_out),
              ("workspace", workspace))
    W = indices.shape[1]
    need = kp_mla_bwd_workspace_bytes(Tq, D, W)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    d_q = torch.empty((Tq, H, D), dtype=torch.bfloat16, device=dev)
    d_kv = torch.empty((kv.shape[0], D), dtype=torch.float32, device=dev)
    _check(lib().sparse_mla_bwd(_ptr(q), _ptr(kv), _ptr(indices), _ptr(out), _ptr(lse), _ptr(d_out), Tq,
                                kv.shape[0], H, D, W, float(softmax_scale), _ptr(d_q), _ptr(d_kv),
                                _ptr(workspace), workspace.numel(), _stream(dev)))
    return d_q, d_kv


def kp_check_inputs(cu_seqlens: torch.Tensor, num_tokens: int, q_pos: Optional[torch.Tensor] = None) -> None:
    _need(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (None,))
    _on(("cu_seqlens", cu_seqlens), ("q_pos", q_pos))
    nq = 0 if q_pos is None else q_pos.shape[0]
    _check(lib().kp_check_inputs(_ptr(cu_seqlens), cu_seqlens.shape[0] - 1, num_tokens, _ptr(q_pos), nq,
                                 _stream(cu_seqlens.device)))


def dsa_forward_shared(q, kv, indices, *, softmax_scale):
    """A shared DSA layer (IndexShare): attention with the index rows of the
    previous full layer (its dsa_forward's ``indices``); no pooling, scoring or
    selection. Returns (out, lse)."""
    return sparse_mla_fwd(q, kv, indices, softmax_scale)


def dsa_forward(cu_seqlens, k_idx, gate, ape, q_idx, w_idx, q, kv, *, kpool=4, topk_pools=512,
                softmax_scale, q_pos=None, workspace=None):
    """One KPool-DSA forward: kpool_build, indexer_score_topk, sparse_mla_fwd."""
    cu_pools, _, k8, ks, _ = kpool_build(cu_seqlens, k_idx, gate, ape, kpool)
    idx, nv, _ = indexer_score_topk(cu_seqlens, cu_pools, k8, ks, q_idx, w_idx, k_idx.shape[0], kpool,
                                    topk_pools, q_pos=q_pos, workspace=workspace)
    out, lse = sparse_mla_fwd(q, kv, idx, softmax_scale)
    return out, lse, idx, nv
