"""The C ABI loads on a host without a GPU, exports every entry point its
header declares, and rejects bad arguments before touching the device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kpool.h")


@pytest.fixture(scope="module")
def L():
    from sparse_attention_kpool_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_kpool_amd import build
        build.build()
    return _lib.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(k\w+|indexer_\w+|sparse_\w+)\s*\(", src, re.M)))


def test_header_symbols_exported(L):
    from sparse_attention_kpool_amd import _lib
    names = _declared()
    assert set(names) == {n for n, _, _ in _lib.SIGNATURES}
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_row_width(L):
    assert L.kp_row_width(4, 512) == 2176          # 2051 raw slots -> 2176
    assert L.kp_row_width(4, 4) == 128
    assert L.kp_row_width(4, 0) == 128
    assert L.kp_row_width(1, 128) == 128
    assert L.kp_row_width(1, 129) == 256
    assert L.kp_row_width(0, 4) == -1 and L.kp_row_width(4, -1) == -1
    assert L.kp_version() >= 100


def test_workspace_size(L):
    ws = L.kp_indexer_workspace_bytes(32768, 8192, 32, 128, 512)
    assert ws >= 32768 * 32 * 128 + 32768 * 32 * 4 + 32768 * 8192 * 4
    assert ws % 256 == 0
    assert L.kp_indexer_workspace_bytes(0, 8192, 32, 128, 512) == 0
    # rows of at least 32768 pools with top-k <= 8192: no score tensor, 128 KiB of
    # candidates per query instead (the 1M-token decode: 64 MiB of scores -> 8 MiB)
    q_part = 64 * 32 * 128 + 64 * 32 * 4
    per_q = 16384 * 8
    fused = L.kp_indexer_workspace_bytes(64, 1 << 18, 32, 128, 512)
    assert q_part + 64 * per_q <= fused < q_part + 64 * per_q + 8192
    assert L.kp_indexer_workspace_bytes(64, 1 << 18, 32, 128, 8193) >= 64 * (1 << 18) * 4   # top-k too large
    assert L.kp_indexer_workspace_bytes(64, 32767, 32, 128, 512) >= 64 * 32767 * 4          # rows too short
    # the paged path: the pool layout, the queries and the candidate lists
    pw = L.kp_indexer_paged_workspace_bytes(64, 3, 32, 128)
    assert pw % 256 == 0 and fused < pw <= fused + 256
    assert L.kp_indexer_paged_workspace_bytes(0, 3, 32, 128) == 0
    # the backward: one chunk of at most 8192 queries (coefficients, bf16 d_kv terms,
    # the sort's keys and positions, carries, delta corrections), the same for any larger num_q
    QC = 8192
    bw = L.kp_mla_bwd_workspace_bytes(QC, 512, 2176)
    E = QC * 2176
    assert bw % 256 == 0
    assert QC * 128 * 2176 * 2 + E * 512 * 2 + 4 * E * 4 <= bw < QC * 128 * 2176 * 2 + E * 512 * 2 + 4 * E * 4 \
        + (E // 128 + 1) * (2 * 512 * 4 + 8) + 256 * (E // 4096 + 2) * 4 + QC * 64 * 4 + 4096
    assert L.kp_mla_bwd_workspace_bytes(32768, 512, 2176) == bw
    assert L.kp_mla_bwd_workspace_bytes(2048, 512, 2176) < bw
    assert L.kp_mla_bwd_workspace_bytes(24, 64, 256) < L.kp_mla_bwd_workspace_bytes(24, 512, 256)
    assert L.kp_mla_bwd_workspace_bytes(24, 576, 256) == 0
    assert L.kp_mla_bwd_workspace_bytes(0, 512, 256) == 0


def test_invalid_args_rejected_on_host(L):
    """Each of these fails its host-side check and returns before any HIP call."""
    P = C.c_void_p
    fake = P(0x1000)
    # kpool_build: bad kpool / d_idx / missing pointers
    assert L.kpool_build(fake, 1, 64, fake, fake, fake, 128, 0, fake, fake, fake, fake, None, None) == 2
    assert L.kpool_build(fake, 1, 64, fake, fake, fake, 100, 4, fake, fake, fake, fake, None, None) == 2
    assert L.kpool_build(None, 1, 64, fake, fake, fake, 128, 4, fake, fake, fake, fake, None, None) == 1
    assert b"required" in L.kp_last_error()
    assert L.kpool_build(fake, -1, 64, fake, fake, fake, 128, 4, fake, fake, fake, fake, None, None) == 1
    # empty row: a no-op
    assert L.kpool_build(fake, 0, 0, None, None, None, 128, 4, fake, None, None, None, None, None) == 0
    # the first token of the pooled-key tail must lie in 0 .. num_tokens
    for lo in (-1, 65):
        assert L.kpool_build_from(fake, 1, 64, fake, fake, fake, 128, 4, lo, fake, fake, fake, fake, None, None) == 1
    assert b"token_lo" in L.kp_last_error()
    # indexer: row width not a multiple of 128 / too narrow / max_pools mismatch
    args = lambda W, mp=16, nq=64, qpos=None: (fake, 1, 64, fake, mp, fake, fake, qpos, nq, fake, fake, 2, 32, 4,
                                               4, W, fake, None, None, fake, 1 << 30, None)
    assert L.indexer_score_topk(*args(100)) == 1
    assert L.indexer_score_topk(*args(0)) == 1
    assert L.indexer_score_topk(*args(128, mp=15)) == 1
    assert L.indexer_score_topk(*args(128, nq=10)) == 1          # q_pos NULL needs num_q == num_tokens
    assert L.indexer_score_topk(*args(128, nq=0)) == 0           # empty shard: no-op
    # workspace too small
    a = list(args(128))
    a[20] = 16
    assert L.indexer_score_topk(*a) == 1
    assert b"workspace" in L.kp_last_error()
    # unsupported head count / latent width
    assert L.sparse_mla_fwd(fake, fake, fake, 4, 10, 65, 512, 128, C.c_float(0.1), fake, None, None, 0, None) == 2
    assert L.sparse_mla_fwd(fake, fake, fake, 4, 10, 64, 640, 128, C.c_float(0.1), fake, None, None, 0, None) == 2
    # 576-wide keys (the RoPE-tail contract) take index rows of at most 2048 entries
    assert L.sparse_mla_fwd(fake, fake, fake, 0, 10, 64, 576, 2048, C.c_float(0.1), fake, None, None, 0, None) == 0
    assert L.sparse_mla_fwd(fake, fake, fake, 4, 10, 64, 576, 2176, C.c_float(0.1), fake, None, None, 0, None) == 2
    # the backward takes 64- and 512-wide latents
    assert L.sparse_mla_bwd(fake, fake, fake, fake, fake, fake, 4, 10, 64, 576, 128, C.c_float(0.1), fake, fake,
                            fake, 1 << 30, None) == 2
    assert L.sparse_mla_fwd(None, fake, fake, 4, 10, 64, 512, 128, C.c_float(0.1), fake, None, None, 0, None) == 1
    # a latent of more than 4 GiB - 4 KiB (the row loads address it from 4 KiB below)
    assert L.sparse_mla_fwd(fake, fake, fake, 4, 1 << 22, 64, 512, 128, C.c_float(0.1), fake, None, None, 0, None) == 2
    assert b"4 GiB" in L.kp_last_error()
    # the boundary: 4,194,300 rows of 1 KiB are exactly 4 GiB - 4 KiB (the descriptor's
    # record count would wrap to 0), one row fewer fits (checked with no queries: no launch)
    edge = ((1 << 32) - 4096) // 1024
    assert L.sparse_mla_fwd(fake, fake, fake, 0, edge, 64, 512, 128, C.c_float(0.1), fake, None, None, 0, None) == 2
    assert L.sparse_mla_fwd(fake, fake, fake, 0, edge - 1, 64, 512, 128, C.c_float(0.1), fake, None, None, 0, None) == 0
    # index rows wider than the attention's LDS list
    assert L.sparse_mla_fwd(fake, fake, fake, 4, 10, 64, 512, 4097, C.c_float(0.1), fake, None, None, 0, None) == 2
    assert b"row_width" in L.kp_last_error()
    assert L.sparse_mla_fwd(fake, fake, fake, 0, 10, 64, 512, 128, C.c_float(0.1), fake, None, None, 0, None) == 0
    for bad in (0.0, -0.1, float("inf"), float("nan")):          # the softmax scale must be positive
        assert L.sparse_mla_fwd(fake, fake, fake, 4, 10, 64, 512, 128, C.c_float(bad), fake, None, None, 0, None) == 1
    # the allocation-free variant: argument checks as indexer_score_topk's, and sizes
    # whose workspace exceeds the library's device scratch are refused before launch
    nargs = lambda T, nq, qpos: (fake, 1, T, fake, T // 4, fake, fake, qpos, nq, fake, fake, 32, 128, 4, 512, 2176,
                                 fake, None, None, None)
    assert L.indexer_score_topk_noalloc(*nargs(4096, 0, None)) == 0           # empty shard
    assert L.indexer_score_topk_noalloc(*nargs(4096, 10, None)) == 1          # q_pos NULL needs num_q == T
    assert L.indexer_score_topk_noalloc(*nargs(32768, 32768, None)) == 2      # 32K: 671 MB of workspace
    assert b"scratch" in L.kp_last_error()
    assert L.kp_indexer_workspace_bytes(64, 1 << 18, 32, 128, 512) <= 72 << 20     # 1M-token decode fits
    assert L.indexer_rotate_quant(fake, 4, 2, 48, fake, fake, None) == 2
    assert L.indexer_topk_from_scores(fake, 1, 64, fake, 16, None, 64, None, 4, 4, 128, fake, None, None) == 1


def test_paged_args_rejected_on_host(L):
    """Argument checks of the paged cache's two entry points (no launch)."""
    fake = C.c_void_p(0x1000)
    # kpool_update_paged(cu, B, table, max_pages, num_pages, k_idx, gate, ape, d, kpool, last, k8, sk, stream)
    up = lambda **kw: L.kpool_update_paged(*[kw.get(k, v) for k, v in (
        ("cu", fake), ("B", 1), ("tab", fake), ("mp", 4), ("np", 8), ("ki", fake), ("ga", fake), ("ape", fake),
        ("d", 128), ("kp", 4), ("last", 1), ("k8", fake), ("sk", fake), ("st", None))])
    assert up(kp=0) == 2 and up(d=48) == 2
    assert up(last=-1) == 1 and up(np=-1) == 1
    assert up(last=0) == 0 and up(B=0) == 0                    # nothing to do
    assert up(tab=None) == 1 and b"required" in L.kp_last_error()
    assert up(np=1 << 26) == 2                                 # slots past 2^31
    # indexer_score_topk_paged(cu, B, T, table, max_pages, num_pages, k8, sk, q_pos, nq, q, w, h, d, kpool, topk,
    #                          W, idx, nv, row_path, ws, ws_bytes, stream)
    sp = lambda **kw: L.indexer_score_topk_paged(*[kw.get(k, v) for k, v in (
        ("cu", fake), ("B", 1), ("T", 4096), ("tab", fake), ("mp", 32), ("np", 32), ("k8", fake), ("sk", fake),
        ("qpos", fake), ("nq", 4), ("q", fake), ("w", fake), ("h", 32), ("d", 128), ("kp", 4), ("topk", 512),
        ("W", 2176), ("idx", fake), ("nv", None), ("rp", None), ("ws", fake), ("wsb", 1 << 30), ("st", None))])
    assert sp(topk=8193, W=32896) == 2 and b"8192" in L.kp_last_error()
    assert sp(W=2048) == 1 and sp(W=2200) == 1                   # narrower than 4*512+3 / not a multiple of 128
    assert sp(h=65) == 2 and sp(d=96) == 2
    assert sp(nq=0) == 0                                         # empty shard
    assert sp(qpos=None) == 1                                    # q_pos NULL needs num_q == num_tokens
    assert sp(tab=None) == 1 and sp(k8=None) == 1
    assert sp(wsb=1024) == 1 and b"workspace" in L.kp_last_error()
    assert sp(ws=C.c_void_p(0x1010)) == 1 and b"aligned" in L.kp_last_error()
