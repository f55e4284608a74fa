"""Out-of-bounds writes: every output and workspace of the main entry points lies
inside a larger buffer whose 4 KiB guard bands before and after hold a known
byte. The entry points are called through the C ABI on those buffers; the guard
bands must come back untouched, and the outputs must equal, bit for bit, those
of the same call through the binding (into buffers of exactly the output's
size). Inputs: the packed 4,096-token row of five documents (ragged document
lengths, a top-k that selects from 1,021-1,024 pools), 64 of its queries for the
split (few-query) attention path."""
import ctypes as C

import numpy as np
import pytest
import torch

from workloads import Workload, spec

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of guard band on each side (keeps the body 4 KiB aligned)
FILL_GUARD = 0xA5
FILL_BODY = 0x5A


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_kpool_amd as K
    K.lib()
    return K


class Guarded:
    """A device buffer of `nbytes` between two guard bands."""

    def __init__(self, nbytes: int):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * GUARD,), FILL_GUARD, dtype=torch.uint8, device="cuda")
        self.buf[GUARD:GUARD + self.n] = FILL_BODY

    @property
    def ptr(self):
        return C.c_void_p(self.buf.data_ptr() + GUARD)

    def body(self, dtype, shape):
        return self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def guards_intact(self) -> bool:
        return bool((self.buf[:GUARD] == FILL_GUARD).all() and (self.buf[GUARD + self.n:] == FILL_GUARD).all())


def _nbytes(dtype, shape):
    return int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _check_all(K, status, outs, name):
    assert status == 0, f"{name}: status {status}: {K.lib().kp_last_error().decode()}"
    torch.cuda.synchronize()
    for label, g in outs.items():
        assert g.guards_intact(), f"{name}: a write landed outside {label}"


@pytest.fixture(scope="module")
def packed(K):
    s = spec("packed4k")
    wl = Workload(s)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    d = dict(s=s, cu=torch.from_numpy(s.cu).cuda(), k_idx=bf(wl.full("k_idx")), gate=bf(wl.full("gate")),
             ape=torch.from_numpy(wl.ape()).cuda(), q_idx=bf(wl.full("q_idx")),
             w=torch.from_numpy(wl.full("w")).cuda(), q=bf(wl.full("q")), kv=bf(wl.full("kv")))
    return d


def test_kpool_build_guarded(K, packed):
    s, cu, k_idx, gate, ape = packed["s"], packed["cu"], packed["k_idx"], packed["gate"], packed["ape"]
    ref = K.kpool_build(cu, k_idx, gate, ape, s.kpool, with_f32=True)
    B, cap, d = s.B, s.T // s.kpool, s.D_I
    shapes = {"cu_pools": (torch.int32, (B + 1,)), "pool_start": (torch.int32, (cap,)),
              "k8": (torch.uint8, (cap, d)), "ks": (torch.float32, (cap,)), "kf": (torch.float32, (cap, d))}
    g = {k: Guarded(_nbytes(*v)) for k, v in shapes.items()}
    st = K.lib().kpool_build(_p(cu), B, s.T, _p(k_idx), _p(gate), _p(ape), d, s.kpool, g["cu_pools"].ptr,
                             g["pool_start"].ptr, g["k8"].ptr, g["ks"].ptr, g["kf"].ptr, _stream())
    _check_all(K, st, g, "kpool_build")
    for (k, (dt, sh)), r in zip(shapes.items(), ref):
        assert torch.equal(g[k].body(dt, sh).view(torch.uint8), r.contiguous().view(torch.uint8)), k


def test_indexer_guarded(K, packed):
    s, cu = packed["s"], packed["cu"]
    cp, _, k8, ks, _ = K.kpool_build(cu, packed["k_idx"], packed["gate"], packed["ape"], s.kpool)
    idx, nv, sc = K.indexer_score_topk(cu, cp, k8, ks, packed["q_idx"], packed["w"], s.T, s.kpool, s.topk,
                                       return_scores=True)
    W, P = s.row_width, s.max_pools
    ws = K.kp_indexer_workspace_bytes(s.Tq, P, s.H_I, s.D_I, s.topk)
    g = {"indices": Guarded(4 * s.Tq * W), "num_valid": Guarded(4 * s.Tq), "scores": Guarded(4 * s.Tq * P),
         "workspace": Guarded(ws)}
    st = K.lib().indexer_score_topk(_p(cu), s.B, s.T, _p(cp), P, _p(k8), _p(ks), None, s.Tq, _p(packed["q_idx"]),
                                    _p(packed["w"]), s.H_I, s.D_I, s.kpool, s.topk, W, g["indices"].ptr,
                                    g["num_valid"].ptr, g["scores"].ptr, g["workspace"].ptr, ws, _stream())
    _check_all(K, st, g, "indexer_score_topk")
    assert torch.equal(g["indices"].body(torch.int32, (s.Tq, W)), idx)
    assert torch.equal(g["num_valid"].body(torch.int32, (s.Tq,)), nv)
    assert torch.equal(g["scores"].body(torch.int32, (s.Tq, P)), sc.view(torch.int32))
    # the top-k alone, from the scores
    g2 = {"indices": Guarded(4 * s.Tq * W), "num_valid": Guarded(4 * s.Tq)}
    st = K.lib().indexer_topk_from_scores(_p(cu), s.B, s.T, _p(cp), P, None, s.Tq, _p(sc), s.kpool, s.topk, W,
                                          g2["indices"].ptr, g2["num_valid"].ptr, _stream())
    _check_all(K, st, g2, "indexer_topk_from_scores")
    assert torch.equal(g2["indices"].body(torch.int32, (s.Tq, W)), idx)
    # the query codes
    codes, scales = K.indexer_rotate_quant(packed["q_idx"])
    g3 = {"codes": Guarded(s.Tq * s.H_I * s.D_I), "scales": Guarded(4 * s.Tq * s.H_I)}
    st = K.lib().indexer_rotate_quant(_p(packed["q_idx"]), s.Tq, s.H_I, s.D_I, g3["codes"].ptr, g3["scales"].ptr,
                                      _stream())
    _check_all(K, st, g3, "indexer_rotate_quant")
    assert torch.equal(g3["codes"].body(torch.uint8, codes.shape), codes)
    assert torch.equal(g3["scales"].body(torch.float32, scales.shape), scales)


@pytest.mark.parametrize("nq", [None, 64])
def test_attention_guarded(K, packed, nq):
    """All queries (one workgroup per query) and 64 queries (rows split over
    workgroups, with a workspace), forward and backward."""
    s, cu = packed["s"], packed["cu"]
    cp, _, k8, ks, _ = K.kpool_build(cu, packed["k_idx"], packed["gate"], packed["ape"], s.kpool)
    idx, _, _ = K.indexer_score_topk(cu, cp, k8, ks, packed["q_idx"], packed["w"], s.T, s.kpool, s.topk)
    q, kv = packed["q"], packed["kv"]
    if nq is not None:   # the last 64 queries (the longest rows)
        q, idx = q[-nq:].contiguous(), idx[-nq:].contiguous()
    Tq, H, D = q.shape
    W = idx.shape[1]
    out, lse = K.sparse_mla_fwd(q, kv, idx, s.scale)
    ws = K.kp_mla_fwd_workspace_bytes(Tq, H, D, W)
    print("guarded attention", "queries", Tq, "workspace", ws, flush=True)
    g = {"out": Guarded(2 * Tq * H * D), "lse": Guarded(4 * Tq * H), "workspace": Guarded(max(ws, 16))}
    st = K.lib().sparse_mla_fwd(_p(q), _p(kv), _p(idx), Tq, kv.shape[0], H, D, W, C.c_float(s.scale),
                                g["out"].ptr, g["lse"].ptr, g["workspace"].ptr if ws > 0 else None, ws, _stream())
    _check_all(K, st, g, "sparse_mla_fwd")
    assert torch.equal(g["out"].body(torch.int16, (Tq, H, D)), out.view(torch.int16))
    assert torch.equal(g["lse"].body(torch.int32, (Tq, H)), lse.view(torch.int32))
    # backward
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    d_out = (torch.randn((Tq, H, D), generator=gen, device="cuda") * 0.1).bfloat16()
    d_q, d_kv = K.sparse_mla_bwd(q, kv, idx, out, lse, d_out, s.scale)
    wb = K.kp_mla_bwd_workspace_bytes(Tq, D, W)
    gb = {"d_q": Guarded(2 * Tq * H * D), "d_kv": Guarded(4 * kv.shape[0] * D), "workspace": Guarded(wb)}
    st = K.lib().sparse_mla_bwd(_p(q), _p(kv), _p(idx), _p(out), _p(lse), _p(d_out), Tq, kv.shape[0], H, D, W,
                                C.c_float(s.scale), gb["d_q"].ptr, gb["d_kv"].ptr, gb["workspace"].ptr, wb,
                                _stream())
    _check_all(K, st, gb, "sparse_mla_bwd")
    assert torch.equal(gb["d_q"].body(torch.int16, (Tq, H, D)), d_q.view(torch.int16))
    assert torch.equal(gb["d_kv"].body(torch.int32, (kv.shape[0], D)), d_kv.view(torch.int32))
