"""GPU parity of the sparse-MLA backward (sparse_mla_bwd, through the C ABI)
against the oracle's float64 backward, on the same inputs: the GPU forward's
out and lse feed the GPU backward (as in training); the oracle recomputes
everything from q, kv and the index rows.

Bar (derived from the arithmetic): the kernels round p and scale*ds to bf16
for the products, and dQ to bf16 at the end; each element's error is then a
few 2^-9 relative of the terms it sums. Asserted per tensor: relative RMSE
<= 5e-3 and cosine >= 0.99999 (the form the pages use for dQ and dKV: their
cuDNN kernel reports relRMSE 1.7e-3 for dQ and 3.7e-3 for dKV against a dense
reference), and per element |d| <= 2e-2 * max(1, A) with A the magnitude of the
terms the element sums (for dQ: scale * sum_j p_j |dp_j - delta| |k_j|; for
dKV: the same over its contributions), which the oracle side computes below.
"""
import numpy as np
import pytest
import torch

from tests._util import dev, dev_bf16, host
from workloads import Workload, bf16_bits_to_f32, f32_to_bf16_bits, spec

pytestmark = pytest.mark.gpu

REL_RMSE = 5e-3
COS_MIN = 0.99999
ELEM = 2e-2


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_kpool_amd as K
    K.lib()
    return K


def _log(*a):
    print(*a, flush=True)


def _metrics(g, r):
    g = g.astype(np.float64)
    r = r.astype(np.float64)
    rel = float(np.sqrt(((g - r) ** 2).sum() / max((r ** 2).sum(), 1e-300)))
    cos = float((g * r).sum() / max(np.sqrt((g * g).sum() * (r * r).sum()), 1e-300))
    return rel, cos


def _magnitudes(q, kv, idx, d_out, scale):
    """Per-element magnitude of the summed terms of dQ and dKV (float64)."""
    qf = bf16_bits_to_f32(q).astype(np.float64)
    kvf = bf16_bits_to_f32(kv).astype(np.float64)
    g = bf16_bits_to_f32(d_out).astype(np.float64)
    N = kv.shape[0]
    aq = np.zeros(qf.shape)
    akv = np.zeros(kvf.shape)
    for i in range(q.shape[0]):
        sel = np.array([r for r in idx[i] if 0 <= r < N], np.int64)
        if sel.size == 0:
            continue
        Kr = kvf[sel]
        s = scale * qf[i] @ Kr.T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = g[i] @ Kr.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        w = scale * p * np.abs(dp - delta)                       # [H, n]
        aq[i] = w @ np.abs(Kr)
        contrib = w.T @ np.abs(qf[i]) + p.T @ np.abs(g[i])       # [n, D]
        np.add.at(akv, sel, contrib)
    return aq, akv


def _run(K, oracle_mod, q, kv, idx, d_out, scale, name):
    qd, kvd, idxd = dev_bf16(q), dev_bf16(kv), dev(idx)
    out, lse = K.sparse_mla_fwd(qd, kvd, idxd, scale)
    dq, dkv = K.sparse_mla_bwd(qd, kvd, idxd, out, lse, dev_bf16(d_out), scale)
    g_dq = host(dq.float())
    g_dkv = host(dkv)
    r_dq, r_dkv = oracle_mod.sparse_mla_bwd(q, kv, idx, d_out, scale)
    aq, akv = _magnitudes(q, kv, idx, d_out, scale)
    info = {}
    for nm, g, r, a in (("dq", g_dq, r_dq, aq), ("dkv", g_dkv, r_dkv, akv)):
        rel, cos = _metrics(g, r)
        e = np.abs(g.astype(np.float64) - r) / np.maximum(1.0, a)
        info[nm] = {"rel_rmse": rel, "cos": cos, "elem_max": float(e.max()), "abs_max": float(np.abs(g - r).max())}
        assert rel <= REL_RMSE and cos >= COS_MIN, f"{name} {nm}: relRMSE {rel:.3e} cos {cos:.9f}"
        assert e.max() <= ELEM, f"{name} {nm}: element error {e.max():.3e}"
    _log("  ", name, info)
    return info


def _rand_case(seed, Tq, H, D, N, W, kind="dense"):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((Tq, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    d_out = f32_to_bf16_bits(rng.standard_normal((Tq, H, D)))
    idx = rng.integers(0, N, size=(Tq, W)).astype(np.int32)
    if kind == "masked":
        m = rng.random(idx.shape) < 0.3
        idx[m] = rng.choice([-1, N, 2 ** 31 - 1], size=m.sum())
        idx[1] = -1                                   # an empty row
        idx[2, :] = -1
        idx[2, 5] = 7                                 # a single entry
    if kind == "ragged":
        for i in range(Tq):
            idx[i, int(rng.integers(1, W)):] = -1
    if kind == "heavy":
        # half of every row names one of three latent rows (repeats included), so
        # those rows collect long runs of terms across queries
        m = rng.random(idx.shape) < 0.5
        idx[m] = rng.integers(0, 3, size=m.sum())
        idx[:, -3:] = -1
    return q, kv, idx, d_out


@pytest.mark.parametrize("case", ["tiny", "d512_dense", "d512_masked", "d512_ragged", "d512_heavy", "heads40",
                                  "d64_masked"])
def test_bwd_random(K, oracle_mod, case):
    if case == "tiny":
        s = spec("tiny")
        wl = Workload(s)
        res = oracle_mod.dsa_forward(wl, with_mla=False)
        q, kv, idx = wl.full("q"), wl.full("kv"), res["indices"]
        d_out = f32_to_bf16_bits(np.random.default_rng(4).standard_normal(q.shape))
        scale = s.scale
    else:
        H, D = (40 if case == "heads40" else 64), (64 if case.startswith("d64") else 512)
        kind = case.split("_")[-1] if "_" in case else "masked"
        q, kv, idx, d_out = _rand_case(21, 24, H, D, 700, 256, kind)
        scale = 1 / np.sqrt(D)
    _log("bwd", case, q.shape, idx.shape)
    _run(K, oracle_mod, q, kv, idx, d_out, scale, case)


@pytest.mark.parametrize("name", ["2k", "packed4k", "32k"])
def test_bwd_workload_rows(K, oracle_mod, name):
    """The oracle's index rows of sampled queries of the training-shaped
    workloads (the backward of a subset of queries is the same computation
    restricted to them: dKV sums over the given queries only)."""
    s = spec(name)
    wl = Workload(s)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(s.Tq, 14, replace=False), [0, 1, 5, s.Tq - 1]]))
    if name == "packed4k":
        rows = np.unique(np.concatenate([rows, s.cu[:-1], s.cu[1:] - 1]))
    res = oracle_mod.dsa_forward(wl, q_rows=rows, with_mla=False)
    q = np.concatenate([wl.rows("q", int(r), int(r) + 1) for r in rows])
    d_out = f32_to_bf16_bits(np.random.default_rng(6).standard_normal(q.shape))
    _log("bwd", name, len(rows), "rows")
    _run(K, oracle_mod, q, wl.full("kv"), res["indices"], d_out, s.scale, name)


def test_bwd_query_chunks(K, oracle_mod):
    """More queries than one chunk of the dKV sum (8192): the chunks' sums are
    added in order; rows named by queries of both chunks, long runs included."""
    q, kv, idx, d_out = _rand_case(31, 8300, 8, 64, 300, 64, "heavy")
    _log("bwd chunks", q.shape, idx.shape)
    _run(K, oracle_mod, q, kv, idx, d_out, 1 / 8, "chunks")


def test_bwd_deterministic(K):
    """dQ and dKV are bit-reproducible (the dKV sum runs in a fixed order)."""
    rng = np.random.default_rng(8)
    q, kv, idx, d_out = _rand_case(9, 300, 64, 512, 2000, 512, "ragged")
    qd, kvd, idxd = dev_bf16(q), dev_bf16(kv), dev(idx)
    out, lse = K.sparse_mla_fwd(qd, kvd, idxd, 1 / np.sqrt(512))
    g = dev_bf16(d_out)
    a = K.sparse_mla_bwd(qd, kvd, idxd, out, lse, g, 1 / np.sqrt(512))
    b = K.sparse_mla_bwd(qd, kvd, idxd, out, lse, g, 1 / np.sqrt(512))
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
