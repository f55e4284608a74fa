"""Pins of the oracle's sparse latent attention and of the whole forward.

Sparse MLA in absorbed form with no RoPE: the query heads attend over rows of
one shared 512-wide latent that is both key and value (NeMo AutoModel PR "add
GLM-5.3-Flash training support", Changelog; prime-rl PR "GLM-5.3-Flash text
model", Summary, second bullet). The pages validate fast sparse kernels against
a dense SDPA reference path (NeMo AutoModel "GLM-5.3-Flash" page, Attention
Backends); here torch's scaled_dot_product_attention in float64 on the CPU is
that library routine.
"""
import numpy as np
import pytest
import torch

from workloads import Workload, bf16_bits_to_f32, custom, f32_to_bf16_bits, spec


def _sdpa(q, kv, mask, scale):
    """q [Tq,H,D] f64, kv [N,D] f64, mask [Tq,N] bool -> [Tq,H,D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)                # [H, Tq, D]
    k = torch.from_numpy(kv)[None].expand(q.shape[1], -1, -1)
    m = torch.from_numpy(mask)[None].expand(q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, k, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()


def _rows_to_mask(idx, n):
    m = np.zeros((idx.shape[0], n), bool)
    for i in range(idx.shape[0]):
        v = idx[i][(idx[i] >= 0) & (idx[i] < n)]
        m[i, v] = True
    return m


def test_mla_equals_dense_masked_sdpa(oracle_mod):
    rng = np.random.default_rng(0)
    Tq, H, D, N, W = 12, 4, 64, 90, 128
    q = f32_to_bf16_bits(rng.standard_normal((Tq, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    idx = np.full((Tq, W), -1, np.int32)
    for i in range(Tq):
        n = int(rng.integers(1, 60))
        idx[i, :n] = np.sort(rng.choice(N, size=n, replace=False))
        idx[i, n:n + 3] = [N, N + 5, -7]                    # out-of-range entries are masked
    out, lse = oracle_mod.sparse_mla(q, kv, idx, 0.125)
    ref = _sdpa(bf16_bits_to_f32(q).astype(np.float64), bf16_bits_to_f32(kv).astype(np.float64),
                _rows_to_mask(idx, N), 0.125)
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)
    # lse against a direct log-sum-exp of the masked logits
    s = np.einsum("thd,nd->thn", bf16_bits_to_f32(q).astype(np.float64),
                  bf16_bits_to_f32(kv).astype(np.float64)) * 0.125
    m = _rows_to_mask(idx, N)[:, None, :]
    ref_lse = np.log(np.where(m, np.exp(s), 0.0).sum(-1))
    assert np.allclose(lse, ref_lse, rtol=1e-6, atol=1e-6)


def test_mla_single_row_and_identical_rows(oracle_mod):
    rng = np.random.default_rng(1)
    H, D, N = 4, 64, 10
    q = f32_to_bf16_bits(rng.standard_normal((3, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    idx = np.full((3, 128), -1, np.int32)
    idx[0, 0] = 7                                           # one valid index -> that row
    idx[1, :5] = [2, 2, 2, 2, 2]                            # the same row five times -> that row
    kv2 = kv.copy()
    kv2[[1, 4, 8]] = kv2[3]
    idx[2, :4] = [1, 3, 4, 8]                               # identical rows -> that row
    out, lse = oracle_mod.sparse_mla(q, kv, idx[:2], 0.1)
    assert np.array_equal(out[0], np.broadcast_to(bf16_bits_to_f32(kv[7]), (H, D)))
    assert np.allclose(out[1], np.broadcast_to(bf16_bits_to_f32(kv[2]), (H, D)), rtol=1e-7, atol=0)
    out2, _ = oracle_mod.sparse_mla(q[2:], kv2, idx[2:], 0.1)
    assert np.allclose(out2[0], np.broadcast_to(bf16_bits_to_f32(kv2[3]), (H, D)), rtol=1e-7, atol=0)
    assert np.allclose(lse[1] - lse[1], 0)


def test_mla_row_order_and_empty_rows(oracle_mod):
    rng = np.random.default_rng(2)
    H, D, N = 4, 64, 50
    q = f32_to_bf16_bits(rng.standard_normal((2, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    idx = np.full((2, 128), -1, np.int32)
    idx[0, :30] = rng.choice(N, 30, replace=False)
    perm = idx.copy()
    perm[0, :30] = idx[0, :30][::-1]
    perm[0, 50:80] = perm[0, :30]
    perm[0, :30] = -1                                        # padding may sit anywhere
    a, la = oracle_mod.sparse_mla(q, kv, idx, 0.2)
    b, lb = oracle_mod.sparse_mla(q, kv, perm, 0.2)
    assert np.allclose(a[0], b[0], rtol=1e-6, atol=1e-7) and np.allclose(la[0], lb[0], rtol=1e-7)
    assert np.all(a[1] == 0) and np.all(np.isneginf(la[1]))


def _dense_causal(oracle_mod, s, wl, rows):
    q = np.concatenate([wl.rows("q", int(r), int(r) + 1) for r in rows]).astype(np.uint16)
    kv = bf16_bits_to_f32(wl.full("kv")).astype(np.float64)
    qpos = s.query_positions()[rows]
    doc = np.searchsorted(s.cu, np.arange(s.T), side="right") - 1
    mask = np.zeros((len(rows), s.T), bool)
    for i, t in enumerate(qpos):
        mask[i] = (doc == doc[t]) & (np.arange(s.T) <= t)
    return _sdpa(bf16_bits_to_f32(q).astype(np.float64), kv, mask, s.scale)


def test_end_to_end_tiny_dense_equals_causal(oracle_mod):
    """Top-k 16 covers every pool of the 64-token document: the whole forward
    (pooling, rotation, FP8 scoring, selection, sparse MLA) must equal dense
    causal attention, whatever the indexer computes."""
    s = spec("tiny_dense")
    wl = Workload(s)
    res = oracle_mod.dsa_forward(wl)
    ref = _dense_causal(oracle_mod, s, wl, np.arange(s.T))
    assert np.allclose(res["out"], ref, rtol=1e-6, atol=1e-6)


def test_end_to_end_2k_sampled_equals_causal(oracle_mod):
    """The 2,048-token document with top-k 512: selection covers every visible
    pool, so sparse equals dense causal attention (sampled query rows)."""
    s = spec("2k")
    wl = Workload(s)
    rows = np.array([0, 1, 2, 3, 4, 7, 100, 511, 1024, 1500, 2046, 2047])
    res = oracle_mod.dsa_forward(wl, q_rows=rows)
    assert all(res["num_valid"][i] == t + 1 for i, t in enumerate(rows))
    ref = _dense_causal(oracle_mod, s, wl, rows)
    assert np.allclose(res["out"], ref, rtol=1e-6, atol=1e-6)


def test_end_to_end_packed_isolation(oracle_mod):
    """Packed row of 5 documents: every index row stays inside the query's own
    document and at or before the query."""
    s = spec("packed4k")
    wl = Workload(s)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(s.T, 40, replace=False), s.cu[1:-1] - 1, s.cu[1:-1],
                                     s.cu[1:-1] + 3, [s.T - 1]]))
    res = oracle_mod.dsa_forward(wl, q_rows=rows, with_mla=False)
    doc = np.searchsorted(s.cu, np.arange(s.T), side="right") - 1
    for i, t in enumerate(rows):
        r = res["indices"][i, :res["num_valid"][i]]
        assert np.all(doc[r] == doc[t]) and np.all(r <= t) and r[-1] <= t
        assert np.all(res["indices"][i, res["num_valid"][i]:] == -1)


def test_mla_abs_magnitude(oracle_mod):
    """The error scale sum_j p_j |v_j| bounds |o| and equals o when every value
    is non-negative."""
    rng = np.random.default_rng(4)
    H, D, N = 4, 64, 40
    q = f32_to_bf16_bits(rng.standard_normal((3, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    idx = np.full((3, 128), -1, np.int32)
    idx[:, :25] = rng.choice(N, (3, 25))
    out, lse, oabs = oracle_mod.sparse_mla(q, kv, idx, 0.125, with_abs=True)
    assert np.all(oabs >= np.abs(out) - 1e-6)
    kv_pos = kv & np.uint16(0x7FFF)              # clear the sign bit: |v|
    out_p, _, oabs_p = oracle_mod.sparse_mla(q, kv_pos, idx, 0.125, with_abs=True)
    assert np.allclose(out_p, oabs_p, rtol=1e-6, atol=0)
