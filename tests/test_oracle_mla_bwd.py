"""Pins of the oracle's sparse-MLA backward and of its narrow-value forward.

The pages train GLM-5.3-Flash with a fast sparse-attention backward (NeMo
AutoModel "GLM-5.3-Flash" page, Attention Backends: FlashMLA forward, cuDNN
backward, validated against a dense SDPA reference by cosine and relative RMSE
of the output, dQ and dKV in NeMo AutoModel PR "add GLM-5.3-Flash training
support", "cuDNN sparse MLA parity and performance"); the indexer is frozen,
so the index rows are constants of the backward (prime-rl PR "GLM-5.3-Flash
text model", Summary, third bullet). The backward here is pinned to:

* torch's float64 autograd through the forward's definition (gather the named
  rows, softmax, weighted sum), an independent differentiation;
* central finite differences of a float64 forward on sampled coordinates;
* closed forms: the values' share of dKV sums to the sum of dO over every
  (query, head) with a non-empty row, the keys' share sums to zero (the softmax
  weights of a row sum to one); a row with one valid entry has dQ = 0.

The narrow-value forward (keys 576 wide, values their first 512 columns: the
GLM-5.2 contract kept by the NeMo PR, Changelog) is pinned to torch's float64
scaled_dot_product_attention with separate key and value tensors.
"""
import numpy as np
import pytest
import torch

from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _case(seed, Tq=6, H=4, D=48, N=40, W=64, d_v=None):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((Tq, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    dv = D if d_v is None else d_v
    d_out = f32_to_bf16_bits(rng.standard_normal((Tq, H, dv)))
    idx = np.full((Tq, W), -1, np.int32)
    for i in range(Tq):
        n = int(rng.integers(2, W // 2))
        idx[i, :n] = rng.integers(0, N, size=n)              # repeats allowed: they count twice
        idx[i, rng.integers(0, W, size=4)] = rng.choice([-1, N, N + 3, -9], size=4)   # scattered masked entries
    return q, kv, idx, d_out


def _torch_grads(q, kv, idx, d_out, scale):
    """float64 autograd of the forward's definition, query by query."""
    qf = torch.tensor(bf16_bits_to_f32(q), dtype=torch.float64, requires_grad=True)
    kvf = torch.tensor(bf16_bits_to_f32(kv), dtype=torch.float64, requires_grad=True)
    g = torch.tensor(bf16_bits_to_f32(d_out), dtype=torch.float64)
    d_v = d_out.shape[-1]
    loss = 0.0
    N = kv.shape[0]
    for i in range(q.shape[0]):
        sel = [int(r) for r in idx[i] if 0 <= r < N]
        if not sel:
            continue
        K = kvf[torch.tensor(sel)]                                  # [n, D], repeats kept
        p = torch.softmax(scale * qf[i] @ K.T, dim=-1)             # [H, n]
        o = p @ K[:, :d_v]
        loss = loss + (o * g[i]).sum()
    dq, dkv = torch.autograd.grad(loss, [qf, kvf], allow_unused=True)
    return dq.numpy(), dkv.numpy()


@pytest.mark.parametrize("seed,d_v", [(0, None), (1, None), (2, 32)])
def test_bwd_equals_torch_autograd(oracle_mod, seed, d_v):
    q, kv, idx, d_out = _case(seed, d_v=d_v)
    idx[3] = -1                                                     # an empty row: no gradient at all
    scale = 0.15
    dq, dkv = oracle_mod.sparse_mla_bwd(q, kv, idx, d_out, scale)
    rq, rkv = _torch_grads(q, kv, idx, d_out, scale)
    assert np.allclose(dq, rq, rtol=1e-6, atol=1e-6)
    assert np.allclose(dkv, rkv, rtol=1e-6, atol=1e-6)
    assert np.all(dq[3] == 0)


def test_bwd_finite_differences(oracle_mod):
    """Central differences of a float64 forward at 16 coordinates of q and of kv."""
    q, kv, idx, d_out = _case(5, Tq=3, H=2, D=16, N=12, W=16)
    scale = 0.3
    qf = bf16_bits_to_f32(q).astype(np.float64)
    kvf = bf16_bits_to_f32(kv).astype(np.float64)
    g = bf16_bits_to_f32(d_out).astype(np.float64)

    def loss(qv, kvv):
        tot = 0.0
        for i in range(qv.shape[0]):
            sel = [int(r) for r in idx[i] if 0 <= r < kvv.shape[0]]
            K = kvv[sel]
            s = scale * qv[i] @ K.T
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            tot += float(((p @ K) * g[i]).sum())
        return tot

    dq, dkv = oracle_mod.sparse_mla_bwd(q, kv, idx, d_out, scale)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for _ in range(16):
        i, h, c = rng.integers(0, q.shape[0]), rng.integers(0, q.shape[1]), rng.integers(0, q.shape[2])
        a, b = qf.copy(), qf.copy()
        a[i, h, c] += eps
        b[i, h, c] -= eps
        fd = (loss(a, kvf) - loss(b, kvf)) / (2 * eps)
        assert abs(fd - dq[i, h, c]) <= 1e-5 * max(1.0, abs(fd)), (i, h, c, fd, dq[i, h, c])
        r, c = rng.integers(0, kv.shape[0]), rng.integers(0, kv.shape[1])
        a, b = kvf.copy(), kvf.copy()
        a[r, c] += eps
        b[r, c] -= eps
        fd = (loss(qf, a) - loss(qf, b)) / (2 * eps)
        assert abs(fd - dkv[r, c]) <= 1e-5 * max(1.0, abs(fd)), (r, c, fd, dkv[r, c])


def test_bwd_closed_forms(oracle_mod):
    """Summed over latent rows, the values' share of dKV is the sum of dO over
    the non-empty (query, head) rows and the keys' share is zero; narrower
    values leave the key-only columns with the keys' share alone."""
    q, kv, idx, d_out = _case(7, Tq=8, H=4, D=40, N=30, W=64, d_v=32)
    idx[2] = -1
    scale = 0.2
    dq, dkv = oracle_mod.sparse_mla_bwd(q, kv, idx, d_out, scale)
    g = bf16_bits_to_f32(d_out).astype(np.float64)
    nonempty = np.array([np.any((r >= 0) & (r < kv.shape[0])) for r in idx])
    want_v = g[nonempty].sum(axis=(0, 1))
    tot = dkv.astype(np.float64).sum(axis=0)
    assert np.allclose(tot[:32], want_v, rtol=1e-5, atol=1e-4)
    assert np.allclose(tot[32:], 0.0, atol=1e-4)
    # one valid entry: the softmax is constant, so no gradient reaches q
    idx1 = np.full((1, 64), -1, np.int32)
    idx1[0, 17] = 5
    dq1, dkv1 = oracle_mod.sparse_mla_bwd(q[:1], kv, idx1, d_out[:1], scale)
    assert np.all(dq1 == 0)
    assert np.allclose(dkv1[5, :32], g[0].sum(axis=0), rtol=1e-6)       # that row takes dO as its value
    assert np.all(np.delete(dkv1, 5, axis=0) == 0)


def test_narrow_value_forward_equals_sdpa(oracle_mod):
    q, kv, idx, _ = _case(3, Tq=5, H=4, D=72, N=50, W=64, d_v=64)
    scale = 1 / np.sqrt(72)
    out, lse = oracle_mod.sparse_mla_dv(q, kv, idx, scale, 64)
    qf = torch.tensor(bf16_bits_to_f32(q), dtype=torch.float64).permute(1, 0, 2)   # [H, Tq, D]
    kvf = torch.tensor(bf16_bits_to_f32(kv), dtype=torch.float64)
    mask = np.zeros((q.shape[0], kv.shape[0]), bool)
    count = np.zeros((q.shape[0], kv.shape[0]))
    for i in range(q.shape[0]):
        for r in idx[i]:
            if 0 <= r < kv.shape[0]:
                count[i, r] += 1
    # repeated entries weigh their row count times: add log(count) to the logits
    bias = torch.tensor(np.where(count > 0, np.log(np.maximum(count, 1)), -np.inf))[None]
    K = kvf[None].expand(q.shape[1], -1, -1)
    V = kvf[:, :64][None].expand(q.shape[1], -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qf, K, V, attn_mask=bias, scale=scale)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-6, atol=1e-6)
    # with values as wide as the keys it is the ordinary forward
    o1, l1 = oracle_mod.sparse_mla_dv(q, kv, idx, scale, 72)
    o2, l2 = oracle_mod.sparse_mla(q, kv, idx, scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
