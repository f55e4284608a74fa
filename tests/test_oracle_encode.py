"""Pins of the oracle's k-pool compression, Hadamard rotation and E4M3 code.

Pooling: per-channel softmax(gate + ape)-weighted mean of each group of 4
(prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet). Rotation: fp32
butterfly Hadamard of queries and pooled keys before FP8 scoring (same bullet).
E4M3FN: the OCP 8-bit floating point format (4 exponent bits, bias 7, 3
mantissa bits, no infinities, max 448).
"""
import numpy as np
import pytest
import scipy.linalg
import torch

from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------------ pooling --
def test_pool_identical_rows_give_the_row(oracle_mod):
    rng = np.random.default_rng(0)
    d, kp, P = 32, 4, 9
    row = rng.standard_normal((P, d)).astype(np.float32)
    k = _bf16(np.repeat(row, kp, axis=0))
    gate = _bf16(rng.standard_normal((P * kp, d)) * 3)
    ape = rng.standard_normal((kp, d)).astype(np.float32)
    out = oracle_mod.pool(k, gate, ape, np.arange(0, P * kp, kp, dtype=np.int32), kp)
    assert np.array_equal(out, bf16_bits_to_f32(k[::kp]))


def test_pool_constant_logits_give_the_mean(oracle_mod):
    rng = np.random.default_rng(1)
    d, kp, P = 128, 4, 7
    k = _bf16(rng.standard_normal((P * kp, d)))
    gate = _bf16(np.full((P * kp, d), 0.75))
    ape = np.zeros((kp, d), np.float32)
    out = oracle_mod.pool(k, gate, ape, np.arange(0, P * kp, kp, dtype=np.int32), kp)
    want = bf16_bits_to_f32(k).astype(np.float64).reshape(P, kp, d).mean(axis=1).astype(np.float32)
    assert np.array_equal(out, want)


def test_pool_one_hot_logit_selects_a_row(oracle_mod):
    rng = np.random.default_rng(2)
    d, kp, P = 32, 4, 5
    k = _bf16(rng.standard_normal((P * kp, d)))
    gate = _bf16(rng.standard_normal((P * kp, d)))
    hot = rng.integers(0, kp, size=(P, d))
    g = bf16_bits_to_f32(gate).reshape(P, kp, d).copy()
    for p in range(P):
        for c in range(d):
            g[p, hot[p, c], c] = 96.0
    ape = np.zeros((kp, d), np.float32)
    out = oracle_mod.pool(k, _bf16(g.reshape(P * kp, d)), ape,
                          np.arange(0, P * kp, kp, dtype=np.int32), kp)
    kk = bf16_bits_to_f32(k).reshape(P, kp, d)
    want = np.take_along_axis(kk, hot[:, None, :], axis=1)[:, 0, :]
    assert np.array_equal(out, want)


def test_pool_shift_invariance_and_ape_position(oracle_mod):
    """Adding one constant to every logit of a channel changes nothing; ape is
    a per-position bias: moving it into the gate of the token at that position
    gives the same pooled key."""
    rng = np.random.default_rng(3)
    d, kp, P = 32, 4, 6
    k = _bf16(rng.standard_normal((P * kp, d)))
    # eighths in [-4, 4] and [-2, 2]: every sum below is exact in bf16 and fp32
    gate8 = rng.integers(-32, 33, size=(P * kp, d)).astype(np.float32) / 8
    ape8 = rng.integers(-16, 17, size=(kp, d)).astype(np.float32) / 8
    ps = np.arange(0, P * kp, kp, dtype=np.int32)
    base = oracle_mod.pool(k, _bf16(gate8), ape8, ps, kp)
    assert np.array_equal(base, oracle_mod.pool(k, _bf16(gate8 + 1.5), ape8, ps, kp))
    assert np.array_equal(base, oracle_mod.pool(k, _bf16(gate8), ape8 - 0.75, ps, kp))
    moved = (gate8.reshape(P, kp, d) + ape8[None]).reshape(P * kp, d)
    assert np.array_equal(base, oracle_mod.pool(k, _bf16(moved), np.zeros_like(ape8), ps, kp))
    assert not np.array_equal(base, oracle_mod.pool(k, _bf16(gate8), np.zeros_like(ape8), ps, kp))


def test_pool_vs_torch_softmax(oracle_mod):
    rng = np.random.default_rng(4)
    d, kp = 128, 4
    cu = np.array([0, 10, 31, 64], np.int32)
    T = 64
    k = _bf16(rng.standard_normal((T, d)))
    gate = _bf16(rng.standard_normal((T, d)) * 2)
    ape = rng.standard_normal((kp, d)).astype(np.float32)
    _, ps = oracle_mod.layout(cu, T, kp)
    out = oracle_mod.pool(k, gate, ape, ps, kp)
    kk = torch.from_numpy(bf16_bits_to_f32(k)).double()
    gg = torch.from_numpy(bf16_bits_to_f32(gate)).double()
    aa = torch.from_numpy(ape).double()
    for p, s in enumerate(ps):
        wts = torch.softmax(gg[s:s + kp] + aa, dim=0)
        ref = (wts * kk[s:s + kp]).sum(0)
        assert np.allclose(out[p], ref.numpy(), rtol=1e-6, atol=1e-7)


# -------------------------------------------------------------------- FWHT --
@pytest.mark.parametrize("n", [32, 64, 128])
def test_fwht_is_the_normalised_sylvester_matrix(oracle_mod, n):
    H = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    assert np.allclose(H @ H.T, np.eye(n), atol=1e-12)            # orthonormal
    rng = np.random.default_rng(n)
    X = rng.standard_normal((40, n)).astype(np.float32)
    Y = oracle_mod.fwht(X)
    ref = X.astype(np.float64) @ H.T
    assert np.allclose(Y, ref, rtol=1e-5, atol=1e-5)
    # columns of the identity map to the rows of H
    E = oracle_mod.fwht(np.eye(n, dtype=np.float32))
    assert np.allclose(E, H, atol=1e-7)


@pytest.mark.parametrize("n", [32, 128])
def test_fwht_involution_and_dot_products(oracle_mod, n):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((16, n)).astype(np.float32)
    k = rng.standard_normal((16, n)).astype(np.float32)
    assert np.allclose(oracle_mod.fwht(oracle_mod.fwht(q)), q, rtol=1e-5, atol=1e-6)
    hq, hk = oracle_mod.fwht(q), oracle_mod.fwht(k)
    assert np.allclose((hq.astype(np.float64) * hk).sum(1), (q.astype(np.float64) * k).sum(1),
                       rtol=1e-5, atol=1e-4)
    assert np.allclose(np.linalg.norm(hq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-6)


# -------------------------------------------------------------------- E4M3 --
def test_e4m3_decode_all_codes_vs_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_mod.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and set(codes[nan].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_finite_codes_round_trip(oracle_mod):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle_mod.e4m3_decode(codes)
    back = oracle_mod.e4m3_encode(vals)
    back[codes == 0x80] = 0x80        # -0 encodes to 0x80 (sign kept)
    assert np.array_equal(back, codes)


def test_e4m3_encode_vs_torch_rne(oracle_mod):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000) * 100,
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(5000) * 0.01,                  # subnormal range
    ]).astype(np.float32)
    # every midpoint between neighbouring finite values, where ties-to-even decides
    pos = np.sort(np.unique(oracle_mod.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = oracle_mod.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates(oracle_mod):
    big = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e6, -470.0], np.float32)
    codes = oracle_mod.e4m3_encode(big)
    assert codes.tolist() == [0x7E] * 6 + [0xFE]


def test_quant_rows_maps_amax_to_448(oracle_mod):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    x[3] = 0.0
    codes, scales = oracle_mod.quant_rows(x)
    dec = oracle_mod.e4m3_decode(codes)
    for r in range(50):
        if r == 3:
            assert scales[r] == 1.0 and not codes[r].any()
            continue
        j = int(np.argmax(np.abs(x[r])))
        assert abs(dec[r, j]) == 448.0
        assert scales[r] == np.float32(np.abs(x[r]).max()) / np.float32(448.0)
        # dequantised values are within half a quantum (relative 2^-4) of the input
        rel = np.abs(dec[r] * scales[r] - x[r]) / np.maximum(np.abs(x[r]), 2.0 ** -6 * scales[r])
        assert rel.max() <= 2.0 ** -4 + 1e-6
