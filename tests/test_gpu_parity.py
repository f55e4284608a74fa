"""GPU parity: every stage of the HIP path against the CPU oracle, through the
C ABI, on the same seeded inputs. Each GPU stage is fed the oracle's upstream
outputs so that errors do not compound; the end-to-end tests then run the
GPU pipeline alone and compare what is unique (layout, selection where it
covers every pool, attention on the oracle's rows).

Bars: layout and index rows bit-exact; query FP8 codes bit-exact (same fp32
butterfly order and IEEE division on both sides); pooled keys within fp32
rounding with at most rare one-step FP8 code flips; scores, attention and lse
within the tolerances of tests/_util.py.
"""
import numpy as np
import pytest
import torch

from tests._util import (OUT_MAX, check_key_codes, check_lse, check_out, check_scores, dev, dev_bf16, host, host_bf16_f32)
from workloads import Workload, custom, spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_kpool_amd as K
    K.lib()
    return K


def _log(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- layout -----
LAYOUT_ROWS = [
    [0, 64], [0, 2048], [0, 3, 11, 11, 20, 24, 25], [0, 1, 2, 3, 4, 5, 6, 7],
    [0, 0, 0, 9], [0, 5, 5, 5, 100, 101, 333, 1000],
]


@pytest.mark.parametrize("cu", LAYOUT_ROWS + ["rand%d" % s for s in range(5)])
def test_layout_bitexact(K, oracle_mod, cu):
    if isinstance(cu, str):
        rng = np.random.default_rng(int(cu[4:]))
        lens = rng.integers(0, 40, size=int(rng.integers(1, 30)))
        lens[rng.random(len(lens)) < 0.15] = 0
        lens[0] += 1
        cu = [0, *np.cumsum(lens).tolist()]
    cu = np.array(cu, np.int32)
    T = int(cu[-1])
    _log("layout", cu.tolist()[:12])
    s = custom("lay", T, cu, D_I=32)
    wl = Workload(s)
    cp, ps, k8, ks, _ = K.kpool_build(dev(cu), dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")),
                                      dev(wl.ape()), 4)
    want_cp, want_ps = oracle_mod.layout(cu, T, 4)
    assert host(cp).tolist() == want_cp.tolist()
    got_ps = host(ps)
    assert got_ps[:len(want_ps)].tolist() == want_ps.tolist()
    assert np.all(got_ps[len(want_ps):] == -1)


# ------------------------------------------------------------ pooled keys ----
@pytest.mark.parametrize("name", ["tiny", "2k", "packed4k"])
def test_pooled_keys(K, oracle_mod, name):
    s = spec(name)
    wl = Workload(s)
    _log("keys", name)
    cp, ps, k8, ks, kf = K.kpool_build(dev(s.cu), dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")),
                                       dev(wl.ape()), s.kpool, with_f32=True)
    _, want_ps = oracle_mod.layout(s.cu, s.T, s.kpool)
    kc, kscale, pooled = oracle_mod.keys(wl.full("k_idx"), wl.full("gate"), wl.ape(), want_ps, s.kpool)
    P = len(want_ps)
    g_pooled = host(kf)[:P]
    assert np.all(np.abs(g_pooled - pooled) <= 1e-5 * np.abs(pooled) + 1e-6)
    check_key_codes(host(k8)[:P], kc, name)
    assert np.allclose(host(ks)[:P], kscale, rtol=1e-5)


@pytest.mark.parametrize("ndocs,seed", [(1, 11), (1024, 12), (1025, 13), (3000, 14), (1024, 15)])
def test_layout_and_keys_many_documents(K, oracle_mod, ndocs, seed):
    """Rows of one document (layout known on the host), of up to 1,024 documents
    (layout scanned inside the pooling launch) and of more (a separate layout
    scan first): layout bit-exact and pooled keys as the oracle computes them.
    Seed 15 gives a quarter of the 1,024 documents no tokens."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 14, size=ndocs)
    if seed == 15:
        lens[rng.random(ndocs) < 0.25] = 0
        lens[0] += 1
    cu = np.array([0, *np.cumsum(lens).tolist()], np.int32)
    T = int(cu[-1])
    _log("many documents", ndocs, "T", T)
    s = custom("many", T, cu, D_I=32)
    wl = Workload(s)
    cp, ps, k8, ks, kf = K.kpool_build(dev(cu), dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")),
                                       dev(wl.ape()), 4, with_f32=True)
    want_cp, want_ps = oracle_mod.layout(cu, T, 4)
    assert host(cp).tolist() == want_cp.tolist()
    got_ps = host(ps)
    P = len(want_ps)
    assert got_ps[:P].tolist() == want_ps.tolist()
    assert np.all(got_ps[P:] == -1)
    kc, kscale, pooled = oracle_mod.keys(wl.full("k_idx"), wl.full("gate"), wl.ape(), want_ps, 4)
    g_pooled = host(kf)[:P]
    assert np.all(np.abs(g_pooled - pooled) <= 1e-5 * np.abs(pooled) + 1e-6)
    check_key_codes(host(k8)[:P], kc, "many%d" % ndocs)
    assert np.allclose(host(ks)[:P], kscale, rtol=1e-5)
    assert np.all(host(ks)[P:] == 0) and np.all(host(k8)[P:] == 0)


@pytest.mark.parametrize("name", ["tiny", "2k", "packed4k"])
def test_pooled_keys_from_token(K, name):
    """kpool_build_from rebuilds exactly the pools that end at or after token_lo
    (bit for bit as kpool_build writes them) and the rows past the last pool,
    and leaves the rows of earlier pools (the caller's cache) as they were."""
    s = spec(name)
    wl = Workload(s)
    args = (dev(s.cu), dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")), dev(wl.ape()))
    ref = [host(t) for t in K.kpool_build(*args, s.kpool, with_f32=True)]
    ref_cp, ref_ps = ref[0], ref[1]
    P = int(ref_cp[-1])
    ends = np.full(len(ref_ps), -1, np.int64)
    ends[:P] = ref_ps[:P].astype(np.int64) + s.kpool - 1
    starts = s.cu[:-1]
    cases = sorted({0, 1, s.T // 2, s.T // 2 + 1, int(starts[-1]), s.T - 1, s.T - s.kpool, s.T})
    for token_lo in cases:
        out = K.kpool_build(*args, s.kpool, with_f32=True)
        cached = ends < token_lo          # rows of pools the call must not write (rows >= P are rebuilt)
        cached[P:] = False
        # sentinels everywhere: the cache rows must keep theirs, every other row must be rebuilt
        out[0].fill_(-7)
        out[1].fill_(-9)
        out[2].fill_(0x5A)
        out[3].fill_(3.5)
        out[4].fill_(-1.25)
        K.kpool_build_from(*args, token_lo, out, s.kpool)
        got = [host(t) for t in out]
        _log("keys from", name, token_lo, int(cached.sum()), "cached of", len(ends))
        assert np.array_equal(got[0], ref_cp)
        keep = ~cached
        for g, r, sentinel in zip(got[1:], ref[1:], (-9, 0x5A, 3.5, -1.25)):
            assert np.array_equal(g[keep], r[keep]), f"token_lo {token_lo}: a rebuilt row differs"
            assert np.all(g[cached] == sentinel), f"token_lo {token_lo}: a cached row was written"


@pytest.mark.parametrize("name", ["tiny", "2k", "packed4k"])
def test_query_codes_bitexact(K, oracle_mod, name):
    s = spec(name)
    wl = Workload(s)
    q_idx = wl.full("q_idx")
    _log("query codes", name, q_idx.shape)
    codes, scales = K.indexer_rotate_quant(dev_bf16(q_idx))
    qc, qs = oracle_mod.queries(q_idx)
    assert np.array_equal(host(codes), qc)
    assert np.array_equal(host(scales), qs)


@pytest.mark.parametrize("tq,h,d", [(7, 3, 128), (5, 5, 64), (3, 7, 32), (1, 1, 128), (1001, 32, 128),
                                    (333, 9, 64)])
def test_query_codes_ragged(K, oracle_mod, tq, h, d):
    """Vector counts that leave the last block of the rotation partly filled,
    for each supported width, with one all-zero vector (scale 1, zero codes)."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(1000 + tq * 31 + h * 7 + d)
    x = rng.standard_normal((tq, h, d)).astype(np.float32) * 3.0
    x[tq // 2, h // 2] = 0.0
    q_idx = f32_to_bf16_bits(x)
    _log("query codes ragged", (tq, h, d))
    codes, scales = K.indexer_rotate_quant(dev_bf16(q_idx))
    qc, qs = oracle_mod.queries(q_idx)
    assert np.array_equal(host(codes), qc)
    assert np.array_equal(host(scales), qs)
    assert qs[tq // 2, h // 2] == 1.0


# ---------------------------------------------------------------- scoring ----
def _oracle_keys(oracle_mod, s, wl):
    cp, ps = oracle_mod.layout(s.cu, s.T, s.kpool)
    kc, kscale, _ = oracle_mod.keys(wl.full("k_idx"), wl.full("gate"), wl.ape(), ps, s.kpool)
    # capacity rows past the last pool: zero codes and scale, as the library writes them
    cap = s.max_pools
    k8 = np.zeros((cap, s.D_I), np.uint8)
    k8[:len(ps)] = kc
    sk = np.zeros(cap, np.float32)
    sk[:len(ps)] = kscale
    return cp, ps, k8, sk


def _gpu_scores(K, s, wl, cp, k8, sk, rows=None):
    qpos = s.query_positions()
    q_idx = wl.full("q_idx")
    w = wl.full("w")
    if rows is not None:
        qpos, q_idx, w = qpos[rows], q_idx[rows], w[rows]
    idx, nv, sc = K.indexer_score_topk(dev(s.cu), dev(cp), dev(k8), dev(sk), dev_bf16(q_idx), dev(w), s.T,
                                       s.kpool, s.topk, q_pos=dev(qpos.astype(np.int32)), return_scores=True)
    return host(idx), host(nv), host(sc)


@pytest.mark.parametrize("name", ["tiny", "2k", "packed4k", "32k_rows", "decode1m_rows", "decode1m_tiles2"])
def test_scores_fed_oracle_keys(K, oracle_mod, name):
    """decode1m_tiles2: 17 decode queries make two query tiles, so each tile's
    pools are split over fewer workgroups than there are 512-pool chunks and
    every workgroup walks several chunks."""
    base = name.replace("_rows", "").replace("_tiles2", "")
    s = spec(base)
    wl = Workload(s)
    rng = np.random.default_rng(0)
    rows = None
    if name.endswith("_rows"):
        nr = 4 if base == "decode1m" else 12
        rows = np.unique(np.concatenate([rng.choice(s.Tq, nr, replace=False), [0, s.Tq - 1]]))
    if name.endswith("_tiles2"):
        rows = np.append(np.arange(0, s.Tq, 4), s.Tq - 1)
    _log("scores", name, "rows", None if rows is None else rows.tolist())
    cp, ps, k8, sk = _oracle_keys(oracle_mod, s, wl)
    _, _, g_sc = _gpu_scores(K, s, wl, cp, k8, sk, rows)
    qpos = s.query_positions() if rows is None else s.query_positions()[rows]
    q_idx = wl.full("q_idx") if rows is None else wl.full("q_idx")[rows]
    w = wl.full("w") if rows is None else wl.full("w")[rows]
    qc, qs = oracle_mod.queries(q_idx)
    ref = oracle_mod.scores(s.cu, cp, s.kpool, qpos, s.max_pools, w, qc, qs, k8[:len(ps)], sk[:len(ps)])
    info = check_scores(g_sc, ref, name)
    _log("  worst rel", info)


# ------------------------------------------------------------------ top-k -----
@pytest.mark.parametrize("case", ["tiny", "2k", "packed4k", "ties", "zeros", "negzero", "nan", "topk0",
                                  "decode1m_rows", "long_rand", "long_ties", "long_zeros", "long_nan",
                                  "long_bigk", "long_smallk", "mid_rand", "mid_ties", "mid_nan",
                                  "mid_sampled_top", "mid_multidoc", "mid_multidoc_nan"])
def test_topk_from_oracle_scores_bitexact(K, oracle_mod, case):
    rng = np.random.default_rng(7)
    if case in ("tiny", "2k", "packed4k"):
        s = spec(case)
        wl = Workload(s)
        cp, ps, k8, sk = _oracle_keys(oracle_mod, s, wl)
        qc, qs = oracle_mod.queries(wl.full("q_idx"))
        qpos = s.query_positions()
        sc = oracle_mod.scores(s.cu, cp, s.kpool, qpos, s.max_pools, wl.full("w"), qc, qs, k8[:len(ps)],
                               sk[:len(ps)])
        T, topk, cu = s.T, s.topk, s.cu
    elif case == "decode1m_rows":
        s = spec("decode1m")
        wl = Workload(s)
        cp, ps, k8, sk = _oracle_keys(oracle_mod, s, wl)
        rows = np.array([0, 31, 63])
        qpos = s.query_positions()[rows]
        qc, qs = oracle_mod.queries(wl.full("q_idx")[rows])
        sc = oracle_mod.scores(s.cu, cp, s.kpool, qpos, s.max_pools, wl.full("w")[rows], qc, qs, k8[:len(ps)],
                               sk[:len(ps)])
        T, topk, cu = s.T, s.topk, s.cu
    elif case.startswith("long_"):
        # rows with more visible pools than the short-row kernel caches (decode-like),
        # mixed with short rows in the same launch
        T = 65536
        cu = np.array([0, T], np.int32)
        cp, _ = oracle_mod.layout(cu, T, 4)
        qpos = np.array([100, 32770, 32771, 33000, 35000, 40000, 45000, 50001, 60000, 65533, 65534, 65535],
                        np.int32)
        sc = rng.standard_normal((len(qpos), T // 4)).astype(np.float32)
        if case == "long_ties":
            sc = np.round(sc * 2).astype(np.float32)          # heavy ties: the k-th score is shared
        if case == "long_zeros":
            sc = np.maximum(np.round(sc * 2), 0).astype(np.float32)
        if case == "long_nan":
            sc[rng.random(sc.shape) < 0.01] = np.nan
            sc[rng.random(sc.shape) < 0.01] = -np.inf
            sc[rng.random(sc.shape) < 0.2] = -0.0
        # (a small k leaves the rows no room for the many-workgroup scratch: the
        # one-workgroup long-row kernel runs instead)
        topk = 5000 if case == "long_bigk" else (37 if case == "long_smallk" else 512)
    elif case.startswith("mid_multidoc"):
        # documents whose first pools sit 1, 2 and 1 floats past a 16-byte boundary
        # of the score rows (a stride of 8192 pools: the 16-byte-load layout)
        T = 32768
        cu = np.array([0, 4101, 4105, 16390, 32768], np.int32)
        cp, _ = oracle_mod.layout(cu, T, 4)
        qpos = np.array([0, 3, 2000, 4100, 4101, 4104, 4200, 9000, 12291, 16389, 16390, 16393, 17000, 24000,
                         28675, 32767], np.int32)
        sc = rng.standard_normal((len(qpos), T // 4)).astype(np.float32)
        if case == "mid_multidoc_nan":
            sc = np.round(sc * 2).astype(np.float32)
            sc[rng.random(sc.shape) < 0.02] = np.nan
            sc[rng.random(sc.shape) < 0.2] = -0.0
        topk = 512
    elif case.startswith("mid_"):
        # rows of up to 8192 pools (the one-wave-per-row kernels: rows of 2048 or
        # more pools first bound the histogrammed keys from 64 sampled pools)
        T = 32768
        cu = np.array([0, T], np.int32)
        cp, _ = oracle_mod.layout(cu, T, 4)
        qpos = np.array([5, 4000, 8191, 8195, 9000, 12000, 16383, 16387, 16390, 20000, 24575, 28000, 30001,
                         32766, 32767], np.int32)
        sc = rng.standard_normal((len(qpos), T // 4)).astype(np.float32)
        if case == "mid_ties":
            sc = np.round(sc * 2).astype(np.float32)
        if case == "mid_nan":
            sc[rng.random(sc.shape) < 0.01] = np.nan
            sc[rng.random(sc.shape) < 0.01] = -np.inf
            sc[rng.random(sc.shape) < 0.2] = -0.0
        if case == "mid_sampled_top":
            # the 64 sampled pools of each row hold its largest scores: fewer than
            # top-k pools lie above the sampled bound, so the row is selected again
            # over every key
            for r, t in enumerate(qpos):
                n = (int(t) + 1) // 4
                if n >= 64:
                    sc[r, (np.arange(64) * n) >> 6] = 100.0 + np.arange(64)
        topk = 512
    else:
        T = 5000
        cu = np.array([0, 700, 700, 2900, 2903, 5000], np.int32)
        cp, _ = oracle_mod.layout(cu, T, 4)
        qpos = np.arange(T, dtype=np.int32)
        sc = np.round(rng.standard_normal((T, T // 4)) * 2).astype(np.float32)     # heavy ties
        if case == "zeros":
            sc = np.maximum(sc, 0).astype(np.float32)
        if case == "negzero":
            sc[rng.random(sc.shape) < 0.3] = -0.0
            sc[rng.random(sc.shape) < 0.3] = 0.0
        if case == "nan":
            sc[rng.random(sc.shape) < 0.01] = np.nan
            sc[rng.random(sc.shape) < 0.01] = -np.inf
        topk = 0 if case == "topk0" else 37
    W = -(-(4 * topk + 3) // 128) * 128
    _log("topk", case, sc.shape, topk)
    ref_idx, ref_nv = oracle_mod.topk(cu, cp, 4, qpos, sc, topk, W)
    g_idx, g_nv = K.indexer_topk_from_scores(dev(cu), dev(cp), dev(sc), T, 4, topk, W, q_pos=dev(qpos))
    g_idx, g_nv = host(g_idx), host(g_nv)
    assert np.array_equal(g_nv, ref_nv)
    bad = np.nonzero(np.any(g_idx != ref_idx, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"


# ------------------------------------------------------------ sparse MLA -----
def _oracle_rows(oracle_mod, s, wl, rows):
    res = oracle_mod.dsa_forward(wl, q_rows=rows, with_mla=False)
    return res["indices"], res["num_valid"]


@pytest.mark.parametrize("name", ["tiny", "2k", "packed4k", "32k_rows", "decode1m_rows"])
def test_mla_fed_oracle_rows(K, oracle_mod, name):
    base = name.replace("_rows", "")
    s = spec(base)
    wl = Workload(s)
    rows = np.arange(s.Tq)
    if name.endswith("_rows"):
        rng = np.random.default_rng(1)
        nr = 3 if base == "decode1m" else 10
        rows = np.unique(np.concatenate([rng.choice(s.Tq, nr, replace=False), [0, 1, 2, 3, s.Tq - 1]]))
    elif s.Tq > 512:
        rows = np.unique(np.concatenate([np.arange(0, s.Tq, 97), [s.Tq - 1]]))
    _log("mla", name, len(rows))
    idx, nv = _oracle_rows(oracle_mod, s, wl, rows)
    q = wl.full("q")[rows] if s.Tq * s.H * s.D <= (1 << 28) else \
        np.concatenate([wl.rows("q", int(r), int(r) + 1) for r in rows])
    kv = wl.full("kv")
    g_out, g_lse = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv), dev(idx), s.scale)
    ref_out, ref_lse, ref_abs = oracle_mod.sparse_mla(q, kv, idx, s.scale, with_abs=True)
    scaled = s.boost_frac > 0          # the 32K workload's x8 latent rows
    info = check_out(host_bf16_f32(g_out), ref_out, name, ref_abs, scaled=scaled)
    info["lse"] = check_lse(host(g_lse), ref_lse, name, scaled=scaled)
    _log("  ", info)


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("case", ["scattered_mask", "empty_rows", "single", "duplicates", "heads40",
                                  "rising", "rising_tail", "max_width", "w2_width", "above_w2_width"])
def test_mla_edge_rows(K, oracle_mod, case, split):
    """Edge rows of the attention. "rising" and "rising_tail" put rows whose
    scores lie hundreds of log2 units above those of the first tile after it
    (from the second tile on, or only in the last tile): a pass that takes its
    softmax reference from the first tile cannot hold them, so the kernel must
    fall back to its exact-max passes and still agree with the oracle. With
    split, these few-query launches cut each row into tile ranges (2 to 16)
    that are merged afterwards; without, one workgroup takes each row."""
    rng = np.random.default_rng(3)
    H, D, N, W, Tq = 64, 512, 3000, 256, 9
    if case == "heads40":
        H = 40
    if case == "max_width":   # the widest index row the attention accepts: 64 tiles of rows
        W, Tq = 4096, 3
    if case == "w2_width":    # the widest row of the two-wave form (its LDS list), whole rows
        W, Tq = 2560, 3
    if case == "above_w2_width":   # one 128-entry step wider: the four-wave form takes it
        W, Tq = 2688, 3
    q = (rng.standard_normal((Tq, H, D))).astype(np.float32)
    kv = (rng.standard_normal((N, D))).astype(np.float32)
    if case.startswith("rising"):
        kv[N // 2:] *= 100.0   # scores of these rows: ~100x larger
    from workloads import f32_to_bf16_bits
    q, kv = f32_to_bf16_bits(q), f32_to_bf16_bits(kv)
    idx = rng.integers(0, N, size=(Tq, W)).astype(np.int32)
    if case == "rising":   # first tile from the small rows, the rest from the large ones
        idx[:, :64] = rng.integers(0, N // 2, size=(Tq, 64))
        idx[:, 64:] = rng.integers(N // 2, N, size=(Tq, W - 64))
    if case == "rising_tail":   # large rows only in the last tile
        idx[:, :W - 8] = rng.integers(0, N // 2, size=(Tq, W - 8))
        idx[:, W - 8:] = rng.integers(N // 2, N, size=(Tq, 8))
    if case == "scattered_mask":
        m = rng.random(idx.shape) < 0.4
        idx[m] = rng.choice([-1, -5, N, N + 7, 2 ** 31 - 1], size=m.sum())
    if case == "empty_rows":
        idx[::2] = -1
    if case == "single":
        idx[:] = -1
        idx[np.arange(Tq), rng.integers(0, W, Tq)] = rng.integers(0, N, Tq)
    if case == "duplicates":
        idx[:, 100:] = idx[:, :W - 100][:, :W - 100]
    if case in ("max_width", "w2_width", "above_w2_width"):
        # row 0 full; rows 1, 2 with masked entries spread over the row
        idx[1:][rng.random((Tq - 1, W)) < 0.3] = -1
        idx[2, W - 50:] = -1
    _log("mla edge", case, "split" if split else "whole rows")
    g_out, g_lse = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv), dev(idx), 1 / np.sqrt(D), split=split)
    # (errors are scaled by sum_j p_j |v_j|, as in the fed-oracle test: the bf16
    # weights perturb each p_j by up to 2^-9 of itself, which moves an output by
    # that much of the spread of the values it mixes)
    ref_out, ref_lse, ref_abs = oracle_mod.sparse_mla(q, kv, idx, 1 / np.sqrt(D), with_abs=True)
    scaled = case.startswith("rising")   # x100 latent rows
    info = check_out(host_bf16_f32(g_out), ref_out, case, ref_abs=ref_abs, scaled=scaled)
    info["lse"] = check_lse(host(g_lse), ref_lse, case, scaled=scaled)
    _log("  ", info)


@pytest.mark.parametrize("case", ["d512", "d512_h24", "d64", "d512_few", "d64_few", "d512_h40_few"])
def test_mla_many_queries(K, oracle_mod, case):
    """More queries than the GPU has compute units, so that every workgroup
    takes several queries in turn, with row kinds interleaved so that
    neighbouring queries of a workgroup differ: empty rows, full rows, ragged
    short rows, scattered masks, single entries, and rows that force the
    exact-max passes (from the second tile on, or in the last tile only).
    The *_few cases have fewer workgroups than twice the compute units (a
    decode-sized launch), one of them with 40 heads."""
    rng = np.random.default_rng(11)
    H, D, N, W, Tq = 64, 512, 3000, 192, 777
    if case == "d512_h24":
        H = 24
    if case.startswith("d64"):
        D = 64
    if case.endswith("_few"):
        Tq = 300
    if case == "d512_h40_few":
        H = 40
    q = (rng.standard_normal((Tq, H, D))).astype(np.float32)
    kv = (rng.standard_normal((N, D))).astype(np.float32)
    kv[N // 2:] *= 100.0   # rows whose scores lie far above those of the others
    from workloads import f32_to_bf16_bits
    q, kv = f32_to_bf16_bits(q), f32_to_bf16_bits(kv)
    small = lambda n: rng.integers(0, N // 2, size=n)
    idx = np.empty((Tq, W), np.int32)
    for r in range(Tq):
        kind = r % 7
        row = small(W)
        if kind == 0:
            row[:] = -1
        elif kind == 2:   # rising: large rows after the first tile
            row[64:] = rng.integers(N // 2, N, size=W - 64)
        elif kind == 3:
            m = rng.random(W) < 0.4
            row[m] = rng.choice([-1, N, 2 ** 31 - 1], size=m.sum())
        elif kind == 4:
            j = rng.integers(0, W)
            row[:] = -1
            row[j] = rng.integers(0, N)
        elif kind == 5:   # rising in the last tile only
            row[W - 5:] = rng.integers(N // 2, N, size=5)
        elif kind == 6:
            row[70:] = -1
        idx[r] = row
    _log("mla many", case, Tq, H, D)
    g_out, g_lse = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv), dev(idx), 1 / np.sqrt(D))
    ref_out, ref_lse, ref_abs = oracle_mod.sparse_mla(q, kv, idx, 1 / np.sqrt(D), with_abs=True)
    # (half the latent rows are scaled by 100: a scaled check)
    info = check_out(host_bf16_f32(g_out), ref_out, case, ref_abs=ref_abs, scaled=True)
    info["lse"] = check_lse(host(g_lse), ref_lse, case, scaled=True)
    _log("  ", info)


@pytest.mark.parametrize("D", [512, 576, 64])
def test_mla_split_decode(K, oracle_mod, D):
    """A decode-shaped launch (64 queries, rows of 2176 entries, or 2048 for
    576-wide keys: four tile ranges per row) with ragged, masked, empty and single-entry rows: the split
    path against the oracle, and against the whole-row path to within the
    bf16 rounding of the output (each path rounds its fp32 result once)."""
    rng = np.random.default_rng(17)
    H, N, Tq = 64, 5000, 64
    W = 2048 if D == 576 else 2176                # (576-wide keys take rows of at most 2048)
    from workloads import f32_to_bf16_bits
    q = f32_to_bf16_bits(rng.standard_normal((Tq, H, D)))
    kv = f32_to_bf16_bits(rng.standard_normal((N, D)))
    idx = rng.integers(0, N, size=(Tq, W)).astype(np.int32)
    idx[1] = -1                                   # empty
    idx[2, :] = -1
    idx[2, 1500] = 9                              # one entry, in the third range
    idx[3, 600:] = -1                             # ragged: the later ranges are empty
    idx[4][rng.random(W) < 0.5] = -1              # scattered masks
    nd = min(2051, W)
    idx[5, :nd] = rng.integers(0, N, nd)          # the decode row: 2051 entries, then padding
    idx[5, nd:] = -1
    assert K.kp_mla_fwd_workspace_bytes(Tq, H, D, W) > 0
    scale = 1 / np.sqrt(D)
    qd, kvd, idxd = dev_bf16(q), dev_bf16(kv), dev(idx)
    s_out, s_lse = K.sparse_mla_fwd(qd, kvd, idxd, scale, split=True)
    w_out, w_lse = K.sparse_mla_fwd(qd, kvd, idxd, scale, split=False)
    dv = 512 if D == 576 else D
    if D == 576:
        ref_out, ref_lse, ref_abs = oracle_mod.sparse_mla_dv(q, kv, idx, scale, 512, with_abs=True)
    else:
        ref_out, ref_lse, ref_abs = oracle_mod.sparse_mla(q, kv, idx, scale, with_abs=True)
    info = check_out(host_bf16_f32(s_out), ref_out, f"split D={D}", ref_abs=ref_abs)
    info["lse"] = check_lse(host(s_lse), ref_lse, f"split D={D}")
    # two bf16 ulps of the larger of the output and the magnitude of the terms it sums
    a, b = host_bf16_f32(s_out).astype(np.float64), host_bf16_f32(w_out).astype(np.float64)
    unit = np.maximum(np.maximum(np.abs(b), ref_abs), 2.0 ** -100) * 2.0 ** -8
    info["split_vs_whole_ulps"] = float((np.abs(a - b) / unit).max())
    assert info["split_vs_whole_ulps"] <= 2.0, info
    assert np.array_equal(np.isneginf(host(s_lse)), np.isneginf(host(w_lse)))
    fin = np.isfinite(host(w_lse))
    info["lse_split_vs_whole"] = float(np.abs(host(s_lse)[fin] - host(w_lse)[fin]).max())
    assert info["lse_split_vs_whole"] <= 1e-4
    assert np.all(host_bf16_f32(s_out)[1] == 0) and s_out.shape == (Tq, H, dv)
    _log("  ", info)


# ------------------------------------------------------------ end to end -----
@pytest.mark.parametrize("name", ["tiny_dense", "2k"])
def test_end_to_end_dense_cover(K, oracle_mod, name):
    """Top-k covers every visible pool: the GPU pipeline's index rows must equal
    the oracle's bit for bit whatever the scores, and attention must match."""
    s = spec(name)
    wl = Workload(s)
    _log("e2e", name)
    out, lse, idx, nv = K.dsa_forward(dev(s.cu), dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")),
                                      dev(wl.ape()), dev_bf16(wl.full("q_idx")), dev(wl.full("w")),
                                      dev_bf16(wl.full("q")), dev_bf16(wl.full("kv")), kpool=s.kpool,
                                      topk_pools=s.topk, softmax_scale=s.scale)
    rows = np.arange(s.Tq) if s.Tq <= 64 else np.unique(np.concatenate([np.arange(0, s.Tq, 61), [s.Tq - 1]]))
    res = oracle_mod.dsa_forward(wl, q_rows=rows)
    assert np.array_equal(host(idx)[rows], res["indices"])
    assert np.array_equal(host(nv)[rows], res["num_valid"])
    info = check_out(host_bf16_f32(out)[rows], res["out"], name)
    info["lse"] = check_lse(host(lse)[rows], res["lse"], name)
    _log("  ", info)


@pytest.mark.parametrize("name", ["packed4k", "32k"])
def test_end_to_end_selection_agreement(K, oracle_mod, name):
    """GPU pipeline on its own: index rows stay in the query's document and at
    or before it, and agree with the oracle's selection (the two differ only
    where FP8 rounding of pooled keys flips a near-tie)."""
    s = spec(name)
    wl = Workload(s)
    _log("e2e selection", name)
    cu_d = dev(s.cu)
    cp, ps, k8, ks, _ = K.kpool_build(cu_d, dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")),
                                      dev(wl.ape()), s.kpool)
    idx, nv, _ = K.indexer_score_topk(cu_d, cp, k8, ks, dev_bf16(wl.full("q_idx")), dev(wl.full("w")), s.T,
                                      s.kpool, s.topk)
    idx, nv = host(idx), host(nv)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(s.Tq, 24, replace=False), [s.Tq - 1]]))
    res = oracle_mod.dsa_forward(wl, q_rows=rows, with_mla=False)
    doc = np.searchsorted(s.cu, np.arange(s.T), side="right") - 1
    jac = []
    for i, t in enumerate(rows):
        g = idx[t, :nv[t]]
        assert nv[t] == res["num_valid"][i]
        assert np.all(doc[g] == doc[t]) and np.all(g <= t) and np.all(np.diff(g) > 0)
        assert np.all(idx[t, nv[t]:] == -1)
        a, b = set(g.tolist()), set(res["indices"][i, :nv[t]].tolist())
        jac.append(len(a & b) / len(a | b))
    _log("  jaccard mean", np.mean(jac), "min", np.min(jac), "identical", np.mean(np.array(jac) == 1.0))
    assert np.mean(jac) >= 0.97


# -------------------------------------------------------- shared layers -----
@pytest.mark.parametrize("name", ["tiny_dense", "2k", "packed4k"])
def test_index_share(K, oracle_mod, name):
    """IndexShare: a second layer with its own q and latent reuses the first
    layer's index rows (no pooling, scoring or selection of its own). Its
    output must equal the oracle's attention of the second layer's q and
    latent over those same rows, and differ from the first layer's."""
    s = spec(name)
    wl = Workload(s)
    _log("index share", name)
    out_a, _, idx, nv = K.dsa_forward(dev(s.cu), dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")),
                                      dev(wl.ape()), dev_bf16(wl.full("q_idx")), dev(wl.full("w")),
                                      dev_bf16(wl.full("q")), dev_bf16(wl.full("kv")), kpool=s.kpool,
                                      topk_pools=s.topk, softmax_scale=s.scale)
    # the second layer: fresh q and latent of the same shapes (another seed)
    wl_b = Workload(spec(name).__class__(**{**spec(name).__dict__, "seed": s.seed + 100}))
    q_b, kv_b = wl_b.full("q"), wl_b.full("kv")
    out_b, lse_b = K.dsa_forward_shared(dev_bf16(q_b), dev_bf16(kv_b), idx, softmax_scale=s.scale)
    rows = np.arange(s.Tq) if s.Tq <= 64 else np.unique(np.concatenate([np.arange(0, s.Tq, 127), [s.Tq - 1]]))
    g_idx = host(idx)[rows]
    ref_out, ref_lse = oracle_mod.sparse_mla(q_b[rows], kv_b, g_idx, s.scale)
    info = check_out(host_bf16_f32(out_b)[rows], ref_out, name)
    info["lse"] = check_lse(host(lse_b)[rows], ref_lse, name)
    assert not torch.equal(out_a, out_b)
    # the full layer's rows are the oracle's where selection covers every pool
    if name != "packed4k":
        assert np.array_equal(g_idx, oracle_mod.dsa_forward(wl, q_rows=rows, with_mla=False)["indices"])
    _log("  ", info)


# ----------------------------------------------- 576-wide keys (RoPE tail) --
@pytest.mark.parametrize("case", ["dense_2k_rows", "scattered_mask", "single", "duplicates", "heads40",
                                  "rising", "max_width", "many_queries"])
def test_mla_rope_tail(K, oracle_mod, case):
    """Keys 576 wide (512 + a 64-wide RoPE tail), values their first 512
    columns: the GLM-5.2 contract (top-k at most 2048 tokens) the NeMo PR keeps,
    against the oracle's narrow-value attention. The tail is gathered and read
    through its own LDS tile, so every case checks that its columns count."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(13)
    H, DQ, N, W, Tq = 64, 576, 3000, 256, 9
    if case == "heads40":
        H = 40
    if case == "max_width":
        W, Tq = 2048, 3
    if case == "many_queries":
        Tq, W = 600, 192
    if case == "dense_2k_rows":      # the 2K workload's causal rows, sampled queries
        N, W = 2048, 2048
        rows = np.array([0, 1, 2, 3, 100, 511, 1024, 2047])
        Tq = len(rows)
    q = rng.standard_normal((Tq, H, DQ)).astype(np.float32)
    kv = rng.standard_normal((N, DQ)).astype(np.float32)
    if case == "rising":
        kv[N // 2:] *= 100.0
    q, kv = f32_to_bf16_bits(q), f32_to_bf16_bits(kv)
    idx = rng.integers(0, N, size=(Tq, W)).astype(np.int32)
    if case == "dense_2k_rows":
        idx = np.full((Tq, W), -1, np.int32)
        for i, t in enumerate(rows):
            idx[i, :t + 1] = np.arange(t + 1)
    if case == "scattered_mask":
        m = rng.random(idx.shape) < 0.4
        idx[m] = rng.choice([-1, -5, N, N + 7, 2 ** 31 - 1], size=m.sum())
    if case == "single":
        idx[:] = -1
        idx[np.arange(Tq), rng.integers(0, W, Tq)] = rng.integers(0, N, Tq)
    if case == "duplicates":
        idx[:, 100:] = idx[:, :W - 100]
    if case == "rising":
        idx[:, :64] = rng.integers(0, N // 2, size=(Tq, 64))
        idx[:, 64:] = rng.integers(N // 2, N, size=(Tq, W - 64))
    if case in ("max_width", "many_queries"):
        idx[1::2][rng.random((len(idx[1::2]), W)) < 0.3] = -1
        idx[0::7] = -1
    _log("mla rope tail", case, (Tq, H, DQ), W)
    scale = 1 / np.sqrt(DQ)
    g_out, g_lse = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv), dev(idx), scale)
    assert tuple(g_out.shape) == (Tq, H, 512)
    ref_out, ref_lse, ref_abs = oracle_mod.sparse_mla_dv(q, kv, idx, scale, 512, with_abs=True)
    scaled = case == "rising"
    info = check_out(host_bf16_f32(g_out), ref_out, case, ref_abs, scaled=scaled)
    info["lse"] = check_lse(host(g_lse), ref_lse, case, scaled=scaled)
    # the tail matters: dropping it (attention over the first 512 key columns) differs
    if case == "dense_2k_rows":
        no_tail, _ = oracle_mod.sparse_mla_dv(np.ascontiguousarray(q[:, :, :512]),
                                              np.ascontiguousarray(kv[:, :512]), idx, scale, 512)
        assert np.abs(no_tail - ref_out).max() > 10 * OUT_MAX
    _log("  ", info)
