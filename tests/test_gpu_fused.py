"""GPU parity of the fused scoring + top-k (no score tensor) and of the paged
pooled-key cache, through the C ABI.

The fused path must write the index rows the score-tensor path writes, bit for
bit (both rank the same fp32 keys), and agree with the oracle's selection on
the oracle's scores up to near-ties at the k-th score (tests/_util.py,
check_selection). Cases cover the decode rows of a 1M-token context, rows that
take every pool as a candidate, ties that the selection must break by pool
number, rows whose candidates fall outside [k, cap] (the exact rescoring path,
forced by key scales that mislead the sampled threshold), packed documents, and
the paged cache grown a few tokens at a time against the oracle's keys.
"""
import numpy as np
import pytest
import torch

from tests._util import check_key_codes, check_selection, dev, dev_bf16, host
from workloads import Workload, f32_to_bf16_bits, spec

pytestmark = pytest.mark.gpu

KPOOL = 4
PAGE_POOLS = 32
PAGE_TOK = PAGE_POOLS * KPOOL


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_kpool_amd as K
    K.lib()
    return K


def _log(*a):
    print(*a, flush=True)


def _width(topk):
    return -(-(KPOOL * topk + KPOOL - 1) // 128) * 128


# ---------------------------------------------------------------- inputs -----
def _rand_case(oracle_mod, seed, cu, q_pos, h=32, d=128):
    """Random FP8 pooled keys (oracle-quantised) for the layout of cu, and
    random indexer queries and weights for the given positions."""
    rng = np.random.default_rng(seed)
    T = int(cu[-1])
    cp, ps = oracle_mod.layout(cu, T, KPOOL)
    P = T // KPOOL
    k8 = np.zeros((P, d), np.uint8)
    sk = np.zeros(P, np.float32)
    c, s = oracle_mod.quant_rows(rng.standard_normal((len(ps), d)).astype(np.float32))
    k8[:len(ps)], sk[:len(ps)] = c, s
    q_idx = f32_to_bf16_bits(rng.standard_normal((len(q_pos), h, d)))
    w = rng.standard_normal((len(q_pos), h)).astype(np.float32)
    return cp, k8, sk, q_idx, w


def _pages(rng, cu, spare=3):
    """A page table scattering each document's pages over a shuffled pool of
    physical pages (unused entries -1)."""
    lens = np.diff(cu)
    npg = [-(-int(L) // PAGE_TOK) for L in lens]
    max_pages = max(npg + [1]) + 1
    total = sum(npg) + spare
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, np.int32)
    o = 0
    for dd, n in enumerate(npg):
        table[dd, :n] = perm[o:o + n]
        o += n
    return table, total


def _pool_rows(table, cu, cp):
    """Page row of every pool (packed numbering)."""
    rows = np.zeros(int(cp[-1]), np.int64)
    for dd in range(len(cu) - 1):
        j = np.arange(int(cp[dd + 1] - cp[dd]))
        rows[cp[dd] + j] = table[dd, j // PAGE_POOLS].astype(np.int64) * PAGE_POOLS + j % PAGE_POOLS
    return rows


def _token_slots(table, cu):
    """Page slot of every token (packed numbering)."""
    slots = np.zeros(int(cu[-1]), np.int64)
    for dd in range(len(cu) - 1):
        l = np.arange(int(cu[dd + 1] - cu[dd]))
        slots[cu[dd] + l] = table[dd, l // PAGE_TOK].astype(np.int64) * PAGE_TOK + l % PAGE_TOK
    return slots


def _to_pages(table, total, cu, cp, k8, sk):
    rows = _pool_rows(table, cu, cp)
    k8p = np.zeros((total * PAGE_POOLS, k8.shape[1]), np.uint8)
    skp = np.zeros(total * PAGE_POOLS, np.float32)
    k8p[rows] = k8[:len(rows)]
    skp[rows] = sk[:len(rows)]
    return k8p, skp


def _slots_to_tokens(idx, table, total, cu):
    """Map page-slot index rows back to packed token numbers (-1 stays -1)."""
    inv = np.full(total * PAGE_TOK, -1, np.int64)
    inv[_token_slots(table, cu)] = np.arange(int(cu[-1]))
    out = np.where(idx >= 0, inv[np.maximum(idx, 0)], -1)
    assert np.all((idx < 0) == (out < 0)), "a slot outside the documents' pages"
    return out.astype(np.int32)


# ------------------------------------------------------------ the runners ----
def _gpu_flat(K, cu, cp, k8, sk, q_idx, w, q_pos, topk, scores):
    T = int(cu[-1])
    idx, nv, sc = K.indexer_score_topk(dev(cu), dev(cp), dev(k8), dev(sk), dev_bf16(q_idx), dev(w), T, KPOOL, topk,
                                       row_width=_width(topk), q_pos=dev(q_pos), return_scores=scores)
    return host(idx), host(nv), (None if sc is None else host(sc))


def _gpu_paged(K, cu, table, total, k8p, skp, q_idx, w, q_pos, topk):
    idx, nv, path = K.indexer_score_topk_paged(dev(cu), dev(table), dev(k8p), dev(skp), dev_bf16(q_idx), dev(w),
                                               int(cu[-1]), KPOOL, topk, row_width=_width(topk),
                                               q_pos=dev(q_pos), return_row_path=True)
    return _slots_to_tokens(host(idx), table, total, cu), host(nv), host(path)


def _oracle_sel(oracle_mod, cu, cp, k8, sk, q_idx, w, q_pos, topk):
    qc, qs = oracle_mod.queries(q_idx)
    P = int(cp[-1])
    sc = oracle_mod.scores(cu, cp, KPOOL, q_pos, int(cu[-1]) // KPOOL, w, qc, qs, k8[:P], sk[:P])
    idx, nv = oracle_mod.topk(cu, cp, KPOOL, q_pos, sc, topk, _width(topk))
    return idx, nv, sc


def _run_all(K, oracle_mod, name, cu, cp, k8, sk, q_idx, w, q_pos, topk, seed=0, expect_path=None):
    """Fused flat, score-tensor flat, fused paged and the oracle on one case."""
    q_pos = np.asarray(q_pos, np.int32)
    f_idx, f_nv, _ = _gpu_flat(K, cu, cp, k8, sk, q_idx, w, q_pos, topk, False)
    m_idx, m_nv, _ = _gpu_flat(K, cu, cp, k8, sk, q_idx, w, q_pos, topk, True)
    table, total = _pages(np.random.default_rng(seed + 99), cu)
    k8p, skp = _to_pages(table, total, cu, cp, k8, sk)
    p_idx, p_nv, path = _gpu_paged(K, cu, table, total, k8p, skp, q_idx, w, q_pos, topk)
    assert np.array_equal(f_nv, m_nv) and np.array_equal(p_nv, m_nv), f"{name}: slot counts differ"
    bad_f = np.nonzero(np.any(f_idx != m_idx, axis=1))[0]
    bad_p = np.nonzero(np.any(p_idx != m_idx, axis=1))[0]
    assert bad_f.size == 0, f"{name}: fused rows {bad_f[:5]} differ from the score-tensor path"
    assert bad_p.size == 0, f"{name}: paged rows {bad_p[:5]} differ from the score-tensor path"
    if expect_path is not None:
        assert np.array_equal(path, expect_path), f"{name}: row paths {path.tolist()}"
    r_idx, r_nv, r_sc = _oracle_sel(oracle_mod, cu, cp, k8, sk, q_idx, w, q_pos, topk)
    info = check_selection(f_idx, f_nv, r_idx, r_nv, r_sc, cu, cp, KPOOL, q_pos, topk, name)
    info["rescored_rows"] = int(path.sum())
    _log("  ", name, info)
    return info


# --------------------------------------------------------------- cases -------
def test_fused_decode_rows(K, oracle_mod):
    """Decode rows of the 1M-token workload (262,144 pools per row), on the
    oracle's pooled keys: every row is selected among its candidates."""
    s = spec("decode1m")
    wl = Workload(s)
    cp, ps = oracle_mod.layout(s.cu, s.T, s.kpool)
    kc, kscale, _ = oracle_mod.keys(wl.full("k_idx"), wl.full("gate"), wl.ape(), ps, s.kpool)
    k8 = np.zeros((s.max_pools, s.D_I), np.uint8)
    sk = np.zeros(s.max_pools, np.float32)
    k8[:len(ps)], sk[:len(ps)] = kc, kscale
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(s.Tq, 6, replace=False), [0, s.Tq - 1]]))
    q_pos = s.query_positions()[rows]
    _log("fused decode rows", rows.tolist())
    _run_all(K, oracle_mod, "decode1m_rows", s.cu, cp, k8, sk, wl.full("q_idx")[rows], wl.full("w")[rows], q_pos,
             s.topk, expect_path=np.zeros(len(rows), np.int32))


def test_fused_packed_documents(K, oracle_mod):
    """Packed documents of mixed lengths: long rows (sampled threshold), rows of
    at most 16,384 pools (every pool a candidate), rows with fewer pools than
    k (all kept), an empty-pool query, first and last tokens of documents."""
    cu = np.array([0, 140_003, 140_008, 140_008, 240_000, 400_001], np.int32)
    q_pos = [0, 3, 4, 1000, 65_539, 70_000, 140_002, 140_003, 140_007, 140_008, 150_000, 239_999,
             240_000, 240_003, 260_000, 310_000, 400_000]
    cp, k8, sk, q_idx, w = _rand_case(oracle_mod, 11, cu, q_pos)
    _log("fused packed", len(q_pos), "queries")
    _run_all(K, oracle_mod, "packed", cu, cp, k8, sk, q_idx, w, q_pos, 512, seed=1)


def test_fused_ties(K, oracle_mod):
    """Most pools score exactly zero (zero key codes) and fewer than k score
    above it: the k-th score is a tie of thousands, broken by pool number both
    in the sampled threshold and in the final selection."""
    cu = np.array([0, 1 << 18], np.int32)
    q_pos = [100_000, 200_000, (1 << 18) - 5, (1 << 18) - 1]
    cp, k8, sk, q_idx, w = _rand_case(oracle_mod, 12, cu, q_pos)
    rng = np.random.default_rng(13)
    zero = rng.random(len(sk)) < 0.995
    k8[zero] = 0
    _log("fused ties")
    _run_all(K, oracle_mod, "ties", cu, cp, k8, sk, q_idx, w, q_pos, 512, seed=2,
             expect_path=np.zeros(len(q_pos), np.int32))


@pytest.mark.parametrize("mode", ["too_few", "too_many"])
def test_fused_rescoring_rows(K, oracle_mod, mode):
    """Key scales that make every 128th pool of a row (among them every pool
    the threshold samples: every 256th at this length) score far above
    (too_few: fewer than k pools clear the threshold) or far below (too_many:
    more than 16,384 clear it) the rest: those rows are selected by the exact
    rescoring path, with the same result as the score-tensor path."""
    cu = np.array([0, 1 << 17], np.int32)
    q_pos = np.array([(1 << 17) - 9, (1 << 17) - 2, 70_001, 40_000], np.int32)   # the last: 10,000 pools
    cp, k8, sk, q_idx, w = _rand_case(oracle_mod, 14, cu, q_pos)
    w = np.abs(w)                                      # scores >= 0: nearly every pool clears a tiny threshold
    sampled = (np.arange(len(sk)) % 128) == 0          # one document: its rows start at pool 0
    sk[sampled] *= 1000.0 if mode == "too_few" else 1e-3
    _log("fused rescoring", mode)
    _run_all(K, oracle_mod, mode, cu, cp, k8, sk, q_idx, w, q_pos, 512, seed=3,
             expect_path=np.array([1, 1, 1, 0], np.int32))


@pytest.mark.parametrize("topk", [0, 7, 2000])
def test_fused_topk_sizes(K, oracle_mod, topk):
    """No pool kept, a handful, and a top-k of 2000 pools."""
    cu = np.array([0, 150_000], np.int32)
    q_pos = [2, 30, 9000, 80_000, 149_999]
    cp, k8, sk, q_idx, w = _rand_case(oracle_mod, 15 + topk, cu, q_pos)
    _log("fused topk", topk)
    _run_all(K, oracle_mod, f"topk{topk}", cu, cp, k8, sk, q_idx, w, q_pos, topk, seed=4)


# ------------------------------------------------------------ paged cache ----
def test_paged_cache_grows(K, oracle_mod):
    """Three documents grow over eight steps of 1 to 300 tokens; after each step
    kpool_update_paged pools what the new tokens close. The pages must then
    hold, for every complete pool, the oracle's keys (up to one-step FP8 code
    flips on rounding boundaries, as for kpool_build) and exactly kpool_build's
    bytes for the same tokens."""
    rng = np.random.default_rng(21)
    d = 128
    final = np.array([1500, 7, 2333])
    start = np.array([900, 0, 2000])
    steps = [np.minimum(final, start + c) for c in (1, 2, 3, 67, 128, 131, 300, 10_000)]
    cu_final = np.concatenate([[0], np.cumsum(final)]).astype(np.int32)
    table, total = _pages(rng, cu_final)
    k_tok = f32_to_bf16_bits(rng.standard_normal((int(cu_final[-1]), d)))
    g_tok = f32_to_bf16_bits(rng.standard_normal((int(cu_final[-1]), d)))
    ape = (0.1 * rng.standard_normal((KPOOL, d))).astype(np.float32)
    slots = _token_slots(table, cu_final)
    kp_pages = np.zeros((total * PAGE_TOK, d), np.uint16)
    gp_pages = np.zeros((total * PAGE_TOK, d), np.uint16)
    k8p = torch.zeros((total * PAGE_POOLS, d), dtype=torch.uint8, device="cuda")
    skp = torch.zeros(total * PAGE_POOLS, dtype=torch.float32, device="cuda")
    tab_d = dev(table)
    ape_d = dev(ape)
    lens = start.copy()
    # the starting context: every pool (last_tokens covers each document)
    seq = [start] + steps
    for si, new in enumerate(seq):
        added = new - (lens if si > 0 else 0)
        cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        for dd in range(3):   # the caller writes the new tokens' rows into their slots
            lo, hi = int(new[dd] - added[dd]), int(new[dd])
            src = cu_final[dd] + np.arange(lo, hi)
            kp_pages[slots[src]] = k_tok[src]
            gp_pages[slots[src]] = g_tok[src]
        K.kpool_update_paged(dev(cu), tab_d, dev_bf16(kp_pages), dev_bf16(gp_pages), ape_d, k8p, skp,
                             int(added.max()), KPOOL)
        lens = new
    torch.cuda.synchronize()
    # compare every complete pool of the final context
    cu = cu_final
    cp, ps = oracle_mod.layout(cu, int(cu[-1]), KPOOL)
    rows = _pool_rows(table, cu, cp)
    got8, gots = host(k8p)[rows], host(skp)[rows]
    kc, ks, _ = oracle_mod.keys(k_tok, g_tok, ape, ps, KPOOL)
    frac = check_key_codes(got8, kc, "paged cache")
    assert np.allclose(gots, ks, rtol=1e-5), "paged scales differ from the oracle's"
    b_cp, b_ps, b_k8, b_sk, _ = K.kpool_build(dev(cu), dev_bf16(k_tok), dev_bf16(g_tok), ape_d, KPOOL)
    P = int(cp[-1])
    assert np.array_equal(host(b_k8)[:P], got8) and np.array_equal(host(b_sk)[:P], gots), \
        "paged keys differ from kpool_build's"
    _log("  paged cache: pools", P, "code flips vs oracle", frac)


def test_paged_decode_attention(K, oracle_mod):
    """A decode step on a paged latent: index rows in page slots feed
    sparse_mla_fwd over the latent's pages; the output equals the packed
    path's bit for bit (the same rows, gathered from other addresses)."""
    rng = np.random.default_rng(31)
    cu = np.array([0, 90_000, 90_001, 200_000], np.int32)
    q_pos = np.array([89_990, 89_999, 90_000, 199_998, 199_999], np.int32)
    cp, k8, sk, q_idx, w = _rand_case(oracle_mod, 32, cu, q_pos)
    T = int(cu[-1])
    H, D = 64, 512
    kv = f32_to_bf16_bits(rng.standard_normal((T, D)))
    q = f32_to_bf16_bits(rng.standard_normal((len(q_pos), H, D)))
    table, total = _pages(rng, cu)
    k8p, skp = _to_pages(table, total, cu, cp, k8, sk)
    slots = _token_slots(table, cu)
    kv_pages = np.zeros((total * PAGE_TOK, D), np.uint16)
    kv_pages[slots] = kv
    idx_p, nv_p, _ = K.indexer_score_topk_paged(dev(cu), dev(table), dev(k8p), dev(skp), dev_bf16(q_idx), dev(w), T,
                                                KPOOL, 512, q_pos=dev(q_pos))
    idx_f, nv_f, _ = K.indexer_score_topk(dev(cu), dev(cp), dev(k8), dev(sk), dev_bf16(q_idx), dev(w), T, KPOOL,
                                          512, q_pos=dev(q_pos))
    scale = 1 / np.sqrt(D)
    out_p, lse_p = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv_pages), idx_p, scale)
    out_f, lse_f = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv), idx_f, scale)
    assert torch.equal(nv_p, nv_f)
    assert torch.equal(out_p.view(torch.int16), out_f.view(torch.int16))
    assert torch.equal(lse_p, lse_f)
    _log("  paged decode attention: identical over", int(nv_p.sum().item()), "slots")
