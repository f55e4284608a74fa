"""Pins of the oracle's pool layout and index-row construction.

Pool rule (prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet):
groups of 4 per document starting at the document's first token; a query sees
the complete pools of its own document ending at or before it, keeps the top
512 and its own incomplete pool; rows padded to a multiple of 128. Slot count
2051 (NeMo AutoModel PR "add GLM-5.3-Flash training support", "cuDNN sparse MLA
parity and performance").
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _enumerate_layout(cu, kpool):
    """Token-by-token walk: assign each token its document and group number."""
    T = cu[-1]
    doc_of = np.empty(T, np.int64)
    for d in range(len(cu) - 1):
        doc_of[cu[d]:cu[d + 1]] = d
    starts = []
    counts = [0] * (len(cu) - 1)
    for t in range(T):
        d = doc_of[t]
        l = t - cu[d]
        # a token opens a pool when it begins a group of kpool and the whole group lies in its document
        if l % kpool == 0 and t + kpool - 1 < cu[d + 1]:
            starts.append(t)
            counts[d] += 1
    return np.cumsum([0] + counts).astype(np.int32), np.array(starts, np.int32)


def test_hand_worked_example(oracle_mod):
    g = json.load(open(os.path.join(GOLD, "layout_example.json")))
    cu_pools, ps = oracle_mod.layout(g["cu_seqlens"], g["num_tokens"], g["kpool"])
    assert cu_pools.tolist() == g["cu_pools"]
    assert ps.tolist() == g["pool_start"]
    for q in g["queries"]:
        d, lo, nv, ts = oracle_mod.query_info(g["cu_seqlens"], cu_pools, g["kpool"], q["t"])
        assert (d, lo, nv) == (q["doc"], q["pool_lo"], q["n_vis"]), q
        assert list(range(ts, q["t"] + 1)) == q["tail"], q


def test_hand_worked_index_rows(oracle_mod):
    g = json.load(open(os.path.join(GOLD, "layout_example.json")))
    cu = np.array(g["cu_seqlens"], np.int32)
    T, kp = g["num_tokens"], g["kpool"]
    cu_pools, _ = oracle_mod.layout(cu, T, kp)
    ex = g["index_rows_topk1"]
    for t_str, local in ex["scores"].items():
        t = int(t_str)
        _, lo, nv, _ = oracle_mod.query_info(cu, cu_pools, kp, t)
        sc = np.full((1, T // kp), -np.inf, np.float32)
        sc[0, lo:lo + nv] = local
        idx, n = oracle_mod.topk(cu, cu_pools, kp, np.array([t], np.int32), sc, 1, 128)
        want = ex["rows"][t_str]
        assert idx[0, :n[0]].tolist() == want
        assert np.all(idx[0, n[0]:] == -1)


@pytest.mark.parametrize("seed", range(12))
def test_layout_matches_token_walk(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 12))
    lens = rng.integers(0, 23, size=B)
    lens[rng.random(B) < 0.2] = 0                      # empty documents
    if lens.sum() == 0:
        lens[0] = 5
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    for kpool in (1, 2, 3, 4, 5):
        cu_pools, ps = oracle_mod.layout(cu, T, kpool)
        want_cp, want_ps = _enumerate_layout(cu, kpool)
        assert cu_pools.tolist() == want_cp.tolist()
        assert ps.tolist() == want_ps.tolist()
        # pools never cross a document; total bounded by T // kpool
        for d in range(B):
            for p in range(cu_pools[d], cu_pools[d + 1]):
                assert cu[d] <= ps[p] and ps[p] + kpool - 1 < cu[d + 1]
        assert cu_pools[-1] <= T // kpool


def test_layout_rejects_malformed(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.layout([0, 5, 3, 8], 8, 4)
    with pytest.raises(ValueError):
        oracle_mod.layout([0, 5, 9], 8, 4)
    with pytest.raises(ValueError):
        oracle_mod.layout([1, 8], 8, 4)


def test_query_info_invariants(oracle_mod):
    cu = np.array([0, 1, 2, 7, 7, 40, 41, 100], np.int32)
    T = 100
    cu_pools, ps = oracle_mod.layout(cu, T, 4)
    for t in range(T):
        d, lo, nv, ts = oracle_mod.query_info(cu, cu_pools, 4, t)
        assert cu[d] <= t < cu[d + 1]
        assert 0 <= t + 1 - ts <= 3                  # 1..3 tail tokens, or none when t closes a pool
        assert ts - cu[d] == 4 * nv
        for j in range(nv):                           # every visible pool ends at or before t
            assert ps[lo + j] + 3 <= t


def test_pages_slot_count(oracle_mod):
    """A query deep in a long document fills 4*512 pool slots plus 3 tail slots
    = 2051, padded to 2176; a 2063-slot row pads to the same width."""
    g = json.load(open(os.path.join(GOLD, "pages_constants.json")))
    kp = g["index_kpool"]["value"]
    topk = g["topk_pools"]["value"]
    assert kp * topk == g["index_topk_tokens"]["value"]
    mult = g["row_multiple"]["value"]
    raw = kp * topk + kp - 1
    assert raw == g["raw_slots"]["value"]
    W = -(-raw // mult) * mult
    assert W == -(-g["stress_raw_slots"]["value"] // mult) * mult == 2176
    T = 4 * 700 + 7
    cu = np.array([0, T], np.int32)
    cu_pools, _ = oracle_mod.layout(cu, T, kp)
    qpos = np.arange(T - 8, T, dtype=np.int32)
    rng = np.random.default_rng(0)
    sc = rng.standard_normal((8, T // kp)).astype(np.float32)
    idx, nv = oracle_mod.topk(cu, cu_pools, kp, qpos, sc, topk, W)
    assert nv.max() == g["raw_slots"]["value"]
    assert all(int(n) == kp * topk + ((t + 1) % kp) for n, t in zip(nv, qpos))
    tail_start = qpos + 1 - (qpos + 1) % kp
    pool_tokens = [int(np.sum(idx[i, :nv[i]] < tail_start[i])) for i in range(8)]
    assert set(pool_tokens) == {g["max_selected_tokens"]["value"]}


def test_num_valid_closed_form(oracle_mod):
    """n_valid(t) = 4*min(topk, n_vis) + tail, independent of the scores."""
    cu = np.array([0, 13, 13, 200, 301], np.int32)
    T = 301
    cu_pools, _ = oracle_mod.layout(cu, T, 4)
    rng = np.random.default_rng(3)
    sc = rng.standard_normal((T, T // 4)).astype(np.float32)
    for topk in (1, 4, 16, 64):
        W = -(-(4 * topk + 3) // 128) * 128
        idx, nv = oracle_mod.topk(cu, cu_pools, 4, None, sc, topk, W)
        for t in range(T):
            d = int(np.searchsorted(cu, t, side="right") - 1)
            l = t - cu[d]
            n_vis = (l + 1) // 4
            assert nv[t] == 4 * min(topk, n_vis) + (l + 1 - 4 * n_vis)
            row = idx[t, :nv[t]]
            assert np.all(np.diff(row) > 0)                     # ascending, no repeats
            assert np.all((row >= cu[d]) & (row <= t))          # own document, causal
            if (l + 1) % 4 != 0 or topk >= n_vis:
                assert row[-1] == t                             # the query sees itself
