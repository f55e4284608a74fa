"""GPU parity on packed rows at full size and on the decode context, through
the C ABI, against the CPU oracle:

* the 32K row of eight packed documents: layout bit-exact; pooled keys in full;
  scores fed the oracle's keys, top-k fed the oracle's scores and attention fed
  the oracle's index rows, on rows at and next to every document boundary
  (the first four tokens of each document, whose rows are tail-only or hold
  one pool, and each document's last token) plus random rows;
* the pooled keys of the 32K rows and of the 1,048,576-token decode context;
* kpool_build_from (the decode pooled-key cache) against the oracle's keys;
* kp_check_inputs on device data;
* determinism: two runs of each entry point give bit-identical results.

Bars as in test_gpu_parity.py: integer outputs bit-exact, FP8 key codes equal
up to rare one-step flips (fp32 vs fp64 pooling), scores and attention within
the tolerances of tests/_util.py.
"""
import numpy as np
import pytest
import torch

from tests._util import (check_key_codes, check_lse, check_out, check_scores, dev, dev_bf16, host,
                         host_bf16_f32)
from workloads import Workload, spec

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


_WL = {}


def _wl(name):
    """One Workload per name for the module (its generated tensors are cached)."""
    if name not in _WL:
        _WL[name] = Workload(spec(name))
    return _WL[name]


def boundary_rows(s, n_random=8, seed=0):
    """Query rows at and next to every document boundary, plus random ones."""
    rows = []
    for d in range(s.B):
        a, b = int(s.cu[d]), int(s.cu[d + 1])
        if a == b:
            continue
        rows += [t for t in range(a, min(a + 5, b))] + [b - 1, b - 2]
    rng = np.random.default_rng(seed)
    rows += rng.choice(s.Tq, n_random, replace=False).tolist()
    return np.unique(np.clip(np.array(rows), 0, s.Tq - 1))


def _compare_keys(name, g_codes, g_scales, g_f32, kc, kscale, pooled):
    """GPU pooled keys vs the oracle's (the rows given): fp32 means within
    fp32 rounding, scales within 1e-5, codes equal but for rare one-step flips."""
    if g_f32 is not None:
        assert np.all(np.abs(g_f32 - pooled) <= 1e-5 * np.abs(pooled) + 1e-6), f"{name}: pooled means"
    assert np.allclose(g_scales, kscale, rtol=1e-5, atol=0), f"{name}: key scales"
    frac = check_key_codes(g_codes, kc, name)
    return frac


# ----------------------------------------------------- layout and keys -------
@pytest.mark.parametrize("name", ["32k", "32k_multidoc", "decode1m"])
def test_layout_and_keys_full_size(K, oracle_mod, name):
    """Layout bit-exact and pooled keys against the oracle at full size: every
    pool of the 32K rows; for the 1M-token context, 16,384 sampled pools plus
    the first and last."""
    s = spec(name)
    wl = _wl(name)
    k_idx, gate, ape = wl.full("k_idx"), wl.full("gate"), wl.ape()
    _log("layout+keys", name, s.T)
    cp, ps, k8, ks, kf = K.kpool_build(dev(s.cu), dev_bf16(k_idx), dev_bf16(gate), dev(ape), s.kpool,
                                       with_f32=True)
    want_cp, want_ps = oracle_mod.layout(s.cu, s.T, s.kpool)
    assert host(cp).tolist() == want_cp.tolist()
    g_ps = host(ps)
    P = len(want_ps)
    assert np.array_equal(g_ps[:P], want_ps) and np.all(g_ps[P:] == -1)
    if P > 65536:
        rng = np.random.default_rng(11)
        rows = np.unique(np.concatenate([rng.choice(P, 16384, replace=False), [0, P - 1]]))
    else:
        rows = np.arange(P)
    kc, kscale, pooled = oracle_mod.keys(k_idx, gate, ape, want_ps[rows], s.kpool)
    frac = _compare_keys(name, host(k8)[rows], host(ks)[rows], host(kf)[rows], kc, kscale, pooled)
    _log("  pools compared", len(rows), "of", P, "code flips", frac)


@pytest.mark.parametrize("name,token_lo", [("32k_multidoc", "last64"), ("32k_multidoc", "in_last_doc"),
                                           ("32k_multidoc", "mid_doc"), ("packed4k", "last64"),
                                           ("decode1m", "last64")])
def test_kpool_build_from_vs_oracle(K, oracle_mod, name, token_lo):
    """The pooled-key cache: pools ending before token_lo keep the sentinels
    they were given; every other pool row equals the oracle's keys, and the
    rows past the last pool read -1 / 0 as kpool_build writes them."""
    s = spec(name)
    wl = _wl(name)
    if token_lo == "last64":
        lo = s.T - 64
    elif token_lo == "in_last_doc":
        lo = int(s.cu[-2]) + 5
    else:
        lo = (int(s.cu[3]) + int(s.cu[4])) // 2
    k_idx, gate, ape = wl.full("k_idx"), wl.full("gate"), wl.ape()
    args = (dev(s.cu), dev_bf16(k_idx), dev_bf16(gate), dev(ape))
    cap = s.max_pools
    out = [torch.full((s.B + 1,), -7, dtype=torch.int32, device="cuda"),
           torch.full((cap,), -9, dtype=torch.int32, device="cuda"),
           torch.full((cap, s.D_I), 0x5A, dtype=torch.uint8, device="cuda"),
           torch.full((cap,), 3.5, dtype=torch.float32, device="cuda"),
           torch.full((cap, s.D_I), -1.25, dtype=torch.float32, device="cuda")]
    _log("keys from (oracle)", name, "token_lo", lo)
    K.kpool_build_from(*args, lo, out, s.kpool)
    g = [host(t) for t in out]
    want_cp, want_ps = oracle_mod.layout(s.cu, s.T, s.kpool)
    P = len(want_ps)
    assert g[0].tolist() == want_cp.tolist()
    ends = want_ps.astype(np.int64) + s.kpool - 1
    rebuilt = np.nonzero(ends >= lo)[0]
    cached = np.nonzero(ends < lo)[0]
    assert np.all(g[1][cached] == -9) and np.all(g[2][cached] == 0x5A)
    assert np.all(g[3][cached] == 3.5) and np.all(g[4][cached] == -1.25)
    assert np.array_equal(g[1][rebuilt], want_ps[rebuilt])
    assert np.all(g[1][P:] == -1) and np.all(g[2][P:] == 0) and np.all(g[3][P:] == 0)
    kc, kscale, pooled = oracle_mod.keys(k_idx, gate, ape, want_ps[rebuilt], s.kpool)
    _compare_keys(f"{name}@{lo}", g[2][rebuilt], g[3][rebuilt], g[4][rebuilt], kc, kscale, pooled)
    _log("  rebuilt", len(rebuilt), "cached", len(cached))


# ------------------------------------------------- 32K, eight documents ------
def _oracle_keys(oracle_mod, s, wl):
    cp, ps = oracle_mod.layout(s.cu, s.T, s.kpool)
    kc, kscale, _ = oracle_mod.keys(wl.full("k_idx"), wl.full("gate"), wl.ape(), ps, s.kpool)
    k8 = np.zeros((s.max_pools, s.D_I), np.uint8)
    k8[:len(ps)] = kc
    sk = np.zeros(s.max_pools, np.float32)
    sk[:len(ps)] = kscale
    return cp, ps, k8, sk


@pytest.fixture(scope="module")
def multidoc(oracle_mod):
    """Oracle intermediates of the 32K eight-document row on its boundary rows."""
    s = spec("32k_multidoc")
    wl = _wl("32k_multidoc")
    rows = boundary_rows(s)
    cp, ps, k8, sk = _oracle_keys(oracle_mod, s, wl)
    qpos = s.query_positions()[rows]
    q_idx = wl.full("q_idx")[rows]
    w = wl.full("w")[rows]
    qc, qs = oracle_mod.queries(q_idx)
    sc = oracle_mod.scores(s.cu, cp, s.kpool, qpos, s.max_pools, w, qc, qs, k8[:len(ps)], sk[:len(ps)])
    idx, nv = oracle_mod.topk(s.cu, cp, s.kpool, qpos, sc, s.topk, s.row_width)
    return dict(s=s, wl=wl, rows=rows, cp=cp, k8=k8, sk=sk, qpos=qpos, q_idx=q_idx, w=w, scores=sc, idx=idx, nv=nv)


def test_multidoc_scores(K, multidoc):
    m = multidoc
    s = m["s"]
    _log("multidoc scores", len(m["rows"]), "rows")
    _, _, g_sc = K.indexer_score_topk(dev(s.cu), dev(m["cp"]), dev(m["k8"]), dev(m["sk"]), dev_bf16(m["q_idx"]),
                                      dev(m["w"]), s.T, s.kpool, s.topk, q_pos=dev(m["qpos"].astype(np.int32)),
                                      return_scores=True)
    _log("  ", check_scores(host(g_sc), m["scores"], "32k_multidoc"))


def test_multidoc_topk_bitexact(K, multidoc):
    m = multidoc
    s = m["s"]
    g_idx, g_nv = K.indexer_topk_from_scores(dev(s.cu), dev(m["cp"]), dev(m["scores"]), s.T, s.kpool, s.topk,
                                             q_pos=dev(m["qpos"].astype(np.int32)))
    g_idx, g_nv = host(g_idx), host(g_nv)
    assert np.array_equal(g_nv, m["nv"])
    bad = np.nonzero(np.any(g_idx != m["idx"], axis=1))[0]
    assert bad.size == 0, f"rows {m['rows'][bad[:5]]} differ"
    # document isolation: every entry of a row lies in the query's document, at or before it
    doc_of = np.searchsorted(s.cu, np.arange(s.T), side="right") - 1
    for i, t in enumerate(m["qpos"]):
        g = g_idx[i, :g_nv[i]]
        assert np.all(doc_of[g] == doc_of[t]) and np.all(g <= t), f"row {t} leaves its document"


def test_multidoc_mla(K, oracle_mod, multidoc):
    m = multidoc
    s = m["s"]
    wl = m["wl"]
    q = np.concatenate([wl.rows("q", int(r), int(r) + 1) for r in m["rows"]])
    kv = wl.full("kv")
    _log("multidoc mla", len(m["rows"]), "rows")
    g_out, g_lse = K.sparse_mla_fwd(dev_bf16(q), dev_bf16(kv), dev(m["idx"]), s.scale)
    ref_out, ref_lse = oracle_mod.sparse_mla(q, kv, m["idx"], s.scale)
    info = check_out(host_bf16_f32(g_out), ref_out, "32k_multidoc")
    info["lse"] = check_lse(host(g_lse), ref_lse, "32k_multidoc")
    _log("  ", info)


def test_multidoc_pipeline_selection(K, multidoc):
    """The GPU pipeline alone (its own keys and scores) on the boundary rows:
    rows stay in their document, slot counts equal the oracle's, and the
    selection agrees with the oracle's up to FP8 near-ties."""
    m = multidoc
    s = m["s"]
    wl = m["wl"]
    cu_d = dev(s.cu)
    cp, _, k8, ks, _ = K.kpool_build(cu_d, dev_bf16(wl.full("k_idx")), dev_bf16(wl.full("gate")), dev(wl.ape()),
                                     s.kpool)
    idx, nv, _ = K.indexer_score_topk(cu_d, cp, k8, ks, dev_bf16(m["q_idx"]), dev(m["w"]), s.T, s.kpool, s.topk,
                                      q_pos=dev(m["qpos"].astype(np.int32)))
    idx, nv = host(idx), host(nv)
    assert np.array_equal(nv, m["nv"])
    jac = []
    for i in range(len(m["rows"])):
        a, b = set(idx[i, :nv[i]].tolist()), set(m["idx"][i, :nv[i]].tolist())
        jac.append(len(a & b) / len(a | b))
    _log("  jaccard mean", np.mean(jac), "min", np.min(jac))
    assert np.mean(jac) >= 0.97


# ---------------------------------------------------------- kp_check_inputs --
def test_check_inputs_on_device(K):
    ok = dev(np.array([0, 5, 5, 64], np.int32))
    K.kp_check_inputs(ok, 64)
    K.kp_check_inputs(ok, 64, dev(np.array([0, 17, 63], np.int32)))
    cases = [(np.array([1, 5, 64], np.int32), None, "cu_seqlens\\[0\\]"),
             (np.array([0, 9, 5, 64], np.int32), None, "decreases"),
             (np.array([0, 5, 60], np.int32), None, "expected 64"),
             (np.array([0, 64], np.int32), np.array([0, 64], np.int32), "q_pos\\[1\\]"),
             (np.array([0, 64], np.int32), np.array([-1], np.int32), "q_pos\\[0\\]")]
    for cu, qp, msg in cases:
        with pytest.raises(K.KpoolError, match=msg) as e:
            K.kp_check_inputs(dev(cu), 64, None if qp is None else dev(qp))
        assert e.value.status == 1


# ------------------------------------------------------------ determinism -----
def _rand_bf16(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("name", ["2k", "32k", "decode1m"])
def test_determinism(K, name):
    """Two runs of the whole forward on the same inputs give bit-identical
    keys, index rows, slot counts, outputs and lse (the inputs are drawn on the
    device: this test compares the GPU with itself, no oracle involved). The
    decode case runs the many-workgroup top-k, whose histograms use atomics."""
    s = spec(name)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    cu = dev(s.cu)
    k_idx = _rand_bf16((s.T, s.D_I), gen)
    gate = _rand_bf16((s.T, s.D_I), gen)
    ape = torch.randn((s.kpool, s.D_I), generator=gen, device="cuda")
    q_idx = _rand_bf16((s.Tq, s.H_I, s.D_I), gen)
    w = torch.randn((s.Tq, s.H_I), generator=gen, device="cuda") / np.sqrt(s.H_I * s.D_I)
    q = _rand_bf16((s.Tq, s.H, s.D), gen)
    kv = _rand_bf16((s.T, s.D), gen)
    q_pos = None if s.q_pos is None else dev(s.q_pos)
    _log("determinism", name)
    runs = []
    for _ in range(2):
        cp, ps, k8, ks, _ = K.kpool_build(cu, k_idx, gate, ape, s.kpool)
        idx, nv, _ = K.indexer_score_topk(cu, cp, k8, ks, q_idx, w, s.T, s.kpool, s.topk, q_pos=q_pos)
        out, lse = K.sparse_mla_fwd(q, kv, idx, s.scale)
        runs.append((cp, ps, k8, ks, idx, nv, out, lse))
    torch.cuda.synchronize()
    names = ["cu_pools", "pool_start", "pooled_k_fp8", "pooled_k_scale", "indices", "num_valid", "out", "lse"]
    for nm, a, b in zip(names, *runs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"{name}: {nm} differs"
