"""The allocation-free indexer entry point (indexer_score_topk_noalloc, whose
workspace is the library's own device scratch) against indexer_score_topk with
a caller workspace, through the C ABI: index rows, slot counts and scores must
be bit-identical. Three calls in a row share the scratch, each smaller than the
one before: the 64 decode queries of a 1,048,576-token context (the largest
workspace that fits), the 4,096-token packed row, then the 64-token row. The
second and third calls run over what the first left in the scratch."""
import numpy as np
import pytest
import torch

from workloads import Workload, spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_kpool_amd as K
    K.lib()
    return K


def _inputs(name):
    s = spec(name)
    if name == "decode1m":   # drawn on the device (this test compares the GPU with itself)
        g = torch.Generator(device="cuda")
        g.manual_seed(77)
        r = lambda *sh: torch.randn(sh, generator=g, device="cuda")
        k_idx, gate = r(s.T, s.D_I).bfloat16(), r(s.T, s.D_I).bfloat16()
        ape = r(s.kpool, s.D_I)
        q_idx = r(s.Tq, s.H_I, s.D_I).bfloat16()
        w = r(s.Tq, s.H_I) / np.sqrt(s.H_I * s.D_I)
    else:
        wl = Workload(s)
        bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        k_idx, gate = bf(wl.full("k_idx")), bf(wl.full("gate"))
        ape = torch.from_numpy(wl.ape()).cuda()
        q_idx = bf(wl.full("q_idx"))
        w = torch.from_numpy(wl.full("w")).cuda()
    q_pos = None if s.q_pos is None else torch.from_numpy(s.q_pos).cuda()
    return s, torch.from_numpy(s.cu).cuda(), k_idx, gate, ape, q_idx, w, q_pos


def test_noalloc_matches_workspace_variant(K):
    for name in ["decode1m", "packed4k", "tiny"]:
        s, cu, k_idx, gate, ape, q_idx, w, q_pos = _inputs(name)
        print("no-alloc indexer", name, "T", s.T, "queries", s.Tq,
              "workspace bytes", K.kp_indexer_workspace_bytes(s.Tq, s.max_pools, s.H_I, s.D_I, s.topk), flush=True)
        cp, _, k8, ks, _ = K.kpool_build(cu, k_idx, gate, ape, s.kpool)
        for with_scores in (True, False):
            ref = K.indexer_score_topk(cu, cp, k8, ks, q_idx, w, s.T, s.kpool, s.topk, q_pos=q_pos,
                                       return_scores=with_scores)
            got = K.indexer_score_topk_noalloc(cu, cp, k8, ks, q_idx, w, s.T, s.kpool, s.topk, q_pos=q_pos,
                                               return_scores=with_scores)
            torch.cuda.synchronize()
            assert torch.equal(got[0], ref[0]), f"{name}: index rows differ"
            assert torch.equal(got[1], ref[1]), f"{name}: slot counts differ"
            if with_scores:
                assert torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32)), f"{name}: scores differ"
        # into caller tensors (what a captured graph would do): same rows again
        idx = torch.full_like(ref[0], 7)
        nv = torch.full_like(ref[1], 7)
        K.indexer_score_topk_noalloc(cu, cp, k8, ks, q_idx, w, s.T, s.kpool, s.topk, q_pos=q_pos, out=(idx, nv))
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(nv, ref[1]), f"{name}: caller-tensor outputs differ"


def test_noalloc_rejects_sizes_above_scratch(K):
    s, cu, k_idx, gate, ape, q_idx, w, q_pos = _inputs("packed4k")
    cp, _, k8, ks, _ = K.kpool_build(cu, k_idx, gate, ape, s.kpool)
    # 4,096 queries over a 16x longer context: 268 MB of scores, above the scratch
    T = 16 * s.T
    big_cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    big_cp = torch.tensor([0, T // 4], dtype=torch.int32, device="cuda")
    big_k8 = torch.zeros((T // 4, s.D_I), dtype=torch.uint8, device="cuda")
    big_ks = torch.ones(T // 4, dtype=torch.float32, device="cuda")
    qp = torch.arange(T - s.T, T, dtype=torch.int32, device="cuda")
    with pytest.raises(K.KpoolError, match="scratch") as e:
        K.indexer_score_topk_noalloc(big_cu, big_cp, big_k8, big_ks, q_idx, w, T, s.kpool, s.topk, q_pos=qp)
    assert e.value.status == 2
