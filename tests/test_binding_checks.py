"""The Python binding rejects mismatched tensor arguments before anything is
launched: every shape the C entry points derive sizes from is checked against
the others, so a wrong tensor cannot make a kernel read or write past a
buffer. Runs on the CPU: the tensors here are host tensors, and each call must
raise on its shape (or, with every shape right, on the device) first."""
import pytest
import torch

import sparse_attention_kpool_amd as K

bf, i32, f32, u8 = torch.bfloat16, torch.int32, torch.float32, torch.uint8


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


T, D_I, H_I, KP = 64, 32, 2, 4
P = T // KP


def build_args(**over):
    a = dict(cu_seqlens=z(2, i32), k_idx=z((T, D_I), bf), gate=z((T, D_I), bf), ape=z((KP, D_I), f32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(gate=z((T, 16), bf)), "gate"),
    (dict(gate=z((T + 4, D_I), bf)), "gate"),
    (dict(ape=z((3, D_I), f32)), "ape"),
    (dict(ape=z((KP, D_I), bf)), "ape"),
    (dict(cu_seqlens=z((2, 1), i32)), "cu_seqlens"),
])
def test_kpool_build_shapes(over, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        K.kpool_build(**build_args(**over), kpool=KP)


def test_kpool_build_host_tensors_rejected():
    with pytest.raises(ValueError, match="device tensor"):
        K.kpool_build(**build_args(), kpool=KP)


def _out(cap=P, d=D_I, B=1):
    return [z(B + 1, i32), z(cap, i32), z((cap, d), u8), z(cap, f32), None]


@pytest.mark.parametrize("k,bad,msg", [(0, z(3, i32), "cu_pools"), (1, z(P - 1, i32), "pool_start"),
                                       (2, z((P, 16), u8), "pooled_k_fp8"), (3, z(P + 1, f32), "pooled_k_scale"),
                                       (4, z((P, 8), f32), "pooled_k_f32")])
def test_kpool_build_from_out_shapes(k, bad, msg):
    out = _out()
    out[k] = bad
    with pytest.raises(ValueError, match=msg):
        K.kpool_build_from(**build_args(), token_lo=8, out=out, kpool=KP)


def score_args(**over):
    a = dict(cu_seqlens=z(2, i32), cu_pools=z(2, i32), pooled_k_fp8=z((P, D_I), u8), pooled_k_scale=z(P, f32),
             q_idx=z((T, H_I, D_I), bf), w_idx=z((T, H_I), f32), num_tokens=T, kpool=KP, topk_pools=4)
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(pooled_k_fp8=z((P, 64), u8)), "pooled_k_fp8"),        # width differs from the queries'
    (dict(pooled_k_fp8=z((P - 1, D_I), u8)), "pooled_k_fp8"),
    (dict(pooled_k_scale=z(P - 1, f32)), "pooled_k_scale"),
    (dict(w_idx=z((T, H_I + 1), f32)), "w_idx"),
    (dict(w_idx=z((T - 1, H_I), f32)), "w_idx"),
    (dict(cu_pools=z(3, i32)), "cu_pools"),
    (dict(q_idx=z((T - 1, H_I, D_I), bf), w_idx=z((T - 1, H_I), f32)), "q_pos"),
    (dict(q_pos=z(5, i32)), "q_pos"),
    (dict(workspace=z(16, f32)), "workspace"),
])
def test_indexer_score_topk_shapes(over, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        K.indexer_score_topk(**score_args(**over))


def test_indexer_score_topk_host_tensors_rejected():
    with pytest.raises(ValueError, match="device tensor"):
        K.indexer_score_topk(**score_args())


@pytest.mark.parametrize("over,msg", [(dict(scores=z((T, P + 1), f32)), "scores"),
                                      (dict(cu_pools=z(1, i32)), "cu_pools"),
                                      (dict(q_pos=z(3, i32)), "q_pos")])
def test_topk_from_scores_shapes(over, msg):
    a = dict(cu_seqlens=z(2, i32), cu_pools=z(2, i32), scores=z((T, P), f32), num_tokens=T, kpool=KP, topk_pools=4)
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        K.indexer_topk_from_scores(**a)


@pytest.mark.parametrize("over,msg", [(dict(kv=z((100, 32), bf)), "kv"),
                                      (dict(indices=z((3, 128), i32)), "indices"),
                                      (dict(out=z((4, 8, 32), bf)), "out"),    # fewer heads than q
                                      (dict(out=z((4, 16, 64), f32)), "out")])
def test_sparse_mla_shapes(over, msg):
    a = dict(q=z((4, 16, 64), bf), kv=z((100, 64), bf), indices=z((4, 128), i32), softmax_scale=0.125)
    a.update(over)
    with pytest.raises((ValueError, TypeError), match=msg):
        K.sparse_mla_fwd(**a)


def test_sparse_mla_host_tensors_rejected():
    with pytest.raises(ValueError, match="device tensor"):
        K.sparse_mla_fwd(z((4, 16, 64), bf), z((100, 64), bf), z((4, 128), i32), 0.125)
