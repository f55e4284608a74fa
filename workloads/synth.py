"""Seeded synthetic inputs for the KPool-indexed DSA forward.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the CPU oracle (through the tests) and the HIP path
(through the tests and the benchmark) take their inputs from here, so the two
sides see bit-identical data.

Shapes follow the GLM-5.3-Flash KPool-DSA layer as the pages describe it
(NeMo AutoModel PR "add GLM-5.3-Flash training support", section "cuDNN sparse
MLA parity and performance": 64 query heads, a 512-wide latent, index_topk 2048
tokens = 512 pools of index_kpool 4; prime-rl PR "GLM-5.3-Flash text model",
Summary, third bullet: per-document pools of 4, Hadamard-rotated FP8 indexer).
The pages train on packed THD rows of 2,048 and 4,096 tokens and quote a
1,048,576-token context; the rows below stand in for those workloads with
N(0,1) data (no dataset content is used).

Every tensor is generated in row chunks, each chunk from its own
``numpy.random.default_rng([seed, tag, chunk])`` stream, so any row range can
be regenerated on its own (the oracle checks sampled rows of large workloads
without materialising the rest). bf16 tensors are returned as uint16 bit
patterns, rounded from float32 to nearest-even.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np

# Tensor tags: one independent random stream per tensor.
TAG_K_IDX, TAG_GATE, TAG_APE, TAG_Q_IDX, TAG_W, TAG_Q, TAG_KV, TAG_BOOST, TAG_CUTS = range(9)

_CHUNK_ELEMS = 1 << 22


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Spec:
    """One workload: a packed row of ``T`` tokens split into documents by ``cu``."""

    name: str
    T: int
    cu: np.ndarray                      # int32 [B+1]
    kpool: int = 4
    topk: int = 512                     # pools
    H: int = 64                         # attention heads
    D: int = 512                        # latent width (K = V)
    H_I: int = 32                       # indexer heads
    D_I: int = 128                      # indexer head dim (= Hadamard size)
    scale: float = 1.0 / math.sqrt(512.0)
    seed: int = 0
    q_pos: Optional[np.ndarray] = None  # int32 [Tq] or None (= every token)
    boost_frac: float = 0.0             # fraction of latent/k_idx rows scaled by 8
    note: str = ""

    @property
    def B(self) -> int:
        return int(self.cu.shape[0] - 1)

    @property
    def Tq(self) -> int:
        return self.T if self.q_pos is None else int(self.q_pos.shape[0])

    @property
    def row_width(self) -> int:
        raw = self.kpool * self.topk + self.kpool - 1
        return (raw + 127) // 128 * 128

    @property
    def max_pools(self) -> int:
        return self.T // self.kpool

    def query_positions(self) -> np.ndarray:
        if self.q_pos is None:
            return np.arange(self.T, dtype=np.int32)
        return self.q_pos


def _cu_from_cuts(T: int, cuts: Sequence[int]) -> np.ndarray:
    return np.array([0, *sorted(int(c) for c in cuts), T], dtype=np.int32)


def random_cu(T: int, num_docs: int, seed: int) -> np.ndarray:
    """``num_docs`` documents with uniform-random lengths summing to ``T``:
    ``num_docs - 1`` distinct cut points drawn uniformly from 1..T-1, sorted."""
    rng = np.random.default_rng([seed, TAG_CUTS])
    cuts = rng.choice(np.arange(1, T, dtype=np.int64), size=num_docs - 1, replace=False)
    return _cu_from_cuts(T, cuts)


def spec(name: str) -> Spec:
    """The named workloads (sizes as in the configuration list of the build)."""
    s512 = 1.0 / math.sqrt(512.0)
    if name == "tiny":
        return Spec(name, T=64, cu=_cu_from_cuts(64, []), topk=4, H=4, D=64, H_I=2, D_I=32,
                    scale=1.0 / 8.0, seed=0, note="one 64-token document")
    if name == "tiny_dense":
        return Spec(name, T=64, cu=_cu_from_cuts(64, []), topk=16, H=4, D=64, H_I=2, D_I=32,
                    scale=1.0 / 8.0, seed=0, note="top-k covers every pool")
    if name == "2k":
        return Spec(name, T=2048, cu=_cu_from_cuts(2048, []), scale=s512, seed=1,
                    note="one 2,048-token document; top-k 512 covers every pool")
    if name == "packed4k":
        return Spec(name, T=4096, cu=random_cu(4096, 5, seed=2), scale=s512, seed=2,
                    note="5 packed documents")
    if name == "32k":
        return Spec(name, T=32768, cu=_cu_from_cuts(32768, []), scale=s512, seed=3, boost_frac=0.01,
                    note="one 32,768-token document; 1% of rows scaled by 8")
    if name == "32k_multidoc":
        return Spec(name, T=32768, cu=random_cu(32768, 8, seed=4), scale=s512, seed=4,
                    note="8 packed documents in 32,768 tokens")
    if name == "decode1m":
        T = 1 << 20
        return Spec(name, T=T, cu=_cu_from_cuts(T, []), scale=s512, seed=5,
                    q_pos=np.arange(T - 64, T, dtype=np.int32),
                    note="64 queries at the end of a 1,048,576-token document")
    raise KeyError(name)


NAMED = ["tiny", "tiny_dense", "2k", "packed4k", "32k", "32k_multidoc", "decode1m"]


class Workload:
    """Lazily generated, row-addressable inputs of one :class:`Spec`."""

    def __init__(self, s: Spec, threads: int = 8):
        self.s = s
        self.threads = threads
        self._cache: Dict[str, np.ndarray] = {}
        self._boost: Optional[np.ndarray] = None

    # -- shapes ---------------------------------------------------------------
    def _row_shape(self, name: str):
        s = self.s
        return {
            "k_idx": (s.D_I,), "gate": (s.D_I,), "kv": (s.D,),
            "q_idx": (s.H_I, s.D_I), "w": (s.H_I,), "q": (s.H, s.D),
        }[name]

    def _rows(self, name: str) -> int:
        return self.s.T if name in ("k_idx", "gate", "kv") else self.s.Tq

    def _tag(self, name: str) -> int:
        return {"k_idx": TAG_K_IDX, "gate": TAG_GATE, "q_idx": TAG_Q_IDX, "w": TAG_W,
                "q": TAG_Q, "kv": TAG_KV}[name]

    def _chunk_rows(self, name: str) -> int:
        return max(1, _CHUNK_ELEMS // int(np.prod(self._row_shape(name))))

    # -- generation -----------------------------------------------------------
    def boost_rows(self) -> np.ndarray:
        """Sorted token positions whose latent and indexer-key rows are scaled by 8."""
        if self._boost is None:
            n = int(round(self.s.boost_frac * self.s.T))
            if n == 0:
                self._boost = np.zeros(0, dtype=np.int64)
            else:
                rng = np.random.default_rng([self.s.seed, TAG_BOOST])
                self._boost = np.sort(rng.choice(self.s.T, size=n, replace=False)).astype(np.int64)
        return self._boost

    def _gen_chunk(self, name: str, c: int) -> np.ndarray:
        cr = self._chunk_rows(name)
        r0 = c * cr
        r1 = min(self._rows(name), r0 + cr)
        shape = (r1 - r0, *self._row_shape(name))
        rng = np.random.default_rng([self.s.seed, self._tag(name), c])
        x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
        if name == "w":
            return (x * np.float32(1.0 / math.sqrt(self.s.H_I * self.s.D_I))).astype(np.float32)
        if name in ("kv", "k_idx") and self.s.boost_frac > 0:
            b = self.boost_rows()
            sel = b[(b >= r0) & (b < r1)] - r0
            x[sel] *= np.float32(8.0)          # exact: a power of two
        return f32_to_bf16_bits(x)

    def rows(self, name: str, r0: int, r1: int) -> np.ndarray:
        """Rows ``[r0, r1)`` of tensor ``name`` (bf16 bits, or float32 for ``w``)."""
        if name in self._cache:
            return self._cache[name][r0:r1]
        cr = self._chunk_rows(name)
        parts = [self._gen_chunk(name, c) for c in range(r0 // cr, (max(r1, r0 + 1) - 1) // cr + 1)]
        full = np.concatenate(parts, axis=0)
        off = (r0 // cr) * cr
        return full[r0 - off:r1 - off]

    def full(self, name: str) -> np.ndarray:
        """The whole tensor, generated in parallel chunks and cached."""
        if name in self._cache:
            return self._cache[name]
        R = self._rows(name)
        cr = self._chunk_rows(name)
        nch = (R + cr - 1) // cr
        dtype = np.float32 if name == "w" else np.uint16
        out = np.empty((R, *self._row_shape(name)), dtype=dtype)

        def work(c):
            out[c * cr:min(R, (c + 1) * cr)] = self._gen_chunk(name, c)

        if nch == 1:
            work(0)
        else:
            with ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(work, range(nch)))
        self._cache[name] = out
        return out

    def ape(self) -> np.ndarray:
        """Per-position pool bias ``[kpool, D_I]`` float32, N(0,1)."""
        rng = np.random.default_rng([self.s.seed, TAG_APE])
        return rng.standard_normal((self.s.kpool, self.s.D_I), dtype=np.float32)

    def drop(self, name: str) -> None:
        self._cache.pop(name, None)


def custom(name: str, T: int, cu: Sequence[int], *, kpool=4, topk=4, H=4, D=64, H_I=2, D_I=32,
           scale=None, seed=0, q_pos=None, boost_frac=0.0) -> Spec:
    """A small ad-hoc workload for edge-case tests."""
    cu_arr = np.asarray(cu, dtype=np.int32)
    assert cu_arr[0] == 0 and cu_arr[-1] == T and np.all(np.diff(cu_arr) >= 0)
    return Spec(name, T=T, cu=cu_arr, kpool=kpool, topk=topk, H=H, D=D, H_I=H_I, D_I=D_I,
                scale=(1.0 / math.sqrt(D)) if scale is None else scale, seed=seed,
                q_pos=None if q_pos is None else np.asarray(q_pos, dtype=np.int32),
                boost_frac=boost_frac)
