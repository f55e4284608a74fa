"""Benchmark of the KPool-DSA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 32k] [--no-cpu-baseline] [--backward]

One step = one whole forward of the hot path over one batch of synthetic input
resident in HBM: kpool_build (pool layout, pooled FP8 keys) + indexer_score_topk
(query rotation, FP8 scoring, top-k index rows) + sparse_mla_fwd (absorbed
sparse latent attention). Prints one JSON line on stdout; a per-stage
breakdown goes to stderr. Besides the step, the line reports the key pooling
with cold caches and, with --backward, the sparse-MLA backward on the same
index rows (its own stage, not part of the step).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA fwd query-tokens/sec at 32K packed; sparse-MLA TFLOP/s & % bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
# the highest bf16 MFMA rate the issue-rate microbenchmark reaches on one MI355X (two
# waves per SIMD, MFMA only; sparse_attention_kpool_amd/microbench, summary in profiles/)
MFMA_MEASURED_TFLOPS = 2293.0

# HBM bytes per sparse_mla_fwd launch, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# passes scaled by the same counters' reading of a plain 1 GiB device copy (the
# commands and raw counts are in profiles/dsa_forward_32k_hbm_traffic.md). Keyed
# by the attention kernel's source hash: a changed kernel reports null until its
# counters are taken again.
MEASURED_TRAFFIC = {
    "ec2a9b167a007020": {"workload": "32k", "read": 21383370265, "write": 2155919274},
}
MLA_SOURCE = os.path.join(ROOT, "sparse_attention_kpool_amd", "csrc", "sparse_mla.hip")


def measured_traffic(workload: str):
    import hashlib
    with open(MLA_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    m = MEASURED_TRAFFIC.get(sha)
    if m is None or m["workload"] != workload:
        return None, sha
    return m["read"] + m["write"], sha


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_counts(s):
    """Closed-form algorithmic work of one forward (per-query n_vis, n_valid)."""
    qpos = s.query_positions().astype(np.int64)
    doc = np.searchsorted(s.cu, qpos, side="right") - 1
    l = qpos - s.cu[doc]
    n_vis = (l + 1) // s.kpool
    tail = (l + 1) - s.kpool * n_vis
    n_valid = s.kpool * np.minimum(s.topk, n_vis) + tail
    P = int(sum((s.cu[d + 1] - s.cu[d]) // s.kpool for d in range(s.B)))
    return {
        "visible_pairs": int(n_vis.sum()),
        "sum_n_valid": int(n_valid.sum()),
        "pools": P,
        # flop: scoring 2*H_I*D_I per visible pair; attention 4*H*D per valid slot (QK and PV)
        "score_flop": float(2 * s.H_I * s.D_I) * float(n_vis.sum()),
        "mla_flop": float(4 * s.H * s.D) * float(n_valid.sum()),
        # bytes: pooling reads k_idx + gate rows of every token, writes codes + scale per pool
        "pool_bytes": float(s.T * s.D_I * 2 * 2 + P * (s.D_I + 4)),
        "gather_bytes": float(n_valid.sum()) * s.D * 2,
    }


def cpu_baseline(s, wl, budget_s: float = 12.0):
    """The oracle as it stands, on a bounded sample of the same workload: the
    per-forward key pass over the whole row, then blocks of 32 consecutive
    query rows at random positions (each block's inputs generated once) until
    the time budget is spent. Scaled to query-tokens/s of a whole forward."""
    from oracle import oracle as O
    O.lib()
    t0 = time.perf_counter()
    cu_pools, ps = O.layout(s.cu, s.T, s.kpool)
    kc, ks, _ = O.keys(wl.full("k_idx"), wl.full("gate"), wl.ape(), ps, s.kpool)
    t_keys = time.perf_counter() - t0
    rng = np.random.default_rng(123)
    b = min(32, s.Tq)
    starts = rng.permutation(np.arange(0, s.Tq - b + 1, b))
    done, t_q = 0, 0.0
    kv = wl.full("kv")
    for r0 in starts:
        if t_q >= budget_s:
            break
        rows = np.arange(r0, r0 + b)
        qpos = s.query_positions()[rows]
        q_idx, w, q = wl.rows("q_idx", r0, r0 + b), wl.rows("w", r0, r0 + b), wl.rows("q", r0, r0 + b)
        t1 = time.perf_counter()
        qc, qs = O.queries(q_idx)
        sc = O.scores(s.cu, cu_pools, s.kpool, qpos, s.max_pools, w, qc, qs, kc, ks)
        idx, _ = O.topk(s.cu, cu_pools, s.kpool, qpos, sc, s.topk, s.row_width)
        O.sparse_mla(q, kv, idx, s.scale)
        t_q += time.perf_counter() - t1
        done += b
    per_q = t_q / done
    fwd = t_keys + per_q * s.Tq
    return {"value": s.Tq / fwd, "unit": "query-tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"key pass over all {s.T} tokens ({t_keys:.2f} s) + {done} query rows of {s.Tq} "
                      f"(blocks of {b} consecutive rows at random positions) through scoring, top-k and "
                      f"attention ({t_q:.1f} s); whole-forward time extrapolated as keys + per-query time x {s.Tq}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--full-pool", action="store_true",
                    help="decode: pool the whole context every step instead of the pools of the new tokens")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--backward", action="store_true",
                    help="also time sparse_mla_bwd (dQ, dKV for a random output gradient) on the same rows")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="kpool_build launches timed after a 512 MB write each (cold L2 and Infinity Cache)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference "
                         "reading for rocprofv3's FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards by query; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return
    import sparse_attention_kpool_amd as K
    from workloads import Workload, spec

    s = spec(args.workload)
    wl = Workload(s, threads=min(16, os.cpu_count() or 8))
    t0 = time.perf_counter()

    def bf(name):
        a = wl.full(name)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        wl.drop(name)
        return t

    dev = torch.device("cuda", 0)
    cu = torch.from_numpy(s.cu).cuda()
    k_idx, gate = bf("k_idx"), bf("gate")
    ape = torch.from_numpy(wl.ape()).cuda()
    q_idx = bf("q_idx")
    w = torch.from_numpy(wl.full("w")).cuda()
    q = bf("q")
    kv = bf("kv")
    q_pos = None if s.q_pos is None else torch.from_numpy(s.q_pos).cuda()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s: T={s.T} Tq={s.Tq}")

    # outputs and workspace allocated once; a step launches the three entry points
    L = K.lib()
    import ctypes as C
    P = C.c_void_p
    cap = s.T // s.kpool
    W = s.row_width
    cu_pools = torch.empty(s.B + 1, dtype=torch.int32, device=dev)
    pool_start = torch.empty(cap, dtype=torch.int32, device=dev)
    k8 = torch.empty((cap, s.D_I), dtype=torch.uint8, device=dev)
    ks = torch.empty(cap, dtype=torch.float32, device=dev)
    idx = torch.empty((s.Tq, W), dtype=torch.int32, device=dev)
    nv = torch.empty(s.Tq, dtype=torch.int32, device=dev)
    out = torch.empty((s.Tq, s.H, s.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((s.Tq, s.H), dtype=torch.float32, device=dev)
    ws_bytes = K.kp_indexer_workspace_bytes(s.Tq, cap, s.H_I, s.D_I, s.topk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    mla_ws_bytes = K.kp_mla_fwd_workspace_bytes(s.Tq, s.H, s.D, W)     # (0 unless the rows are split)
    mla_ws = torch.empty(max(mla_ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = P(stream.cuda_stream)
    ptr = lambda t: None if t is None else P(t.data_ptr())

    def call(status):
        if status != 0:
            raise RuntimeError(L.kp_last_error().decode())

    # Decode (queries at the end of the context): the pooled keys of the pools that
    # end before the first query are a cache, built once before timing; a step
    # pools only the rest (kpool_build_from). Other workloads pool everything.
    token_lo = int(s.q_pos.min()) if (s.q_pos is not None and not args.full_pool) else 0
    if token_lo > 0:
        call(L.kpool_build(ptr(cu), s.B, s.T, ptr(k_idx), ptr(gate), ptr(ape), s.D_I, s.kpool, ptr(cu_pools),
                           ptr(pool_start), ptr(k8), ptr(ks), None, sp))

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        call(L.kpool_build_from(ptr(cu), s.B, s.T, ptr(k_idx), ptr(gate), ptr(ape), s.D_I, s.kpool, token_lo,
                                ptr(cu_pools), ptr(pool_start), ptr(k8), ptr(ks), None, sp))
        if ev:
            ev[1].record(stream)
        call(L.indexer_score_topk(ptr(cu), s.B, s.T, ptr(cu_pools), cap, ptr(k8), ptr(ks), ptr(q_pos), s.Tq,
                                  ptr(q_idx), ptr(w), s.H_I, s.D_I, s.kpool, s.topk, W, ptr(idx), ptr(nv), None,
                                  ptr(ws), ws_bytes, sp))
        if ev:
            ev[2].record(stream)
        call(L.sparse_mla_fwd(ptr(q), ptr(kv), ptr(idx), s.Tq, s.T, s.H, s.D, W, C.c_float(s.scale), ptr(out),
                              ptr(lse), ptr(mla_ws) if mla_ws_bytes else None, mla_ws_bytes, sp))
        if ev:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    st = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    ms_stage = st.mean(axis=0)
    ms_med, ms_min = np.median(st, axis=0), st.min(axis=0)
    ms_step = wall * 1e3 / args.steps

    # kpool_build cold: a 512 MB write before each launch evicts the L2s and the
    # Infinity Cache, so the launch reads its k_idx and gate rows from HBM
    cold = []
    if args.cold_reps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for _ in range(args.cold_reps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(L.kpool_build_from(ptr(cu), s.B, s.T, ptr(k_idx), ptr(gate), ptr(ape), s.D_I, s.kpool, 0,
                                    ptr(cu_pools), ptr(pool_start), ptr(k8), ptr(ks), None, sp))
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush

    wc = work_counts(s)
    assert int(nv.sum().item()) == wc["sum_n_valid"], "index rows disagree with the closed-form slot count"
    mla_s = ms_stage[2] / 1e3
    traffic, mla_sha = measured_traffic(s.name)
    mla_tflops = wc["mla_flop"] / mla_s / 1e12
    log(f"stages (ms, mean of {args.steps}): kpool_build {ms_stage[0]:.3f}  indexer_score_topk {ms_stage[1]:.3f}"
        f"  sparse_mla_fwd {ms_stage[2]:.3f}  | step wall {ms_step:.3f}")
    log(f"sparse MLA {mla_tflops:.1f} TFLOP/s ({100 * mla_tflops / BF16_PEAK_TFLOPS:.1f}% bf16 peak); gathered "
        f"{wc['gather_bytes'] / mla_s / 1e9:.0f} GB/s effective; pooling {wc['pool_bytes'] / (ms_stage[0] / 1e3) / 1e9:.0f} GB/s;"
        f" scoring+top-k {wc['score_flop'] / (ms_stage[1] / 1e3) / 1e12:.1f} TFLOP/s (FP8)")

    bwd = None
    if args.backward:
        g = torch.Generator(device=dev)
        g.manual_seed(17)
        d_out = torch.randn((s.Tq, s.H, s.D), generator=g, device=dev).to(torch.bfloat16)
        d_q = torch.empty_like(d_out)
        d_kv = torch.empty((s.T, s.D), dtype=torch.float32, device=dev)
        bws = K.kp_mla_bwd_workspace_bytes(s.Tq, s.D, W)
        bw_ws = torch.empty(bws, dtype=torch.uint8, device=dev)

        def bstep():
            call(L.sparse_mla_bwd(ptr(q), ptr(kv), ptr(idx), ptr(out), ptr(lse), ptr(d_out), s.Tq, s.T, s.H, s.D,
                                  W, C.c_float(s.scale), ptr(d_q), ptr(d_kv), ptr(bw_ws), bws, sp))

        for _ in range(args.warmup):
            bstep()
        torch.cuda.synchronize()
        bt = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            bstep()
            e1.record(stream)
            torch.cuda.synchronize()
            bt.append(e0.elapsed_time(e1))
        # flop: S, dP and dQ products (6*H*D per valid slot) + the dKV product (4*H*D)
        bflop = float(10 * s.H * s.D) * wc["sum_n_valid"]
        bmed = float(np.median(bt))
        btf = bflop / (bmed / 1e3) / 1e12
        bwd = {"ms_median": bmed, "ms_min": float(min(bt)), "tflops": btf, "frac_bf16_peak": btf / BF16_PEAK_TFLOPS,
               "algorithmic": f"10*H*D = {10 * s.H * s.D} flop per valid slot x {wc['sum_n_valid']} slots",
               "workspace_bytes": bws,
               "kernels": "per chunk of 8192 queries: mla_bwd_dq_kernel, mla_bwd_dkv_part_kernel, a radix sort of "
                          "the slots by row, the ordered dKV reduction (+ dKV zero fill)"}
        log(f"sparse MLA backward: {bmed:.3f} ms median, {btf:.1f} TFLOP/s ({100 * btf / BF16_PEAK_TFLOPS:.1f}% "
            f"bf16 peak)")

    res = {
        "metric": METRIC,
        "value": s.Tq / (ms_step / 1e3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{s.name}: {s.note}; top-k {s.topk} pools of {s.kpool}, 64 heads x 512 bf16 "
                               f"latent, indexer {s.H_I}x{s.D_I} FP8", "T": s.T, "num_q": s.Tq,
                   "topk_pools": s.topk, "row_width": W, "heads": s.H, "d_latent": s.D, "h_idx": s.H_I,
                   "d_idx": s.D_I, "pools_rebuilt_from_token": token_lo},
        "stages_ms": {"kpool_build": ms_stage[0], "indexer_score_topk": ms_stage[1], "sparse_mla_fwd": ms_stage[2]},
        "stages_ms_median": {"kpool_build": float(ms_med[0]), "indexer_score_topk": float(ms_med[1]),
                             "sparse_mla_fwd": float(ms_med[2])},
        "stages_ms_min": {"kpool_build": float(ms_min[0]), "indexer_score_topk": float(ms_min[1]),
                          "sparse_mla_fwd": float(ms_min[2])},
        "sparse_mla_tflops": mla_tflops,
        "sparse_mla_pct_bf16_peak": 100 * mla_tflops / BF16_PEAK_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": mla_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": mla_tflops / BF16_PEAK_TFLOPS, "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM read + write)",
                     "kernel": "sparse_mla_kernel<512>", "kernel_source_sha256": mla_sha,
                     "measured_peak": MFMA_MEASURED_TFLOPS,
                     "measured_peak_note": "bf16 MFMA-only issue rate, two waves per SIMD (microbenchmark)",
                     "algorithmic": f"4*H*D = {4 * s.H * s.D} flop per valid slot x {wc['sum_n_valid']} slots"},
    }
    if cold:
        pool_bytes = float(s.T * s.D_I * 2 * 2 + wc["pools"] * (s.D_I + 4))
        cmed = float(np.median(cold))
        res["pooling_cold"] = {"ms_median": cmed, "hbm_gbs": pool_bytes / (cmed / 1e3) / 1e9,
                               "frac_hbm": pool_bytes / (cmed / 1e3) / 1e9 / HBM_PEAK_GBS,
                               "warm_ms_median": float(ms_med[0]), "bytes": pool_bytes,
                               "note": "kpool_build over all tokens after a 512 MB write (L2 and Infinity Cache "
                                       "evicted); warm = the step's own launch"}
    if bwd is not None:
        res["backward"] = bwd
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(s, wl, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
