"""Shared helpers of the GPU parity tests: host<->device marshalling and the
tolerance checks (the thresholds and their derivation are stated once, here)."""
import numpy as np
import torch


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_bf16_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


# ---------------------------------------------------------------- tolerances --
# Indexer scores (FP8 operands, fp32 accumulation on the GPU vs exact float64
# in the oracle): relative 2e-2 per element, relative to the larger of the
# element and the mean magnitude of its row's visible scores (a sum of signed
# per-head terms can cancel to near zero; the row mean is the scale of the
# quantity being ranked).
SCORE_RTOL = 2e-2

# Attention output (bf16 in, fp32 accumulation, bf16 out vs float64): the
# error divided by max(1, a) must stay below 2e-2 at every element and below
# 2e-3 on average, where a = sum_j p_j |v_j| is the magnitude of the terms the
# element sums (the oracle returns it; without it |o_ref| stands in). Wherever
# a <= 1 (every workload without the x8 rows) this is the absolute bound
# itself; with x8 rows one bf16 half-ulp of a term alone exceeds an absolute
# 2e-2, so the bound scales with the terms.
OUT_MAX = 2e-2
OUT_MEAN = 2e-3
LSE_TOL = 1e-3


def check_scores(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    vis = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), vis), f"{what}: visibility pattern differs"
    assert np.all(np.isneginf(gpu[~vis])), f"{what}: non-visible entries must be -inf"
    err = np.zeros_like(ref, dtype=np.float64)
    worst = 0.0
    for r in range(ref.shape[0]):
        v = vis[r]
        if not v.any():
            continue
        rr = ref[r, v].astype(np.float64)
        gg = gpu[r, v].astype(np.float64)
        floor = max(np.abs(rr).mean(), 1e-30)
        rel = np.abs(gg - rr) / np.maximum(np.abs(rr), floor)
        err[r, v] = rel
        worst = max(worst, float(rel.max()))
    assert worst <= SCORE_RTOL, f"{what}: worst relative score error {worst:.3e}"
    return {"worst_rel": worst}


def check_out(gpu: np.ndarray, ref: np.ndarray, what: str = "", ref_abs=None) -> dict:
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    mag = np.abs(r) if ref_abs is None else np.maximum(np.abs(r), ref_abs.astype(np.float64))
    scaled = np.abs(g - r) / np.maximum(1.0, mag)
    mx, mean = float(scaled.max()), float(scaled.mean())
    rel_rmse = float(np.sqrt(((g - r) ** 2).sum() / max((r ** 2).sum(), 1e-30)))
    cos = float((g * r).sum() / max(np.sqrt((g * g).sum() * (r * r).sum()), 1e-30))
    abs_max = float(np.abs(g - r).max())
    assert mx <= OUT_MAX and mean <= OUT_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e} (abs max {abs_max:.3e})"
    return {"max": mx, "mean": mean, "abs_max": abs_max, "rel_rmse": rel_rmse, "cos": cos}


def check_lse(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), what
    d = np.abs(gpu[fin].astype(np.float64) - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
    assert d.size == 0 or d.max() <= LSE_TOL, f"{what}: lse error {d.max():.3e}"
