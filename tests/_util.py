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
# stated bound is absolute, max |d| <= 2e-2 and mean |d| <= 2e-3, and that is
# what every workload of N(0,1) data is held to. Where latent rows are scaled
# up (the x8 rows of the 32K workload, the x100 rows of the exact-max cases)
# the outputs reach |o| of 8 to 100s, where one bf16 half-ulp of the output
# alone exceeds an absolute 2e-2; those cases ("scaled") are held to the same
# numbers relative to A = max(1, |o_ref|, sum_j p_j |v_j|), the magnitude of
# the terms the element sums (bf16 rounding of each weight moves an output by
# up to 2^-9 of that magnitude). Every check also reports the absolute
# figures and the error relative to max(1, |o_ref|), whichever is asserted.
OUT_MAX = 2e-2
OUT_MEAN = 2e-3
# lse (natural log): absolute 1e-3; "scaled" cases relative to max(1, |lse|)
# (their scores, and so the fp32 rounding of the QK dots, grow with the scale)
LSE_TOL = 1e-3


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Position of each E4M3 code on the ordered line of representable values
    (the magnitude bits grow with the value; -0 and +0 both sit at 0), so that
    adjacent values differ by one whatever their signs."""
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_key_codes(gpu: np.ndarray, ref: np.ndarray, what: str = "", max_frac: float = 1e-3) -> float:
    """Pooled-key codes: the GPU pools in fp32 and the oracle in fp64, so a
    rotated value on a rounding boundary may round to either neighbour; codes
    must agree but for at most max_frac of them, each one step apart."""
    step = np.abs(e4m3_ordinal(gpu) - e4m3_ordinal(ref))
    frac = float((step != 0).mean()) if step.size else 0.0
    assert frac <= max_frac, f"{what}: {frac:.2e} of key codes differ"
    assert step.size == 0 or step.max() <= 1, f"{what}: a key code differs by {int(step.max())} steps"
    return frac


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


def check_out(gpu: np.ndarray, ref: np.ndarray, what: str = "", ref_abs=None, scaled: bool = False) -> dict:
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    d = np.abs(g - r)
    info = {"abs_max": float(d.max()), "abs_mean": float(d.mean())}
    rel_o = d / np.maximum(1.0, np.abs(r))
    info.update(rel_o_max=float(rel_o.max()), rel_o_mean=float(rel_o.mean()))
    if ref_abs is not None:
        terms = d / np.maximum(1.0, np.maximum(np.abs(r), ref_abs.astype(np.float64)))
        info.update(rel_terms_max=float(terms.max()), rel_terms_mean=float(terms.mean()))
    info["rel_rmse"] = float(np.sqrt(((g - r) ** 2).sum() / max((r ** 2).sum(), 1e-30)))
    info["cos"] = float((g * r).sum() / max(np.sqrt((g * g).sum() * (r * r).sum()), 1e-30))
    if scaled:
        assert ref_abs is not None, "a scaled check needs the magnitude of the summed terms"
        mx, mean = info["rel_terms_max"], info["rel_terms_mean"]
    else:
        mx, mean = info["abs_max"], info["abs_mean"]
    assert mx <= OUT_MAX and mean <= OUT_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e} ({info})"
    return info


def check_lse(gpu: np.ndarray, ref: np.ndarray, what: str = "", scaled: bool = False) -> float:
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), what
    d = np.abs(gpu[fin].astype(np.float64) - ref[fin])
    if scaled:
        d = d / np.maximum(1.0, np.abs(ref[fin]))
    worst = float(d.max()) if d.size else 0.0
    assert worst <= LSE_TOL, f"{what}: lse error {worst:.3e}"
    return worst
