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


# Top-k selection made on GPU scores vs the oracle's selection on its own
# (float64, rounded to fp32) scores. The GPU scores sit within 2.7e-4 of the
# row scale of the oracle's (worst case measured on the workloads' rows, held
# to SCORE_RTOL), so the two selections can differ only where two pools score
# within twice that of each other at the k-th score: the swapped pools must
# lie within SELECT_RTOL * scale of the oracle's k-th score (scale = the
# larger of |k-th score| and the row's mean |score|). Rows with no other pool
# inside that band must agree bit for bit.
SELECT_RTOL = 2e-3


def _pool_of(tok, cu, cp, kpool):
    d = np.searchsorted(cu, tok, side="right") - 1
    return cp[d] + (tok - cu[d]) // kpool


def check_selection(g_idx, g_nv, ref_idx, ref_nv, ref_scores, cu, cp, kpool, q_pos, topk, what=""):
    """GPU index rows against the oracle's: slot counts, tails and padding equal;
    kept pools ascending, whole and visible; any pool kept by one side only is a
    near-tie at the k-th score; rows without a near-tie are identical."""
    cu = np.asarray(cu, np.int64)
    cp = np.asarray(cp, np.int64)
    assert np.array_equal(g_nv, ref_nv), f"{what}: slot counts differ"
    exact, swaps, worst = 0, 0, 0.0
    for i in range(g_idx.shape[0]):
        t = int(q_pos[i])
        d = int(np.searchsorted(cu, t, side="right") - 1)
        n = (t - int(cu[d]) + 1) // kpool
        lo = int(cp[d])
        k = min(topk, n)
        w = k * kpool
        assert np.array_equal(g_idx[i, w:], ref_idx[i, w:]), f"{what}: row {i} tail or padding differs"
        g = g_idx[i, :w].reshape(k, kpool).astype(np.int64)
        assert np.all(g == g[:, :1] + np.arange(kpool)), f"{what}: row {i} pools not whole"
        gp = _pool_of(g[:, 0], cu, cp, kpool)
        assert np.all(np.diff(gp) > 0), f"{what}: row {i} pools not ascending"
        assert k == 0 or (gp[0] >= lo and gp[-1] < lo + n), f"{what}: row {i} pool outside its visible range"
        if np.array_equal(g_idx[i, :w], ref_idx[i, :w]):
            exact += 1
            continue
        rp = _pool_of(ref_idx[i, :w:kpool].astype(np.int64), cu, cp, kpool)
        a, b = np.setdiff1d(gp, rp), np.setdiff1d(rp, gp)
        s = ref_scores[i, lo:lo + n].astype(np.float64)
        sk = np.sort(s)[::-1][k - 1]
        scale = max(abs(sk), float(np.abs(s).mean()))
        band = SELECT_RTOL * scale
        near = int(np.sum(np.abs(s - sk) <= band))
        assert near > 1, f"{what}: row {i} differs with no near-tie at the k-th score"
        for p in a:
            assert sk - band <= s[p - lo] <= sk, f"{what}: row {i} keeps pool {p} ({s[p - lo]} vs k-th {sk})"
        for p in b:
            assert sk <= s[p - lo] <= sk + band, f"{what}: row {i} drops pool {p} ({s[p - lo]} vs k-th {sk})"
        swaps += len(a)
        worst = max(worst, float(np.abs(s[np.concatenate([a, b]) - lo] - sk).max()) / scale)
    return {"rows": int(g_idx.shape[0]), "identical": exact, "swapped_pools": swaps, "worst_swap_rel": worst}
