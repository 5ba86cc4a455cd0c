"""Shared checks of the HIP path against the oracle.

Protocol: scores within 1e-5 relative (values below 1e-6 of their head's
maximum within 1e-11 of that maximum, absolute); budgets, selections and
offsets bit-exact against the oracle's allocation run on the GPU's own fp32
scores; the flat cache bit-exact against the oracle's gather with those
selections; decode outputs within 1e-2 max-abs and 5e-3 relative L2 of the
oracle's float64 decode over the same cache.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np

from oracle import allocation, cache, scoring

SCORE_RTOL = 1e-5
SMALL = 1e-6
DEC_MAXABS = 1e-2
DEC_RELL2 = 5e-3


def log(msg: str):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def assert_scores_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    mx = np.max(np.abs(ref), axis=-1, keepdims=True)
    big = np.abs(ref) >= SMALL * mx
    err = np.abs(got - ref)
    ok = np.where(big, err <= SCORE_RTOL * np.abs(ref), err <= SCORE_RTOL * SMALL * mx)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        rel = (err / np.maximum(np.abs(ref), 1e-300))[~ok]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} scores out of tolerance, "
                             f"worst rel {rel.max():.3e}, first {idx.tolist()}")
    return float(np.max(np.where(big, err / np.maximum(np.abs(ref), 1e-300), 0.0)))


def assert_decode_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert np.all(np.isfinite(got)), what
    assert err.max() <= DEC_MAXABS and rel <= DEC_RELL2, f"{what}: max-abs {err.max():.3e}, rel-L2 {rel:.3e}"
    return float(err.max()), rel


def oracle_scores(scorer, q, k, v, w_o, pool, eps, lse=None):
    """Oracle scores of one instance (float64 inputs); `lse` [Hq, w] is the
    supplied window-row normaliser of the single-pass entry point."""
    if scorer == "snapkv":
        return scoring.snapkv_scores(q, k, pool, lse), None
    if scorer == "lava":
        s, _ = scoring.lava_scores(q, k, v, pool, lse=lse)
        return s, None
    if scorer == "laprox":   # w_o in the nn.Linear layout; the oracle takes its transpose
        return scoring.laprox_scores(q, k, v, w_o.T, lse), None
    # criticalkv: w_o given in the nn.Linear layout [hidden, hq*d]; the oracle
    # takes the pages' W^O = its transpose.
    s, comp, _, _ = scoring.criticalkv_scores(q, k, v, w_o.T, pool, eps, lse)
    return s, comp


def check_selection(gpu_b, gpu_off, gpu_sel, ref_budgets, ref_sel, what, off_ref=None):
    assert np.array_equal(gpu_b, np.asarray(ref_budgets)), f"{what}: budgets {gpu_b} vs {ref_budgets}"
    for g, (a, b) in enumerate(zip(gpu_sel, ref_sel)):
        assert np.array_equal(a, np.asarray(b)), f"{what}: head {g} selection differs"
    if off_ref is not None:
        assert gpu_off == off_ref, f"{what}: sel_off {gpu_off} vs {off_ref}"


def check_flat(kf, vf, seg_start, seg_len, inst, hkv, k64, v64, sel, w, what):
    """Flat segments of one instance against the oracle gather (exact)."""
    kh = cache.compact(k64, sel, w)
    vh = cache.compact(v64, sel, w)
    for g in range(hkv):
        s = inst * hkv + g
        st, ln = int(seg_start[s]), int(seg_len[s])
        assert ln == kh[g].shape[0], f"{what}: segment {s} length {ln} vs {kh[g].shape[0]}"
        assert np.array_equal(kf[st:st + ln], kh[g]), f"{what}: K segment {s} differs"
        assert np.array_equal(vf[st:st + ln], vh[g]), f"{what}: V segment {s} differs"
    return kh, vh


def jaccard(a_sel, b_sel):
    inter = sum(len(np.intersect1d(a, b)) for a, b in zip(a_sel, b_sel))
    union = sum(len(np.union1d(a, b)) for a, b in zip(a_sel, b_sel))
    return inter / union if union else 1.0


def near_tie_in_layer_split(e: np.ndarray, Bp: int, tol: float = 1e-9) -> bool:
    """True when the largest-remainder split of B' * e / sum(e) can be changed
    by float64 rounding differences of size `tol`: some share lies within tol of
    an integer (its floor can flip), or the remainders at the cut-off rank (the
    last one given an extra unit and the first one not) are within tol of each
    other.  Remainder ties elsewhere decide nothing."""
    e = np.asarray(e, dtype=np.float64)
    E = e.sum()
    x = Bp * e / E if E > 0 else np.full(e.size, Bp / e.size)
    fl = np.floor(x)
    fr = x - fl
    if (np.minimum(fr, 1.0 - fr) < tol).any():
        return True
    deficit = int(round(Bp - fl.sum()))
    if 0 < deficit < e.size:
        srt = np.sort(fr)[::-1]
        return bool(srt[deficit - 1] - srt[deficit] < tol)
    return False


def check_lava_layer_budgets(gpu_lb, ref_lb, e, Bp, what, same_sum: bool = True) -> bool:
    """The device's LAVa layer budgets against the oracle's split.  Equal: True.
    Different: only allowed at a float64 near-tie of the split, and then the
    device's budgets must still be a valid split (non-negative, summing to B',
    each within one unit of the oracle's; with same_sum=False, as under the
    online prefill's caps, the sums may differ); returns False so the caller
    checks the selections under the device's own budgets."""
    gpu_lb = np.asarray(gpu_lb, dtype=np.int64)
    ref_lb = np.asarray(ref_lb, dtype=np.int64)
    if np.array_equal(gpu_lb, ref_lb):
        return True
    assert near_tie_in_layer_split(e, Bp), f"{what}: layer budgets {gpu_lb} vs {ref_lb} with no near-tie"
    assert (gpu_lb >= 0).all() and (not same_sum or int(gpu_lb.sum()) == int(ref_lb.sum())), \
        f"{what}: invalid layer budgets"
    assert np.abs(gpu_lb - ref_lb).max() <= 1, f"{what}: layer budgets differ by more than one unit"
    log(f"  {what}: layer budgets differ at a float64 near-tie (layers "
        f"{np.flatnonzero(gpu_lb != ref_lb).tolist()}); selections checked under the device's budgets")
    return False
