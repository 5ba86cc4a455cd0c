"""Budget allocation and selection (oracle; exact integer budgets; test infrastructure only).

Ordering rule used everywhere: a larger score ranks first; equal scores rank by
the smaller flat index g*p + k (within one head: the smaller token index).
-0.0 equals +0.0.  The pages leave ties open; this is the deterministic reading.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def rank_order(x: np.ndarray) -> np.ndarray:
    """Indices of a 1-D score vector from best to worst: by (-score, index)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    return np.lexsort((np.arange(x.size), -x))


def top_indices(x: np.ndarray, k: int) -> np.ndarray:
    return rank_order(x)[:k]


def safeguard_budgets(counts: Sequence[int], total: int, alpha: Tuple[int, int]) -> np.ndarray:
    """Ada-KV safeguard, integer form.

    Ada-KV notes, Algorithm 2, step 8: the final budget of head i is
    alpha * B_i* + (1 - alpha) * B / h, with B the prefix budget and h the
    number of KV heads.  With alpha = a/b every head's real budget is
    N_g / Den, N_g = a*h*f_g + (b - a)*B, Den = b*h.  The integer budgets are
    the floors plus one extra unit for the heads with the largest remainders
    (equal remainders: the lower head first), so they sum to B exactly.
    """
    a, b = int(alpha[0]), int(alpha[1])
    if not (0 <= a <= b and b > 0):
        raise ValueError("alpha must be a/b with 0 <= a <= b, b > 0")
    h = len(counts)
    den = b * h
    num = [a * h * int(f) + (b - a) * int(total) for f in counts]
    q = [x // den for x in num]
    r = [x % den for x in num]
    deficit = int(total) - sum(q)
    assert 0 <= deficit < max(h, 1) or h == 0
    for g in sorted(range(h), key=lambda g: (-r[g], g))[:deficit]:
        q[g] += 1
    return np.asarray(q, dtype=np.int64)


def ada_allocate(score: np.ndarray, budget: int, w: int, alpha: Tuple[int, int] = (1, 5)) -> Dict:
    """Ada-KV allocation and per-head top-k for one layer instance.

    Ada-KV notes, Algorithm 1 (concatenate all heads' weights, take the top B,
    count per head) inside Algorithm 2: step 6 removes the window from the
    budget (B - winsize * h, h = KV heads because entries are stored per KV
    head), step 7 runs Algorithm 1, step 8 applies the safeguard, step 9 takes
    each head's top-B_i (Theorem 3.2), steps 10-11 keep those entries, in
    ascending token order, followed by the window.
    score: [Hkv, p] float (>= 0).  Returns dict with P, counts f, budgets, sel.
    """
    score = np.asarray(score, dtype=np.float64)
    hkv, p = score.shape
    P = int(budget) - w * hkv
    if P < 0 or P > hkv * p:
        raise ValueError("budget outside [w*Hkv, n*Hkv]")
    top = top_indices(score.ravel(), P)
    counts = np.bincount(top // p, minlength=hkv).astype(np.int64)
    budgets = safeguard_budgets(counts, P, alpha)
    sel = [np.sort(top_indices(score[g], int(budgets[g]))) for g in range(hkv)]
    return {"P": P, "counts": counts, "budgets": budgets, "sel": sel}


def layer_entropy(s: np.ndarray) -> float:
    """LAVa layer uncertainty: entropy of the normalised scores divided by the
    number of entries (LAVa notes, "基于不确定性的层预算分配"), natural log,
    0 * log 0 = 0.  An all-zero layer has entropy 0."""
    s = np.asarray(s, dtype=np.float64).ravel()
    tot = s.sum()
    if tot <= 0:
        return 0.0
    sh = s / tot
    nz = sh > 0
    return float(-(sh[nz] * np.log(sh[nz])).sum() / s.size)


def largest_remainder(x: np.ndarray, total: int) -> np.ndarray:
    """Integers summing to `total`: floors of x plus one for the largest
    fractional parts (equal parts: lower index first)."""
    x = np.asarray(x, dtype=np.float64)
    fl = np.floor(x).astype(np.int64)
    deficit = int(total) - int(fl.sum())
    rem = x - fl
    order = np.lexsort((np.arange(x.size), -rem))
    fl[order[:deficit]] += 1
    return fl


def lava_layer_budgets(scores: np.ndarray, total: int, w: int) -> Tuple[np.ndarray, np.ndarray]:
    """LAVa dynamic layer budgets.

    LAVa notes, "基于不确定性的层预算分配" and the quick summary: the total
    budget is split across layers in proportion to e_l.  Windows are kept
    outside the split: B' = total - L * w * Hkv is what the layers share.  If
    every layer has zero entropy the split is uniform.  B' must not exceed one
    layer's prefix entries (Hkv * p): then no layer's share can overflow it.
    scores: [L, Hkv, p] pooled prefix scores.  Returns (budgets [L], e [L]).
    """
    L, hkv, p = scores.shape
    Bp = int(total) - L * w * hkv
    if Bp < 0 or Bp > hkv * p:
        raise ValueError("LAVa total budget out of range")
    e = np.array([layer_entropy(scores[l]) for l in range(L)])
    E = e.sum()
    x = Bp * e / E if E > 0 else np.full(L, Bp / L)
    return largest_remainder(x, Bp), e


def lava_allocate(scores: np.ndarray, total: int, w: int, layer_budgets: np.ndarray | None = None) -> Dict:
    """LAVa layer-wise eviction with dynamic head budgets.

    LAVa notes, "动态头预算的逐层缓存驱逐": the scores of all heads in a layer
    are flattened into one array and the layer's B_l best entries are kept, so
    head budgets follow from the ranking; no safeguard is applied.
    layer_budgets: the B_l to use instead of the entropy split (the selection
    step alone, e.g. under another device's split of a float64 near-tie); they
    must sum to B' = total - L*w*Hkv, each within [0, Hkv*p].
    Returns dict with layer budgets, e, per-layer head budgets [L, Hkv], sel[l][g].
    """
    scores = np.asarray(scores, dtype=np.float64)
    L, hkv, p = scores.shape
    bl, e = lava_layer_budgets(scores, total, w)
    if layer_budgets is not None:
        bl = np.asarray(layer_budgets, dtype=np.int64)
        if bl.shape != (L,) or int(bl.sum()) != int(total) - L * w * hkv or (bl < 0).any() or (bl > hkv * p).any():
            raise ValueError("layer budgets must be L values in [0, Hkv*p] summing to B'")
    budgets, sel = layer_top_select(scores, bl)
    return {"layer_budgets": bl, "entropy": e, "budgets": budgets, "sel": sel}


def layer_top_select(scores: np.ndarray, layer_budgets: Sequence[int]):
    """Each layer keeps the top B_l of its flattened [Hkv, p] scores, ranked by
    (-score, g*p + t) (LAVa notes, "动态头预算的逐层缓存驱逐"); the head budgets
    are the per-head counts.  Returns (budgets [L, Hkv], sel[l][g] ascending)."""
    scores = np.asarray(scores, dtype=np.float64)
    L, hkv, p = scores.shape
    budgets = np.zeros((L, hkv), dtype=np.int64)
    sel: List[List[np.ndarray]] = []
    for l in range(L):
        top = top_indices(scores[l].ravel(), int(layer_budgets[l]))
        budgets[l] = np.bincount(top // p, minlength=hkv)
        sel.append([np.sort(top[top // p == g] % p) for g in range(hkv)])
    return budgets, sel


def criticalkv_allocate(score: np.ndarray, composite: np.ndarray, budget: int, w: int,
                        alpha: Tuple[int, int] = (1, 5), ck: Tuple[int, int] = (1, 2)) -> Dict:
    """CriticalKV two-stage selection on Ada-KV budgets.

    CriticalKV notes, "两阶段贪心选择算法": per head, stage 1 keeps the top
    b' = alpha_ck * b entries by attention, stage 2 keeps the top
    b'' = (1 - alpha_ck) * b of the remaining entries by the composite score.
    "作为通用插件融入现有驱逐流水线": only the selection changes; the budgets are
    Ada-KV's, computed on the attention score.  b' is rounded down.
    """
    base = ada_allocate(score, budget, w, alpha)
    hkv, p = score.shape
    c0, c1 = int(ck[0]), int(ck[1])
    sel, s1, s2 = [], [], []
    for g in range(hkv):
        b = int(base["budgets"][g])
        b1 = (b * c0) // c1
        b2 = b - b1
        first = top_indices(score[g], b1)
        rest = np.setdiff1d(np.arange(p), first, assume_unique=True)   # ascending
        second = rest[top_indices(np.asarray(composite[g])[rest], b2)]
        s1.append(np.sort(first))
        s2.append(np.sort(second))
        sel.append(np.sort(np.concatenate([first, second])))
    out = dict(base)
    out.update({"sel": sel, "stage1": s1, "stage2": s2})
    return out


def global_allocate(scores: np.ndarray, total: int, w: int) -> Dict:
    """Model-wide top-k over every head of every instance.

    LaProx page, Algorithm 1: S = TopK(p, B_total), with window tokens scored
    infinity (so always kept); abstract and Section 1: tokens of all heads and
    all layers get globally comparable scores and one model-wide selection
    replaces per-head decisions.  The windows are kept outside the ranking:
    B' = total - L * w * Hkv prefix entries are taken from the flattened
    [L, Hkv, p] scores by (-score, flat index).  A per-layer top-k is this
    with L = 1.
    scores: [L, Hkv, p].  Returns dict with B', budgets [L, Hkv], layer totals
    and sel[l][g] (ascending).
    """
    scores = np.asarray(scores, dtype=np.float64)
    L, hkv, p = scores.shape
    Bp = int(total) - L * w * hkv
    if Bp < 0 or Bp > L * hkv * p:
        raise ValueError("total budget out of range")
    top = top_indices(scores.ravel(), Bp)
    row = top // p
    budgets = np.bincount(row, minlength=L * hkv).astype(np.int64).reshape(L, hkv)
    sel = [[np.sort(top[row == l * hkv + g] % p) for g in range(hkv)] for l in range(L)]
    return {"Bp": Bp, "budgets": budgets, "layer_budgets": budgets.sum(axis=1), "sel": sel}


def ada_floor_allocate(score: np.ndarray, budget: int, w: int, alpha: Tuple[int, int] = (1, 5)) -> Dict:
    """The floor-then-global reading of the Ada-KV safeguard.

    Ada-KV notes, Algorithm 2 step 8 and the introduction: the safeguard keeps
    highly sparse heads from receiving too small a budget.  Read as a floor:
    every head first keeps its own top f0 = floor(alpha * P / h) entries, then
    one top (P - h * f0) over all heads' remaining entries (Algorithm 1 on what
    is left) decides the rest; B_g = f0 + head g's share.  Ranking everywhere
    by (-score, flat index g*p + k).  Of all budget splits with B_g >= f0 and
    sum P, this one keeps the largest total score.
    """
    score = np.asarray(score, dtype=np.float64)
    hkv, p = score.shape
    P = int(budget) - w * hkv
    if P < 0 or P > hkv * p:
        raise ValueError("budget outside [w*Hkv, n*Hkv]")
    a, b = int(alpha[0]), int(alpha[1])
    if not (0 <= a <= b and b > 0):
        raise ValueError("alpha must be a/b with 0 <= a <= b, b > 0")
    f0 = (a * P) // (b * hkv)
    first = [top_indices(score[g], f0) for g in range(hkv)]
    taken = np.zeros((hkv, p), dtype=bool)
    for g in range(hkv):
        taken[g, first[g]] = True
    flat = score.ravel()
    rest = np.flatnonzero(~taken.ravel())                      # ascending flat indices
    second = rest[top_indices(flat[rest], P - hkv * f0)]
    counts = np.bincount(second // p, minlength=hkv).astype(np.int64)
    budgets = f0 + counts
    sel = [np.sort(np.concatenate([first[g], second[second // p == g] % p])) for g in range(hkv)]
    return {"P": P, "floor": f0, "counts": counts, "budgets": budgets, "sel": sel}


def streaming_allocate(hkv: int, p: int, budget: int, w: int, sinks: int = 4) -> Dict:
    """StreamingLLM baseline on the same cache layout.

    Ada-KV notes, "缓存驱逐方法的分类与局限" item 1 and the Ada-KV paper,
    "Baselines" / "Parameters": keep a few initial tokens (4 sinks) and the most
    recent window.  Under a budget B the window tokens are kept as for every
    other method, the prefix share P = B - w*Hkv is split evenly over the heads
    (floors, one more for the lowest P mod Hkv heads), and head g keeps its
    first min(sinks, B_g) prefix tokens and its most recent remaining ones.
    """
    P = int(budget) - w * hkv
    if P < 0 or P > hkv * p:
        raise ValueError("budget outside [w*Hkv, n*Hkv]")
    if sinks < 0:
        raise ValueError("sinks must be >= 0")
    budgets = np.full(hkv, P // hkv, dtype=np.int64)
    budgets[:P % hkv] += 1
    sel = []
    for g in range(hkv):
        bg = int(budgets[g])
        s = min(sinks, bg)
        sel.append(np.concatenate([np.arange(s), np.arange(p - (bg - s), p)]).astype(np.int64))
    return {"P": P, "budgets": budgets, "sel": sel}


def lava_online_steps(scores: np.ndarray, total: int, w: int) -> List[Dict]:
    """LAVa online prefill: layer budgets after each layer's prefill.

    LAVa notes, "在线预填充与层预算调整": prefill and eviction run layer by
    layer; after layer l is prefilled the lower layers are compressed again
    with the same LAVa scores, their budgets shrinking as the memory is shared
    with more layers.  The pages leave the schedule open; the reading here:
    after layer l the l + 1 layers present share B'(l) = total - (l+1)*w*Hkv
    prefix entries by the entropy rule of "基于不确定性的层预算分配" (the same
    e_j, from each layer's full scores, and the same largest-remainder split as
    lava_layer_budgets), and no layer may grow: B_j(l) = min(split_j, B_j(l-1)),
    with Hkv*p for a layer's first step.  Each layer keeps the top B_j(l) of its
    flattened scores (no safeguard, "动态头预算的逐层缓存驱逐"); with the same
    ranking every step's selection lies inside the previous one.  The sum of
    the budgets may fall below B'(l) where a cap binds.
    scores: [L, Hkv, p].  Returns one dict per step l with layer_budgets [l+1],
    budgets [l+1, Hkv] and sel[j][g].
    """
    scores = np.asarray(scores, dtype=np.float64)
    L, hkv, p = scores.shape
    if int(total) < L * w * hkv:
        raise ValueError("total budget smaller than the windows")
    steps = []
    prev = np.zeros(0, dtype=np.int64)
    for l in range(L):
        st = lava_online_step(scores[:l + 1], total, w, prev)
        steps.append(st)
        prev = st["layer_budgets"]
    return steps


def lava_online_step(scores: np.ndarray, total: int, w: int, prev: Sequence[int]) -> Dict:
    """One step of lava_online_steps: the I = l + 1 layers present (scores
    [I, Hkv, p]) share B'(l) = total - I*w*Hkv by the entropy split, each
    capped by its budget of the previous step (`prev`, I - 1 values; Hkv*p for
    the newest layer), then each keeps its flattened top B_j."""
    scores = np.asarray(scores, dtype=np.float64)
    I, hkv, p = scores.shape
    e = np.array([layer_entropy(scores[j]) for j in range(I)])
    Bp = int(total) - I * w * hkv
    E = e.sum()
    x = Bp * e / E if E > 0 else np.full(I, Bp / I)
    split = largest_remainder(x, Bp)
    cap = np.concatenate([np.asarray(prev, dtype=np.int64), [hkv * p]])
    lb = np.minimum(split, cap)
    budgets, sel = layer_top_select(scores, lb)
    return {"layer_budgets": lb, "split": split, "budgets": budgets, "sel": sel, "Bp": Bp, "entropy": e}
