"""Pins for the oracle's allocation and selection (CPU): hand-worked fixtures,
exact rational arithmetic, Theorem 3.2 and Theorem 3.3 of the Ada-KV notes by
brute force, closed forms and invariants."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.stats

from oracle import allocation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_sel(tokens):
    heads, cur = [], []
    for t in tokens:
        if t == "|":
            heads.append(cur)
            cur = []
        else:
            cur.append(int(t))
    heads.append(cur)
    return heads


def load_alg1():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "alg1_hand_example.txt")) if l.strip() and not l.startswith("#")]
    d = {"cases": []}
    for r in rows:
        if r[0] == "scores":
            d["scores"] = np.array([float(x) for x in r[1:]])
        elif r[0] in ("heads", "w", "budget"):
            d[r[0]] = int(r[1])
        elif r[0] == "counts":
            d["counts"] = [int(x) for x in r[1:]]
        elif r[0] == "alpha":
            a, b = int(r[1]), int(r[2])
            i = r.index("budgets")
            j = r.index("sel")
            d["cases"].append(((a, b), [int(x) for x in r[i + 1:j]], _parse_sel(r[j + 1:])))
    return d


def check_alg1_fixture(fn) -> bool:
    g = load_alg1()
    s = g["scores"].reshape(g["heads"], -1)
    for alpha, budgets, sel in g["cases"]:
        out = fn(s, g["budget"], g["w"], alpha)
        if list(out["counts"]) != g["counts"] or list(out["budgets"]) != budgets:
            return False
        if [list(x) for x in out["sel"]] != sel:
            return False
    return True


def test_alg1_hand_example():
    assert check_alg1_fixture(allocation.ada_allocate)


def test_ck_hand_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "ck_hand_example.txt")) if l.strip() and not l.startswith("#")]
    att = comp = None
    for r in rows:
        if r[0] == "attention":
            att = np.array([float(x) for x in r[1:]])[None]
        elif r[0] == "composite":
            comp = np.array([float(x) for x in r[1:]])[None]
        elif r[0] == "w":
            w = int(r[1])
        elif r[0] == "budget":
            budget = int(r[1])
        elif r[0] == "ck":
            ck = (int(r[1]), int(r[2]))
            want = [int(x) for x in r[4:]]
            out = allocation.criticalkv_allocate(att, comp, budget, w, (1, 5), ck)
            assert list(out["sel"][0]) == want, ck


def safeguard_fraction(counts, total, alpha):
    """alpha*f + (1-alpha)*P/h in exact rationals, then largest remainder."""
    a = Fraction(alpha[0], alpha[1])
    h = len(counts)
    x = [a * f + (1 - a) * Fraction(total, h) for f in counts]
    fl = [math.floor(v) for v in x]
    rem = [v - f for v, f in zip(x, fl)]
    for g in sorted(range(h), key=lambda g: (-rem[g], g))[:total - sum(fl)]:
        fl[g] += 1
    return fl


def check_safeguard(fn) -> bool:
    r = np.random.default_rng(11)
    for _ in range(300):
        h = int(r.integers(1, 9))
        p = int(r.integers(1, 50))
        f = r.multinomial(int(r.integers(0, h * p + 1)), np.ones(h) / h)
        f = np.minimum(f, p)
        P = int(f.sum())
        alpha = [(1, 5), (0, 1), (1, 1), (1, 2), (3, 7)][int(r.integers(0, 5))]
        if list(fn(f, P, alpha)) != safeguard_fraction(list(f), P, alpha):
            return False
    return True


def test_safeguard_matches_exact_rationals():
    assert check_safeguard(allocation.safeguard_budgets)


def test_budget_invariants_random():
    r = np.random.default_rng(12)
    for t in range(60):
        hkv, p, w = int(r.integers(1, 9)), int(r.integers(1, 40)), int(r.integers(0, 4))
        s = r.random((hkv, p)) ** int(r.integers(1, 8))
        if t % 5 == 0:
            s = np.round(s, 1)                       # many ties
        P = int(r.integers(0, hkv * p + 1))
        out = allocation.ada_allocate(s, P + w * hkv, w, (1, 5))
        b = out["budgets"]
        assert b.sum() == P and np.all(b >= 0) and np.all(b <= p)
        assert out["counts"].sum() == P
        for g in range(hkv):
            assert len(out["sel"][g]) == b[g] and np.all(np.diff(out["sel"][g]) > 0)


def test_alpha_zero_is_uniform_and_alpha_one_is_counts():
    r = np.random.default_rng(13)
    s = r.random((5, 30)) ** 4
    P = 47
    u = allocation.ada_allocate(s, P, 0, (0, 1))["budgets"]
    assert list(u) == [10, 10, 9, 9, 9]
    o = allocation.ada_allocate(s, P, 0, (1, 1))
    assert list(o["budgets"]) == list(o["counts"])


def test_all_equal_scores_take_first_flat_indices():
    s = np.full((4, 10), 0.25)
    out = allocation.ada_allocate(s, 23, 0, (1, 1))
    assert list(out["counts"]) == [10, 10, 3, 0]
    assert list(out["sel"][2]) == [0, 1, 2]


def topsum(row_sorted_cum, b):
    return row_sorted_cum[b]


def test_theorem33_brute_force_tiny_config_shape():
    """Ada-KV notes, Theorem 3.3: Algorithm 1's split attains the largest retained
    mass over every split of the budget.  Tiny config shape: 4 heads, p = 60,
    prefix budget 48 -> 20,825 compositions."""
    r = np.random.default_rng(14)
    hkv, p, P = 4, 60, 48
    temps = [0.2, 0.5, 1.0, 3.0]
    s = np.stack([np.exp(r.standard_normal(p) / t) for t in temps])
    s /= s.sum(axis=1, keepdims=True)
    out = allocation.ada_allocate(s, P, 0, (1, 1))
    cums = [np.concatenate([[0.0], np.cumsum(np.sort(s[g])[::-1])]) for g in range(hkv)]
    best, n_comp = -1.0, 0
    for b0 in range(P + 1):
        for b1 in range(P - b0 + 1):
            for b2 in range(P - b0 - b1 + 1):
                b3 = P - b0 - b1 - b2
                n_comp += 1
                val = cums[0][b0] + cums[1][b1] + cums[2][b2] + cums[3][b3]
                best = max(best, val)
    assert n_comp == 20825
    got = sum(cums[g][out["budgets"][g]] for g in range(hkv))
    assert got >= best * (1 - 1e-12)
    # the adaptive split is not the uniform one here, and beats it
    uni = sum(cums[g][P // hkv] for g in range(hkv))
    assert got > uni


def test_theorem32_brute_force_subsets():
    """Ada-KV notes, Theorem 3.2: given B_i, per-head top-k maximises the
    retained mass; checked over every subset of a 12-token head."""
    r = np.random.default_rng(15)
    p = 12
    for trial in range(6):
        s = r.random(p) ** 3
        if trial == 5:
            s = np.round(s, 1)
        for b in range(p + 1):
            best = max(s[list(c)].sum() for c in itertools.combinations(range(p), b)) if b else 0.0
            sel = allocation.top_indices(s, b)
            assert math.isclose(s[sel].sum(), best, rel_tol=1e-12, abs_tol=1e-15)


def test_tie_break_prefers_lower_index():
    s = np.array([[0.5, 0.2, 0.2, 0.2, 0.1]])
    out = allocation.ada_allocate(s, 3, 0, (1, 1))
    assert list(out["sel"][0]) == [0, 1, 2]
    z = np.array([[0.0, -0.0, 0.0]])
    assert list(allocation.ada_allocate(z, 2, 0, (1, 1))["sel"][0]) == [0, 1]


# ---------------------------------------------------------------- LAVa budgets
def test_entropy_uniform_closed_form_and_scipy():
    hkv, p = 8, 100
    s = np.full((hkv, p), 0.3)
    e = allocation.layer_entropy(s)
    assert math.isclose(e, math.log(hkv * p) / (hkv * p), rel_tol=1e-13)
    r = np.random.default_rng(16)
    x = r.random((3, 17)) ** 5
    assert math.isclose(allocation.layer_entropy(x), scipy.stats.entropy(x.ravel()) / x.size, rel_tol=1e-12)


def test_lava_budgets_sum_and_symmetry():
    r = np.random.default_rng(17)
    L, hkv, p, w = 6, 4, 50, 3
    layer = r.random((hkv, p)) ** 3
    same = np.stack([layer] * L)
    bl, e = allocation.lava_layer_budgets(same, 150 + L * w * hkv, w)
    assert bl.sum() == 150 and bl.max() - bl.min() <= 1
    mixed = np.stack([r.random((hkv, p)) ** (1 + 2 * l) for l in range(L)])
    bl2, e2 = allocation.lava_layer_budgets(mixed, 150 + L * w * hkv, w)
    assert bl2.sum() == 150
    # lower entropy (sharper layer) -> no larger budget
    order = np.argsort(-e2)
    assert np.all(np.diff(bl2[order]) <= 1)


def test_lava_allocate_is_flattened_top():
    r = np.random.default_rng(18)
    L, hkv, p, w = 3, 4, 30, 2
    s = r.random((L, hkv, p)) ** 4
    out = allocation.lava_allocate(s, 100 + L * w * hkv, w)
    assert out["layer_budgets"].sum() == 100
    for l in range(L):
        flat = s[l].ravel()
        thr = np.sort(flat)[::-1][out["layer_budgets"][l] - 1] if out["layer_budgets"][l] else np.inf
        kept = np.concatenate([g * p + out["sel"][l][g] for g in range(hkv)])
        assert kept.size == out["layer_budgets"][l]
        assert np.all(flat[kept] >= thr)
        assert list(out["budgets"][l]) == [len(x) for x in out["sel"][l]]


# ---------------------------------------------------------------- CriticalKV selection
def test_criticalkv_limits_and_partition():
    r = np.random.default_rng(19)
    hkv, p, w = 4, 40, 2
    a = r.random((hkv, p)) ** 3
    c = r.random((hkv, p))
    budget = 70 + w * hkv
    same = allocation.criticalkv_allocate(a, c, budget, w, (1, 5), (1, 1))
    base = allocation.ada_allocate(a, budget, w, (1, 5))
    assert [list(x) for x in same["sel"]] == [list(x) for x in base["sel"]]
    only2 = allocation.criticalkv_allocate(a, c, budget, w, (1, 5), (0, 1))
    for g in range(hkv):
        assert list(only2["sel"][g]) == sorted(allocation.top_indices(c[g], base["budgets"][g]))
    half = allocation.criticalkv_allocate(a, c, budget, w, (1, 5), (1, 2))
    for g in range(hkv):
        s1, s2 = set(half["stage1"][g]), set(half["stage2"][g])
        assert not (s1 & s2)
        assert len(s1) == base["budgets"][g] // 2 and len(s1) + len(s2) == base["budgets"][g]


# ---------------------------------------------------------------- planted mistakes
def _reversed_alpha(f, P, alpha):
    a, b = alpha
    return allocation.safeguard_budgets(f, P, (b - a, b))


def _index_tie_reversed(score, budget, w, alpha):
    flipped = np.asarray(score)[:, ::-1]
    out = allocation.ada_allocate(flipped, budget, w, alpha)
    p = flipped.shape[1]
    out["sel"] = [np.sort(p - 1 - s) for s in out["sel"]]
    return out


def test_pins_catch_planted_mistakes():
    assert not check_safeguard(_reversed_alpha)
    assert not check_alg1_fixture(_index_tie_reversed)


# ---------------------------------------------------------------- model-wide top-k (LaProx)
def check_global_brute_force(fn) -> bool:
    """Scores drawn from a few values (many ties): the kept entries are the
    first B' of every (instance, head, token) triple sorted by Python's own
    tuple order (-score, l, g, t); budgets are their counts."""
    r = np.random.default_rng(51)
    L, hkv, p, w = 3, 2, 9, 2
    s = r.integers(0, 4, (L, hkv, p)).astype(np.float64)
    for Bp in (0, 1, 7, 20, L * hkv * p):
        out = fn(s, Bp + L * w * hkv, w)
        order = sorted((-s[l, g, t], l, g, t) for l in range(L) for g in range(hkv) for t in range(p))[:Bp]
        for l in range(L):
            for g in range(hkv):
                want = sorted(t for (_, ll, gg, t) in order if (ll, gg) == (l, g))
                if list(out["sel"][l][g]) != want or out["budgets"][l][g] != len(want):
                    return False
    return True


def test_global_allocate_brute_force():
    assert check_global_brute_force(allocation.global_allocate)


def test_global_allocate_single_layer_is_ada_without_safeguard():
    """L = 1: one top-B' over the heads is Ada-KV's Algorithm 1 with the
    counts used as budgets (alpha = 1)."""
    r = np.random.default_rng(52)
    hkv, p, w = 4, 50, 3
    s = r.random((hkv, p)) ** 3
    for B in (w * hkv, w * hkv + 17, w * hkv + hkv * p):
        a = allocation.ada_allocate(s, B, w, (1, 1))
        gl = allocation.global_allocate(s[None], B, w)
        assert list(gl["budgets"][0]) == list(a["budgets"])
        assert all(list(x) == list(y) for x, y in zip(gl["sel"][0], a["sel"]))


def test_global_allocate_threshold_invariant():
    r = np.random.default_rng(53)
    L, hkv, p, w = 4, 3, 40, 2
    s = r.random((L, hkv, p)) ** 5
    out = allocation.global_allocate(s, 150 + L * w * hkv, w)
    assert out["budgets"].sum() == 150 and out["layer_budgets"].sum() == 150
    kept = np.zeros_like(s, dtype=bool)
    for l in range(L):
        for g in range(hkv):
            kept[l, g, out["sel"][l][g]] = True
    assert s[kept].min() >= s[~kept].max()
    with pytest.raises(ValueError):
        allocation.global_allocate(s, L * w * hkv - 1, w)


def _global_per_layer(scores, total, w):
    """Planted: equal per-layer shares instead of one model-wide ranking."""
    L, hkv, p = scores.shape
    Bp = total - L * w * hkv
    outs = [allocation.global_allocate(scores[l:l + 1], Bp // L + (l < Bp % L) + w * hkv, w) for l in range(L)]
    return {"budgets": np.stack([o["budgets"][0] for o in outs]), "sel": [o["sel"][0] for o in outs]}


def test_global_pins_catch_planted_mistakes():
    assert not check_global_brute_force(_global_per_layer)


# ---------------------------------------------------------------- floor-then-global safeguard
def check_floor_is_best_split_with_floor(fn) -> bool:
    """Brute force over every budget split B_g >= f0 with sum P: the floor
    reading keeps the largest total score, and its own split reaches it."""
    r = np.random.default_rng(61)
    hkv, p, w = 3, 7, 1
    ok = True
    for trial in range(6):
        s = r.random((hkv, p)) ** (1 + 3 * trial)
        for P in (0, 2, 5, 9, 14, hkv * p):
            out = fn(s, P + w * hkv, w, (1, 2))
            f0 = (P // 2) // hkv
            srt = -np.sort(-s, axis=1)
            best = max(sum(srt[g, :c[g]].sum() for g in range(hkv))
                       for c in itertools.product(range(f0, p + 1), repeat=hkv) if sum(c) == P)
            got = sum(s[g, out["sel"][g]].sum() for g in range(hkv))
            ok &= bool(np.isclose(got, best, rtol=1e-12)) and all(out["budgets"] >= f0)
            ok &= int(out["budgets"].sum()) == P
    return ok


def test_floor_reading_maximises_retained_score_under_the_floor():
    assert check_floor_is_best_split_with_floor(allocation.ada_floor_allocate)


def test_floor_reading_limits():
    r = np.random.default_rng(62)
    hkv, p, w = 4, 30, 2
    s = r.random((hkv, p)) ** 3
    for B in (w * hkv, w * hkv + 37, w * hkv + hkv * p):
        z = allocation.ada_floor_allocate(s, B, w, (0, 1))      # no floor: Algorithm 1's counts
        a = allocation.ada_allocate(s, B, w, (1, 1))
        assert list(z["budgets"]) == list(a["budgets"]) and all(
            list(x) == list(y) for x, y in zip(z["sel"], a["sel"]))
    full = allocation.ada_floor_allocate(s, w * hkv + 41, w, (1, 1))   # floor P // h = 10
    assert full["floor"] == 10 and sorted(full["budgets"])[0] >= 10 and full["budgets"].sum() == 41
    # every head keeps its own top-f0 entries
    for g in range(hkv):
        assert set(allocation.top_indices(s[g], 10)) <= set(full["sel"][g])


def test_floor_tie_order_brute_force():
    """Integer scores with many ties: the result is the per-head first f0 of
    (-score, k), then the first P - h*f0 of (-score, g, k) over the rest."""
    r = np.random.default_rng(63)
    hkv, p, w = 3, 8, 1
    s = r.integers(0, 3, (hkv, p)).astype(np.float64)
    for P in (0, 4, 11, 17, hkv * p):
        out = allocation.ada_floor_allocate(s, P + w * hkv, w, (3, 4))
        f0 = (3 * P) // (4 * hkv)
        first = {(g, t) for g in range(hkv) for (_, t) in sorted((-s[g, t], t) for t in range(p))[:f0]}
        rest = sorted((-s[g, t], g, t) for g in range(hkv) for t in range(p) if (g, t) not in first)
        keep = first | {(g, t) for (_, g, t) in rest[:P - hkv * f0]}
        for g in range(hkv):
            assert list(out["sel"][g]) == sorted(t for (gg, t) in keep if gg == g)


# ---------------------------------------------------------------- StreamingLLM
def test_streaming_closed_form():
    out = allocation.streaming_allocate(3, 20, 3 * 2 + 14, 2, sinks=4)
    assert list(out["budgets"]) == [5, 5, 4]
    assert list(out["sel"][0]) == [0, 1, 2, 3, 19] and list(out["sel"][2]) == [0, 1, 2, 3]
    small = allocation.streaming_allocate(2, 10, 2 * 3 + 5, 3, sinks=4)     # B_g = 3, 2 < sinks
    assert list(small["sel"][0]) == [0, 1, 2] and list(small["sel"][1]) == [0, 1]
    none = allocation.streaming_allocate(2, 10, 2 * 3, 3)
    assert all(x.size == 0 for x in none["sel"])
    full = allocation.streaming_allocate(2, 10, 2 * 13, 3)
    assert all(list(x) == list(range(10)) for x in full["sel"])
    nos = allocation.streaming_allocate(2, 10, 2 * 3 + 8, 3, sinks=0)       # pure recency
    assert list(nos["sel"][1]) == [6, 7, 8, 9]


def _floor_overlapping_stages(score, budget, w, alpha):
    """Planted: the global stage ranks every entry, the heads' floor entries
    included, so the two stages can pick the same entry twice."""
    hkv, p = score.shape
    P = budget - w * hkv
    f0 = (alpha[0] * P) // (alpha[1] * hkv)
    second = allocation.top_indices(score.ravel(), P - hkv * f0)
    sel = [np.union1d(allocation.top_indices(score[g], f0), second[second // p == g] % p) for g in range(hkv)]
    return {"budgets": np.array([x.size for x in sel]), "sel": sel}


def test_floor_pins_catch_planted_mistakes():
    assert not check_floor_is_best_split_with_floor(_floor_overlapping_stages)


# ---------------------------------------------------------------- LAVa online prefill
def test_lava_online_nested_and_bounded():
    r = np.random.default_rng(71)
    L, hkv, p, w = 5, 3, 40, 2
    s = r.random((L, hkv, p)) ** (1 + 4 * r.random((L, 1, 1)))
    total = L * w * hkv + 150
    steps = allocation.lava_online_steps(s, total, w)
    for l, st in enumerate(steps):
        assert len(st["layer_budgets"]) == l + 1
        # memory: the layers present never hold more than the total
        assert st["layer_budgets"].sum() + (l + 1) * w * hkv <= total
        for j in range(l + 1):
            assert st["budgets"][j].sum() == st["layer_budgets"][j]
            if l > 0 and j < l:
                # budgets only shrink and every selection lies inside the previous one
                assert st["layer_budgets"][j] <= steps[l - 1]["layer_budgets"][j]
                for g in range(hkv):
                    assert set(st["sel"][j][g]) <= set(steps[l - 1]["sel"][j][g])


def test_lava_online_last_step_is_offline_lava_when_no_cap_binds():
    """Smooth score distributions: the shares fall at every step, no cap binds,
    and the last step is the offline LAVa allocation of all layers."""
    r = np.random.default_rng(72)
    L, hkv, p, w = 4, 2, 60, 3
    s = r.random((L, hkv, p)) + 0.5
    total = L * w * hkv + 90
    steps = allocation.lava_online_steps(s, total, w)
    assert all(np.array_equal(st["layer_budgets"], st["split"]) for st in steps)
    off = allocation.lava_allocate(s, total, w)
    last = steps[-1]
    assert np.array_equal(last["layer_budgets"], off["layer_budgets"])
    for j in range(L):
        assert all(list(a) == list(b) for a, b in zip(last["sel"][j], off["sel"][j]))


def test_lava_online_first_step_keeps_at_most_the_layer():
    r = np.random.default_rng(73)
    L, hkv, p, w = 3, 2, 10, 1
    s = r.random((L, hkv, p))
    steps = allocation.lava_online_steps(s, L * w * hkv + 45, w)
    assert steps[0]["layer_budgets"][0] == hkv * p            # capped: the whole prefix of layer 0
    assert steps[1]["layer_budgets"].sum() <= (L * w * hkv + 45) - 2 * w * hkv   # B'(1)
    # closed form of the split: uniform scores have equal entropy, so the shares are equal
    u = np.ones((L, hkv, p))
    st = allocation.lava_online_steps(u, L * w * hkv + 12, w)
    assert list(st[-1]["layer_budgets"]) == [4, 4, 4]
    assert list(st[1]["layer_budgets"]) == [7, 7]             # (12 + 3*2 - 2*2) / 2 = 7 each


def test_largest_remainder_ties_go_to_lower_index():
    """Equal fractional parts: the extra units go to the lower indices first
    (the tie order of the LAVa layer split); larger parts before smaller."""
    np.testing.assert_array_equal(allocation.largest_remainder(np.array([1.5, 2.5, 0.5]), 5), [2, 3, 0])
    np.testing.assert_array_equal(allocation.largest_remainder(np.array([0.5, 0.5, 0.5, 0.5]), 2), [1, 1, 0, 0])
    np.testing.assert_array_equal(allocation.largest_remainder(np.array([0.2, 0.7, 0.7, 1.4]), 3), [0, 1, 1, 1])
    # exact integers take no extra unit
    np.testing.assert_array_equal(allocation.largest_remainder(np.array([2.0, 1.0, 0.0]), 3), [2, 1, 0])
