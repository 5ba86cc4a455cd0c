"""Pins for the oracle's compaction, decode and the pages' bounds (CPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import allocation, bounds, cache, scoring


def sdpa_gqa(q, k, v):
    """Reference decode: torch SDPA over the full cache with each KV head
    repeated for its query heads."""
    hq, d = q.shape
    G = hq // k.shape[0]
    kk = torch.from_numpy(np.repeat(k, G, axis=0))[None]
    vv = torch.from_numpy(np.repeat(v, G, axis=0))[None]
    qq = torch.from_numpy(q)[None, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, :, 0].numpy()


def make(seed, hq=4, hkv=2, d=8, n=30, w=3):
    r = np.random.default_rng(seed)
    return (r.standard_normal((hq, w, d)) * 2, r.standard_normal((hkv, n, d)),
            r.standard_normal((hkv, n, d)), r.standard_normal((hq, d)) * 2)


def test_compact_is_exact_gather_then_window():
    qw, k, v, q = make(20)
    sel = [np.array([0, 5, 9]), np.array([2])]
    kh = cache.compact(k, sel, 3)
    np.testing.assert_array_equal(kh[0], np.concatenate([k[0, [0, 5, 9]], k[0, 27:]]))
    np.testing.assert_array_equal(kh[1], np.concatenate([k[1, [2]], k[1, 27:]]))
    start, ln = cache.flat_layout([3, 1], 3, 2)
    assert list(start) == [0, 8, 14] and list(ln) == [6, 4]


def test_keep_everything_equals_full_attention():
    qw, k, v, q = make(21)
    hkv, n, d = k.shape
    w = qw.shape[1]
    s = scoring.snapkv_scores(qw, k, 7)
    out = allocation.ada_allocate(s, hkv * n, w, (1, 5))
    kh, vh = cache.compact(k, out["sel"], w), cache.compact(v, out["sel"], w)
    np.testing.assert_allclose(cache.decode(q, kh, vh), sdpa_gqa(q, k, v), rtol=1e-12, atol=1e-13)


def test_append_then_attend():
    qw, k, v, q = make(22)
    r = np.random.default_rng(23)
    kn, vn = r.standard_normal((2, 8)), r.standard_normal((2, 8))
    kh, vh = cache.append(list(k), list(v), kn, vn)
    ref = sdpa_gqa(q, np.concatenate([k, kn[:, None]], axis=1), np.concatenate([v, vn[:, None]], axis=1))
    np.testing.assert_allclose(cache.decode(q, kh, vh), ref, rtol=1e-12, atol=1e-13)


def test_decode_of_subset_equals_masked_attention():
    qw, k, v, q = make(24)
    w = qw.shape[1]
    s = scoring.snapkv_scores(qw, k, 3)
    out = allocation.ada_allocate(s, 20, w, (1, 5))
    kh, vh = cache.compact(k, out["sel"], w), cache.compact(v, out["sel"], w)
    keep = np.zeros(k.shape[:2], dtype=bool)
    for g in range(2):
        keep[g, out["sel"][g]] = True
        keep[g, -w:] = True
    Ah = bounds.masked_attention(q, k, keep)
    ref = np.stack([Ah[i] @ v[i // 2] for i in range(4)])
    np.testing.assert_allclose(cache.decode(q, kh, vh), ref, rtol=1e-12, atol=1e-13)
    assert bounds.renormalisation_gap(q, k, keep) < 1e-14


def _masks(seed, hkv, n, w, produced):
    r = np.random.default_rng(seed)
    yield produced
    for _ in range(200):
        m = r.random((hkv, n)) < r.random()
        for g in range(hkv):
            if not m[g].any():
                m[g, r.integers(0, n)] = True
        yield m


def test_bounds_hold_on_produced_and_random_masks():
    r = np.random.default_rng(25)
    hq, hkv, d, n, w, D = 4, 2, 8, 24, 2, 10
    qw = r.standard_normal((hq, w, d)) * 2
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    q = r.standard_normal((hq, d)) * 2
    w_o = r.standard_normal((hq * d, D)) / math.sqrt(D)
    s = scoring.snapkv_scores(qw, k, 3)
    out = allocation.ada_allocate(s, 20, w, (1, 5))
    produced = np.zeros((hkv, n), dtype=bool)
    for g in range(hkv):
        produced[g, out["sel"][g]] = True
        produced[g, n - w:] = True
    for m in _masks(26, hkv, n, w, produced):
        loss, eps = bounds.adakv_theorem31(q, k, v, w_o, m)
        assert loss <= eps * (1 + 1e-12) + 1e-12
        loss2, b2 = bounds.lava_theorem1(q, k, v, w_o, m)
        assert loss2 <= b2 * (1 + 1e-12) + 1e-12
        for l3, th in bounds.criticalkv_theta(q, k, v, w_o, m):
            assert l3 <= th * (1 + 1e-12) + 1e-12
    full = np.ones((hkv, n), dtype=bool)
    loss, eps = bounds.adakv_theorem31(q, k, v, w_o, full)
    assert loss < 1e-12 and abs(eps) < 1e-9


def _two_entry_case(a, c):
    """One head, d = 1, two cached entries with attention (a, 1 - a); the rows
    of V W^O are +c e_1 and -c e_1; entry 0 kept.  The exact loss is
    |c - (2a - 1) c| = 2 c (1 - a)."""
    z1 = math.log((1 - a) / a)            # softmax([0, z1]) = (a, 1 - a)
    q = np.array([[1.0]])
    k = np.array([[[0.0], [z1]]])         # d = 1: logits are q.k exactly
    v = np.array([[[1.0], [-1.0]]])
    w_o = np.array([[c, 0.0, 0.0]])
    keep = np.array([[True, False]])
    return q, k, v, w_o, keep


@pytest.mark.parametrize("a", [0.9, 0.6, 0.25])
def test_bounds_are_attained(a):
    """The three bounds are tight: on the two-entry case each equals the loss
    2 c (1 - a) (Ada-KV notes, Theorem 3.1 with h = 1 and C = c; LAVa notes,
    Theorem 1 with C_hat = c and V_bar = 1; CriticalKV notes, theta with
    sum N A = a), so a looser constant or a dropped term cannot pass."""
    c = 1.7
    q, k, v, w_o, keep = _two_entry_case(a, c)
    want = 2 * c * (1 - a)
    loss, eps = bounds.adakv_theorem31(q, k, v, w_o, keep)
    assert loss == pytest.approx(want, rel=1e-12) and eps == pytest.approx(want, rel=1e-12)
    loss2, b2 = bounds.lava_theorem1(q, k, v, w_o, keep)
    assert loss2 == pytest.approx(want, rel=1e-12) and b2 == pytest.approx(want, rel=1e-12)
    (l3, th), = bounds.criticalkv_theta(q, k, v, w_o, keep)
    assert l3 == pytest.approx(want, rel=1e-12) and th == pytest.approx(want, rel=1e-12)


def test_bound_pins_catch_planted_constants():
    """A bound with its constant doubled, or the kept mass counted twice, is
    no longer attained (or no longer a bound) on the two-entry case."""
    a, c = 0.6, 1.7
    q, k, v, w_o, keep = _two_entry_case(a, c)
    loss, eps = bounds.adakv_theorem31(q, k, v, w_o, keep)
    hq = 1
    looser = 2 * hq * (2 * c) - 2 * (2 * c) * a          # C doubled
    dropped = 2 * hq * c - 4 * c * a                      # kept mass counted twice
    assert looser != pytest.approx(loss, rel=1e-6)
    assert not loss <= dropped * (1 + 1e-12)
