"""Pins for the oracle's scoring (CPU).  Each check compares the oracle with
something other than itself: a library routine (SciPy's 1-D maximum filter,
PyTorch's scaled-dot-product attention used as the definition of softmax
attention), a closed form, or an invariant the mathematics fixes."""
import math

import numpy as np
import pytest
import scipy.ndimage
import torch

from oracle import scoring


def rng(seed):
    return np.random.default_rng(seed)


def sdpa_weights(q, k, mask=None):
    """Attention weights from torch's SDPA: value = identity returns the weights."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None]          # [1,1,r,d]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None, None]          # [1,1,n,d]
    eye = torch.eye(k.shape[0], dtype=torch.float64)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, eye, attn_mask=m)[0, 0].numpy()


# ---------------------------------------------------------------- max pooling
@pytest.mark.parametrize("kernel", [1, 3, 5, 7, 9])
@pytest.mark.parametrize("length", [1, 2, 3, 7, 50])
def test_maxpool_matches_scipy(kernel, length):
    x = rng(kernel * 100 + length).random((3, length))
    ref = scipy.ndimage.maximum_filter1d(x, size=kernel, axis=-1, mode="nearest")
    np.testing.assert_array_equal(scoring.maxpool_same(x, kernel), ref)


def test_maxpool_rejects_even_kernel():
    with pytest.raises(ValueError):
        scoring.maxpool_same(np.zeros(4), 4)


# ---------------------------------------------------------------- Ada-KV / SnapKV
def check_single_row_is_softmax_attention(fn) -> bool:
    """w = 1, pool = 1, G = 1: the score is one row of scaled softmax attention."""
    r = rng(1)
    d, n = 16, 40
    q = r.standard_normal((1, 1, d)) * 2.0
    k = r.standard_normal((1, n, d))
    got = fn(q, k, 1)[0]
    ref = sdpa_weights(q[0], k[0, :n - 1])[0]
    return np.allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_single_row_is_softmax_attention():
    assert check_single_row_is_softmax_attention(scoring.snapkv_head_scores)


def test_window_mean_and_group_mean():
    r = rng(2)
    hq, hkv, w, d, n = 4, 2, 3, 8, 30
    q = r.standard_normal((hq, w, d))
    k = r.standard_normal((hkv, n, d))
    p = n - w
    heads = scoring.snapkv_head_scores(q, k, 1)
    for i in range(hq):
        ref = sdpa_weights(q[i], k[i // 2, :p]).mean(axis=0)
        np.testing.assert_allclose(heads[i], ref, rtol=1e-12, atol=1e-15)
    grp = scoring.snapkv_scores(q, k, 1)
    np.testing.assert_allclose(grp[1], 0.5 * (heads[2] + heads[3]), rtol=1e-14)


def check_pool_each_row_then_mean(fn) -> bool:
    """Algorithm 2 step 4 pools every window row, then averages the rows."""
    r = rng(3)
    w, d, n, pool = 4, 8, 24, 5
    q = r.standard_normal((1, w, d)) * 3
    k = r.standard_normal((1, n, d))
    P = sdpa_weights(q[0], k[0, :n - w])
    ref = scipy.ndimage.maximum_filter1d(P, size=pool, axis=-1, mode="nearest").mean(axis=0)
    return np.allclose(fn(q, k, pool)[0], ref, rtol=1e-12, atol=1e-15)


def test_pool_each_row_then_mean():
    assert check_pool_each_row_then_mean(scoring.snapkv_head_scores)


def test_constant_keys_give_uniform_scores():
    r = rng(4)
    hq, hkv, w, d, n = 4, 2, 5, 8, 37
    q = r.standard_normal((hq, w, d))
    k = np.broadcast_to(r.standard_normal(d), (hkv, n, d)).copy()
    for pool in (1, 3, 7):
        s = scoring.snapkv_scores(q, k, pool)
        np.testing.assert_allclose(s, 1.0 / (n - w), rtol=1e-13)


def test_mass_conservation_without_pooling():
    r = rng(5)
    q = r.standard_normal((6, 4, 8)) * 4
    k = r.standard_normal((3, 50, 8))
    s = scoring.snapkv_scores(q, k, 1)
    np.testing.assert_allclose(s.sum(axis=1), 1.0, rtol=1e-13)


def test_pooling_only_raises_scores():
    r = rng(6)
    q = r.standard_normal((4, 4, 8)) * 3
    k = r.standard_normal((2, 40, 8))
    base = scoring.snapkv_scores(q, k, 1)
    for pool in (3, 7):
        assert np.all(scoring.snapkv_scores(q, k, pool) >= base)


# ---------------------------------------------------------------- LAVa
def test_lava_causal_rows_and_vbar():
    r = rng(7)
    hq, hkv, w, d, n = 2, 2, 4, 8, 21
    q = r.standard_normal((hq, w, d)) * 2
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    p = n - w
    allowed = np.arange(n)[None, :] <= (p + np.arange(w))[:, None]
    s_pre, vbar, s_full, pooled_full = scoring.lava_scores(q, k, v, 1, full=True)
    for g in range(hkv):
        vb = max(sum(abs(v[g, t, e]) for e in range(d)) for t in range(n))
        assert math.isclose(vbar[g], vb, rel_tol=1e-13)
        S = sdpa_weights(q[g], k[g], mask=allowed).sum(axis=0)
        np.testing.assert_allclose(s_full[g], vb / w * S, rtol=1e-12, atol=1e-15)
        # each window row sums to one, so the unpooled vector sums to V-bar
        assert math.isclose(s_full[g].sum(), vb, rel_tol=1e-12)
    np.testing.assert_array_equal(s_pre, s_full[:, :p])


def test_lava_group_max_and_pool_order():
    r = rng(8)
    hq, hkv, w, d, n, pool = 4, 2, 3, 8, 26, 7
    q = r.standard_normal((hq, w, d)) * 2
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    p = n - w
    s_pre, vbar, s_full, pooled_full = scoring.lava_scores(q, k, v, pool, full=True)
    single = [scoring.lava_scores(q[i:i + 1], k[i // 2:i // 2 + 1], v[i // 2:i // 2 + 1], 1, full=True)[2][0]
              for i in range(hq)]
    for g in range(hkv):
        np.testing.assert_allclose(s_full[g], np.maximum(single[2 * g], single[2 * g + 1]), rtol=1e-14)
    ref = scipy.ndimage.maximum_filter1d(s_full, size=pool, axis=-1, mode="nearest")
    np.testing.assert_array_equal(pooled_full, ref)
    np.testing.assert_array_equal(s_pre, ref[:, :p])


# ---------------------------------------------------------------- CriticalKV
def test_projected_norm_identity_projection():
    """W^O made of identity blocks (D = d): ||V W^O_i||_1 = ||V||_1 row-wise."""
    r = rng(9)
    hq, hkv, d, n = 4, 2, 8, 12
    v = r.standard_normal((hkv, n, d))
    w_o = np.concatenate([np.eye(d)] * hq, axis=0)                       # [hq*d, d]
    nrm = scoring.projected_value_norms(v, w_o, hq)
    for i in range(hq):
        np.testing.assert_allclose(nrm[i], np.abs(v[i // 2]).sum(axis=1), rtol=1e-14)
    # a signed permutation and a scale change nothing but the scale
    perm = np.eye(d)[r.permutation(d)] * np.where(r.random(d) < 0.5, -1.0, 1.0)
    w2 = np.concatenate([3.0 * perm] * hq, axis=0)
    np.testing.assert_allclose(scoring.projected_value_norms(v, w2, hq), 3.0 * nrm, rtol=1e-13)


def test_criticalkv_group_rule_and_epsilon():
    r = rng(10)
    hq, hkv, w, d, n, D = 4, 2, 3, 8, 20, 12
    q = r.standard_normal((hq, w, d))
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    w_o = r.standard_normal((hq * d, D))
    score, comp, a, nrm = scoring.criticalkv_scores(q, k, v, w_o, 3, 1e-6)
    np.testing.assert_allclose(score, scoring.snapkv_scores(q, k, 3), rtol=1e-14)
    for g in range(hkv):
        parts = []
        for i in (2 * g, 2 * g + 1):
            _, c1, _, _ = scoring.criticalkv_scores(q[i:i + 1], k[g:g + 1], v[g:g + 1],
                                                    w_o[i * d:(i + 1) * d], 3, 1e-6)
            parts.append(c1[0])
        np.testing.assert_allclose(comp[g], 0.5 * (parts[0] + parts[1]), rtol=1e-13)
    assert np.all(comp > 0)


# ---------------------------------------------------------------- planted mistakes
def _no_sqrt_d(q_win, k, pool):
    return scoring.snapkv_head_scores(q_win * math.sqrt(q_win.shape[-1]), k, pool)


def _mean_then_pool(q_win, k, pool):
    p = k.shape[1] - q_win.shape[1]
    out = []
    for i in range(q_win.shape[0]):
        z = q_win[i] @ k[0, :p].T / math.sqrt(q_win.shape[-1])
        out.append(scoring.maxpool_same(scoring.softmax_rows(z).mean(axis=0), pool))
    return np.asarray(out)


def test_pins_catch_planted_mistakes():
    assert not check_single_row_is_softmax_attention(_no_sqrt_d)
    assert not check_pool_each_row_then_mean(_mean_then_pool)


# ---------------------------------------------------------------- supplied normaliser
def test_window_lse_matches_scipy_logsumexp():
    """The row statistic is SciPy's logsumexp of the scaled logits over the
    row's domain: the prefix keys, or keys 0 .. p + r causally."""
    import scipy.special
    r = rng(31)
    hq, hkv, w, d, n = 4, 2, 3, 8, 25
    q = r.standard_normal((hq, w, d)) * 3.0
    k = r.standard_normal((hkv, n, d))
    p = n - w
    pre = scoring.window_lse(q, k, causal=False)
    cau = scoring.window_lse(q, k, causal=True)
    for i in range(hq):
        z = q[i] @ k[i // 2].T / math.sqrt(d)
        np.testing.assert_allclose(pre[i], scipy.special.logsumexp(z[:, :p], axis=1), rtol=1e-14)
        for row in range(w):
            np.testing.assert_allclose(cau[i, row], scipy.special.logsumexp(z[row, :p + row + 1]), rtol=1e-14)


def test_scores_from_supplied_normaliser():
    """With the exact normaliser supplied the scores are the two-pass scores;
    every row's normaliser raised by delta scales the Ada-KV score by
    exp(-delta) (max pooling and the means are positively homogeneous) and
    the LAVa score likewise."""
    r = rng(32)
    hq, hkv, w, d, n = 4, 2, 4, 16, 40
    q = r.standard_normal((hq, w, d)) * 2.0
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    a = scoring.snapkv_scores(q, k, 3)
    lse = scoring.window_lse(q, k, causal=False)
    np.testing.assert_allclose(scoring.snapkv_scores(q, k, 3, lse), a, rtol=1e-12)
    np.testing.assert_allclose(scoring.snapkv_scores(q, k, 3, lse + 0.7), a * math.exp(-0.7), rtol=1e-12)
    s, _ = scoring.lava_scores(q, k, v, 5)
    lc = scoring.window_lse(q, k, causal=True)
    np.testing.assert_allclose(scoring.lava_scores(q, k, v, 5, lse=lc)[0], s, rtol=1e-12)
    np.testing.assert_allclose(scoring.lava_scores(q, k, v, 5, lse=lc - 0.3)[0], s * math.exp(0.3), rtol=1e-12)
    # the Ada-KV domain excludes the window keys: the causal statistic is not it
    assert not np.allclose(scoring.snapkv_scores(q, k, 3, lc), a, rtol=1e-6)


def check_causal_correction(fn) -> bool:
    """From the exact causal statistic the correction gives each scorer's own
    domain statistic, as window_lse defines it (pinned to SciPy above): the
    prefix for Ada-KV and CriticalKV, all n keys for LaProx, the causal one
    unchanged for LAVa; the prefix share is exp(lse_prefix - lse_causal)."""
    r = rng(33)
    hq, hkv, w, d, n = 6, 3, 5, 8, 30
    q = r.standard_normal((hq, w, d)) * 2.0
    k = r.standard_normal((hkv, n, d))
    lc = scoring.window_lse(q, k, causal=True)
    ok = True
    for scorer, want in (("snapkv", scoring.window_lse(q, k, causal=False)),
                         ("criticalkv", scoring.window_lse(q, k, causal=False)),
                         ("laprox", scoring.window_lse(q, k, causal=False, full=True)),
                         ("lava", lc)):
        got, keep = fn(lc, q, k, scorer)
        ok &= bool(np.allclose(got, want, rtol=0, atol=1e-12))
        if scorer in ("snapkv", "criticalkv"):
            ok &= bool(np.allclose(keep, np.exp(want - lc), rtol=1e-12))
    return ok


def _corr_window_off_by_one(lse_c, q, k, scorer):
    """Planted mistake: the window range stops one key early (p .. p + r - 1)."""
    hq, w, d = q.shape
    hkv, n, _ = k.shape
    p, G = n - w, hq // hkv
    lse = np.array(lse_c, dtype=np.float64, copy=True)
    if scorer in ("snapkv", "criticalkv"):
        for i in range(hq):
            for row in range(w):
                s = sum(math.exp(float(q[i, row] @ k[i // G, t]) / math.sqrt(d) - lse_c[i, row])
                        for t in range(p, p + row))
                lse[i, row] = lse_c[i, row] + math.log(1.0 - s)
        return lse, np.ones((hq, w))
    return scoring.lse_from_causal(lse_c, q, k, scorer)


def _corr_sign(lse_c, q, k, scorer):
    """Planted mistake: the window mass added instead of removed."""
    hq, w, d = q.shape
    hkv, n, _ = k.shape
    p, G = n - w, hq // hkv
    lse = np.array(lse_c, dtype=np.float64, copy=True)
    if scorer in ("snapkv", "criticalkv"):
        for i in range(hq):
            for row in range(w):
                s = sum(math.exp(float(q[i, row] @ k[i // G, t]) / math.sqrt(d) - lse_c[i, row])
                        for t in range(p, p + row + 1))
                lse[i, row] = lse_c[i, row] + math.log1p(s)
        return lse, np.ones((hq, w))
    return scoring.lse_from_causal(lse_c, q, k, scorer)


def _corr_laprox_includes_own(lse_c, q, k, scorer):
    """Planted mistake: LaProx adds the row's own key p + r a second time."""
    hq, w, d = q.shape
    hkv, n, _ = k.shape
    p, G = n - w, hq // hkv
    if scorer != "laprox":
        return scoring.lse_from_causal(lse_c, q, k, scorer)
    lse = np.array(lse_c, dtype=np.float64, copy=True)
    for i in range(hq):
        for row in range(w):
            s = sum(math.exp(float(q[i, row] @ k[i // G, t]) / math.sqrt(d) - lse_c[i, row])
                    for t in range(p + row, n))
            lse[i, row] = lse_c[i, row] + math.log1p(s)
    return lse, np.ones((hq, w))


def test_causal_correction_gives_each_domain():
    assert check_causal_correction(scoring.lse_from_causal)


def test_causal_correction_pins_catch_planted_mistakes():
    assert not check_causal_correction(_corr_window_off_by_one)
    assert not check_causal_correction(_corr_sign)
    assert not check_causal_correction(_corr_laprox_includes_own)


def test_causal_correction_scores():
    """Scores from the corrected causal statistic are the two-pass scores."""
    r = rng(34)
    hq, hkv, w, d, n = 4, 2, 4, 16, 40
    q = r.standard_normal((hq, w, d)) * 2.0
    k = r.standard_normal((hkv, n, d))
    lc = scoring.window_lse(q, k, causal=True)
    lse, keep = scoring.lse_from_causal(lc, q, k, "snapkv")
    np.testing.assert_allclose(scoring.snapkv_scores(q, k, 3, lse), scoring.snapkv_scores(q, k, 3), rtol=1e-11)
    assert (keep > 0).all() and (keep < 1).all()


# ---------------------------------------------------------------- LaProx
def check_laprox_is_frobenius_norm(fn) -> bool:
    """G = 1: p_i[t] is the Frobenius norm of the explicit w x D matrix
    A_i[:, t] (V W^O_i)[t, :], with A from torch's scaled-dot-product attention
    over all n keys (no mask) and the product formed entry by entry."""
    r = rng(41)
    hq, hkv, w, d, n, D = 3, 3, 4, 8, 19, 6
    q = r.standard_normal((hq, w, d)) * 1.5
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    w_o = r.standard_normal((hq * d, D))
    got = fn(q, k, v, w_o)
    p = n - w
    for i in range(hq):
        A = sdpa_weights(q[i], k[i])                                     # [w, n]
        for t in range(p):
            h = [sum(v[i, t, e] * w_o[i * d + e, c] for e in range(d)) for c in range(D)]
            M = np.array([[A[row, t] * h[c] for c in range(D)] for row in range(w)])
            if not np.isclose(got[i, t], np.linalg.norm(M, "fro"), rtol=1e-12, atol=0.0):
                return False
    return True


def test_laprox_is_frobenius_norm_of_token_contribution():
    assert check_laprox_is_frobenius_norm(scoring.laprox_head_scores)


def check_laprox_uniform_closed_form(fn) -> bool:
    """Constant keys: every weight is 1/n, so ||A_i[:, t]||_2 = sqrt(w)/n; with
    W^O_i = c_i * I (D = d) the value factor is c_i ||V_g[t]||_2, and the group
    takes the mean over its heads."""
    r = rng(42)
    hq, hkv, w, d, n = 4, 2, 5, 8, 30
    q = r.standard_normal((hq, w, d))
    k = np.broadcast_to(r.standard_normal((hkv, 1, d)), (hkv, n, d)).copy()
    v = r.standard_normal((hkv, n, d))
    c = np.array([0.5, 2.0, 3.0, 7.0])
    w_o = np.concatenate([c[i] * np.eye(d) for i in range(hq)], axis=0)
    got = fn(q, k, v, w_o)
    p = n - w
    ref = np.stack([math.sqrt(w) / n * np.linalg.norm(v[g, :p], axis=1) * c[2 * g:2 * g + 2].mean()
                    for g in range(hkv)])
    return bool(np.allclose(got, ref, rtol=1e-13, atol=0.0))


def test_laprox_uniform_attention_closed_form():
    assert check_laprox_uniform_closed_form(scoring.laprox_scores)


def test_laprox_group_mean_and_key_subset():
    r = rng(43)
    hq, hkv, w, d, n, D = 4, 2, 3, 8, 26, 10
    q = r.standard_normal((hq, w, d)) * 2.0
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    w_o = r.standard_normal((hq * d, D))
    s = scoring.laprox_scores(q, k, v, w_o)
    for g in range(hkv):
        parts = [scoring.laprox_head_scores(q[i:i + 1], k[g:g + 1], v[g:g + 1], w_o[i * d:(i + 1) * d])[0]
                 for i in (2 * g, 2 * g + 1)]
        np.testing.assert_allclose(s[g], 0.5 * (parts[0] + parts[1]), rtol=1e-13)
    keys = np.array([0, 5, 22])
    np.testing.assert_allclose(scoring.laprox_scores(q, k, v, w_o, keys=keys), s[:, keys], rtol=1e-13)
    # the supplied normaliser over all keys reproduces the two-pass score; the
    # prefix-only normaliser (the Ada-KV domain) does not
    lse = scoring.window_lse(q, k, causal=False, full=True)
    np.testing.assert_allclose(scoring.laprox_scores(q, k, v, w_o, lse), s, rtol=1e-12)
    assert not np.allclose(scoring.laprox_scores(q, k, v, w_o, scoring.window_lse(q, k, causal=False)), s,
                           rtol=1e-6)


def _laprox_causal(q_win, k, v, w_o):
    """Planted: causal window rows (the LAVa domain) instead of the printed softmax."""
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    p = n - w
    out = np.empty((hq, p))
    for i in range(hq):
        g = i // (hq // hkv)
        z = q_win[i] @ k[g].T / math.sqrt(d)
        z = np.where(np.arange(n)[None, :] > (p + np.arange(w))[:, None], -np.inf, z)
        a = np.sqrt((scoring.softmax_rows(z)[:, :p] ** 2).sum(axis=0))
        out[i] = a * scoring.projected_value_l2(v, w_o, hq)[i, :p]
    return out


def _laprox_l1_values(q_win, k, v, w_o):
    """Planted: the L1 value norm of CriticalKV in place of the L2 norm."""
    hkv = k.shape[0]
    a = scoring.laprox_attention_l2(q_win, k)
    nrm = scoring.projected_value_norms(v, w_o, q_win.shape[0], slice(0, a.shape[1]))
    return scoring.group_mean(a * nrm, hkv)


def test_laprox_pins_catch_planted_mistakes():
    assert not check_laprox_is_frobenius_norm(_laprox_causal)
    assert not check_laprox_uniform_closed_form(_laprox_l1_values)


# ---------------------------------------------------------------- CriticalKV composite, entry by entry
def _loop_composite(q, k, v, w_o, pool, eps):
    """The CriticalKV composite written out with explicit loops, sharing nothing
    with the oracle's scorer: for query head i of KV head g and prefix token t,
    A_i[t] = mean over window rows of the max pooled softmax weight (math.exp,
    the pooling window cut at the prefix ends), nrm_i[t] = sum over output
    features c of |sum over e of V[g,t,e] W^O[i*d+e, c]|, and the KV head takes
    the mean over its query heads of (A_i[t] + eps) * nrm_i[t]
    (CriticalKV notes, "两阶段贪心选择算法"; GQA by the group mean)."""
    hq, w, d = q.shape
    hkv, n, _ = k.shape
    D = w_o.shape[1]
    G = hq // hkv
    p = n - w
    rho = (pool - 1) // 2
    out = [[0.0] * p for _ in range(hkv)]
    for i in range(hq):
        g = i // G
        wts = []
        for r in range(w):
            z = [sum(q[i, r, e] * k[g, t, e] for e in range(d)) / math.sqrt(d) for t in range(p)]
            m = max(z)
            ex = [math.exp(x - m) for x in z]
            s = sum(ex)
            wts.append([x / s for x in ex])
        for t in range(p):
            a = 0.0
            for r in range(w):
                a += max(wts[r][u] for u in range(max(0, t - rho), min(p, t + rho + 1)))
            a /= w
            nrm = 0.0
            for c in range(D):
                nrm += abs(sum(v[g, t, e] * w_o[i * d + e, c] for e in range(d)))
            out[g][t] += (a + eps) * nrm / G
    return np.array(out)


def check_criticalkv_composite(fn) -> bool:
    """fn(q, k, v, w_o, pool, eps) -> composite [Hkv, p] must equal the loop
    form on a tiny GQA case (G = 2, pool 3, D != d so a transposed W^O shows),
    at a small and at a large epsilon."""
    r = rng(51)
    hq, hkv, w, d, n, D = 4, 2, 3, 4, 13, 6
    q = r.standard_normal((hq, w, d)) * 1.5
    k = r.standard_normal((hkv, n, d))
    v = r.standard_normal((hkv, n, d))
    w_o = r.standard_normal((hq * d, D))
    for eps in (1e-6, 0.25):
        ref = _loop_composite(q, k, v, w_o, 3, eps)
        if not np.allclose(fn(q, k, v, w_o, 3, eps), ref, rtol=1e-12, atol=0.0):
            return False
    return True


def _oracle_composite(q, k, v, w_o, pool, eps):
    return scoring.criticalkv_scores(q, k, v, w_o, pool, eps)[1]


def _ck_eps_outside(q, k, v, w_o, pool, eps):
    """Planted: A * nrm + eps instead of (A + eps) * nrm."""
    hkv = k.shape[0]
    a = scoring.snapkv_head_scores(q, k, pool)
    nrm = scoring.projected_value_norms(v, w_o, q.shape[0], slice(0, a.shape[1]))
    return scoring.group_mean(a * nrm + eps, hkv)


def _ck_unpooled_attention(q, k, v, w_o, pool, eps):
    """Planted: the attention factor without max pooling."""
    hkv = k.shape[0]
    a = scoring.snapkv_head_scores(q, k, 1)
    nrm = scoring.projected_value_norms(v, w_o, q.shape[0], slice(0, a.shape[1]))
    return scoring.group_mean((a + eps) * nrm, hkv)


def _ck_group_first(q, k, v, w_o, pool, eps):
    """Planted: (group-mean A + eps) * group-mean nrm (the alternative GQA rule)."""
    hkv = k.shape[0]
    a = scoring.snapkv_head_scores(q, k, pool)
    nrm = scoring.projected_value_norms(v, w_o, q.shape[0], slice(0, a.shape[1]))
    return (scoring.group_mean(a, hkv) + eps) * scoring.group_mean(nrm, hkv)


def _ck_group_block(q, k, v, w_o, pool, eps):
    """Planted: every head of a group projected with its group's first W^O block."""
    hq, w, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    a = scoring.snapkv_head_scores(q, k, pool)
    p = a.shape[1]
    nrm = np.stack([np.abs(v[i // G, :p] @ w_o[(i // G) * G * d:((i // G) * G + 1) * d]).sum(axis=1)
                    for i in range(hq)])
    return scoring.group_mean((a + eps) * nrm, hkv)


def test_criticalkv_composite_entry_by_entry():
    assert check_criticalkv_composite(_oracle_composite)


def check_criticalkv_closed_form(fn) -> bool:
    """Constant keys: every pooled weight is 1/p; with W^O_i = c_i * I (D = d)
    nrm_i = c_i ||V_g[t]||_1, so the KV head's composite is
    (1/p + eps) * mean_i(c_i) * ||V_g[t]||_1."""
    r = rng(52)
    hq, hkv, w, d, n = 4, 2, 3, 8, 21
    q = r.standard_normal((hq, w, d))
    k = np.broadcast_to(r.standard_normal((hkv, 1, d)), (hkv, n, d)).copy()
    v = r.standard_normal((hkv, n, d))
    c = np.array([0.5, 2.0, 3.0, 7.0])
    w_o = np.concatenate([c[i] * np.eye(d) for i in range(hq)], axis=0)
    p = n - w
    eps = 0.125
    ref = np.stack([(1.0 / p + eps) * c[2 * g:2 * g + 2].mean() * np.abs(v[g, :p]).sum(axis=1) for g in range(hkv)])
    return bool(np.allclose(fn(q, k, v, w_o, 5, eps), ref, rtol=1e-13, atol=0.0))


def test_criticalkv_composite_closed_form():
    assert check_criticalkv_closed_form(_oracle_composite)


def test_criticalkv_pins_catch_planted_mistakes():
    for planted in (_ck_eps_outside, _ck_unpooled_attention, _ck_group_first, _ck_group_block):
        assert not check_criticalkv_composite(planted), planted.__name__
    assert not check_criticalkv_closed_form(_ck_eps_outside)
