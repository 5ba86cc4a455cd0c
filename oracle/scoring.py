"""Observation-window scoring (oracle; float64; test infrastructure only).

Shapes: q_win [Hq, w, d], k and v [Hkv, n, d], GQA group G = Hq // Hkv,
query head i belongs to KV head g = i // G, prefix length p = n - w.
"""
from __future__ import annotations

import math

import numpy as np


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row-wise softmax; -inf entries get weight 0."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def maxpool_same(x: np.ndarray, kernel: int) -> np.ndarray:
    """1-D max pooling along the last axis: stride 1, output as long as the
    input, the window cut off at both ends (the same as padding with -inf).

    Ada-KV notes, Algorithm 2 ("Ada-KV Integration"), step 4 names
    maxpooling1d(kernel_size) without padding or stride; this is the plainest
    reading that keeps one score per cached token.
    """
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and >= 1")
    out = np.array(x, dtype=np.float64, copy=True)
    for s in range(1, (kernel - 1) // 2 + 1):
        if s >= x.shape[-1]:
            break
        out[..., s:] = np.maximum(out[..., s:], x[..., :-s])
        out[..., :-s] = np.maximum(out[..., :-s], x[..., s:])
    return out


def window_lse(q_win: np.ndarray, k: np.ndarray, causal: bool, full: bool = False) -> np.ndarray:
    """Log-sum-exp (natural log) of every window row's logits over the row's
    key domain, [Hq, w]: the normaliser of the window softmax.

    causal=False: the prefix keys t < p (the Ada-KV / CriticalKV domain,
    Ada-KV notes, Algorithm 2 step 2); causal=True: keys 0 .. p + r for window
    row r (the LAVa domain, LAVa notes, Definition 1); full=True: all n keys
    with no mask (the LaProx domain, see laprox_head_scores).  This is the
    per-row statistic an attention pass over those rows leaves behind; the
    scorers below accept it in place of computing the normaliser themselves.
    """
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    p = n - w
    out = np.empty((hq, w), dtype=np.float64)
    for i in range(hq):
        g = i // G
        if full:
            z = (q_win[i] @ k[g].T) / math.sqrt(d)
        elif causal:
            z = (q_win[i] @ k[g].T) / math.sqrt(d)
            z = np.where(np.arange(n)[None, :] > (p + np.arange(w))[:, None], -np.inf, z)
        else:
            z = (q_win[i] @ k[g, :p].T) / math.sqrt(d)
        m = z.max(axis=1, keepdims=True)
        out[i] = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def lse_from_causal(lse_causal: np.ndarray, q_win: np.ndarray, k: np.ndarray, scorer: str):
    """A scorer's row statistic from the causal one a prefill leaves behind.

    The prefill's causal attention (LAVa notes, "时间复杂度与内存使用分析": the
    O(H N^2 d_h) term, the window-score pass a separate O(H N w d_h) one) leaves
    for window row r, at position p + r, the log-sum-exp of its logits over
    keys 0 .. p + r: the LAVa domain as it is.  The Ada-KV / CriticalKV domain is the prefix t < p
    (Ada-KV notes, Algorithm 2 step 2), so the window keys p .. p + r come out:
        lse = lse_c + ln(1 - sum_{t=p}^{p+r} exp(z_t - lse_c));
    the LaProx domain is all n keys (LaProx page, Algorithm 1), so the later
    window keys p + r + 1 .. n - 1 go in:
        lse = lse_c + ln(1 + sum_{t>p+r} exp(z_t - lse_c)),
    with z_t = q_win[i, r] . k[g, t] / sqrt(d).  Returns (lse [Hq, w], keep
    [Hq, w]): keep is the prefix share 1 - sum(...) for the subtraction (1 for
    the other scorers): the relative error of the causal input grows by 1/keep
    in the result.
    """
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    p = n - w
    lse = np.array(lse_causal, dtype=np.float64, copy=True)
    keep = np.ones((hq, w), dtype=np.float64)
    if scorer == "lava":
        return lse, keep
    for i in range(hq):
        g = i // G
        for r in range(w):
            keys = slice(p + r + 1, n) if scorer == "laprox" else slice(p, p + r + 1)
            z = (k[g, keys] @ q_win[i, r]) / math.sqrt(d)
            s = float(np.exp(z - lse_causal[i, r]).sum())
            if scorer == "laprox":
                lse[i, r] = lse_causal[i, r] + math.log1p(s)
            else:
                keep[i, r] = 1.0 - s
                # no prefix mass left (rounding in a supplied lse_causal): -inf
                lse[i, r] = lse_causal[i, r] + math.log(keep[i, r]) if keep[i, r] > 0 else -math.inf
    return lse, keep


def snapkv_head_scores(q_win: np.ndarray, k: np.ndarray, pool: int, lse: np.ndarray | None = None) -> np.ndarray:
    """Per-query-head window score A-bar_i over the prefix keys, [Hq, p].

    Ada-KV notes, Algorithm 2, steps 2-4: softmax of Q_i^win K_i^T, where K_i is
    the cache outside the observation window, then max pooling of every window
    row, then the mean over the window rows.  Logits are divided by sqrt(d_h):
    the Ada-KV paper (arXiv HTML, Section 3.1, footnote 5) drops the factor only
    to simplify notation, and the LAVa and CriticalKV pages keep it.
    With `lse` [Hq, w] given, the softmax normaliser of row r is exp(lse[i, r])
    (weights exp(z - lse)) instead of being summed here.
    """
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    p = n - w
    out = np.empty((hq, p), dtype=np.float64)
    for i in range(hq):
        g = i // G
        z = (q_win[i] @ k[g, :p].T) / math.sqrt(d)
        P = softmax_rows(z) if lse is None else np.exp(z - np.asarray(lse, dtype=np.float64)[i][:, None])
        out[i] = maxpool_same(P, pool).mean(axis=0)
    return out


def group_mean(a_heads: np.ndarray, hkv: int) -> np.ndarray:
    """GQA reduction of Ada-KV: the mean over the query heads of each group.

    Ada-KV notes, "自适应分配下的计算效率实现" item 2; Ada-KV paper,
    "Compatibility with Group Query Attention".
    """
    hq, p = a_heads.shape
    return a_heads.reshape(hkv, hq // hkv, p).mean(axis=1)


def snapkv_scores(q_win: np.ndarray, k: np.ndarray, pool: int, lse: np.ndarray | None = None) -> np.ndarray:
    """Ada-KV / SnapKV score per KV head, [Hkv, p]."""
    return group_mean(snapkv_head_scores(q_win, k, pool, lse), k.shape[0])


def lava_scores(q_win: np.ndarray, k: np.ndarray, v: np.ndarray, pool: int,
                full: bool = False, lse: np.ndarray | None = None):
    """LAVa score per KV head and the per-head value-norm maximum.

    LAVa notes, Definition 1: s[i] = (max_k ||V[k]||_1 / w) * sum over the w
    recent queries of their attention to token i.  Those queries are decode
    steps, so window row r (absolute position p + r) attends causally to keys
    0 .. p + r.  "适配GQA架构": a group's score is the maximum over its query
    heads.  "实验环境": every score vector is max pooled (kernel 7); the vector
    is pooled over all n tokens and then cut to the evictable prefix, since
    eviction only touches tokens outside the recent window ("动态头预算的逐层缓存驱逐").

    Returns (scores [Hkv, p], vbar [Hkv]); with full=True the unpooled and
    pooled vectors over all n tokens are returned as well.  With `lse` [Hq, w]
    given, row r's weights are exp(z - lse[i, r]) over its causal keys.
    """
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    p = n - w
    causal = np.arange(n)[None, :] > (p + np.arange(w))[:, None]     # [w, n]
    S = np.empty((hq, n), dtype=np.float64)
    for i in range(hq):
        g = i // G
        z = (q_win[i] @ k[g].T) / math.sqrt(d)
        z = np.where(causal, -np.inf, z)
        if lse is None:
            S[i] = softmax_rows(z).sum(axis=0)
        else:
            S[i] = np.exp(z - np.asarray(lse, dtype=np.float64)[i][:, None]).sum(axis=0)
    vbar = np.abs(v).sum(axis=2).max(axis=1)                          # [Hkv]
    s = (vbar[:, None] / w) * S.reshape(hkv, G, n).max(axis=1)
    pooled = maxpool_same(s, pool)
    if full:
        return pooled[:, :p], vbar, s, pooled
    return pooled[:, :p], vbar


def projected_value_norms(v: np.ndarray, w_o: np.ndarray, hq: int, rows: slice | None = None) -> np.ndarray:
    """||(V W^O_i)[k, :]||_1 for every query head i and prefix key k, [Hq, p].

    CriticalKV notes, "损失函数 / 训练策略": the only new runtime quantity is
    the L1 norm of each row of V W^O.  Here W^O_i is the d-row block i of the
    [Hq*d, D] output projection (o = A V W^O with W^O of the pages' shape).
    `rows` picks a subset of keys; the product is formed in row chunks, which
    changes no arithmetic of any output element.
    """
    hkv, n, d = v.shape
    G = hq // hkv
    keys = np.arange(n)[rows] if rows is not None else np.arange(n)
    out = np.empty((hq, keys.size), dtype=np.float64)
    for i in range(hq):
        g = i // G
        wi = w_o[i * d:(i + 1) * d]
        for s in range(0, keys.size, 2048):
            kk = keys[s:s + 2048]
            out[i, s:s + 2048] = np.abs(v[g, kk] @ wi).sum(axis=1)
    return out


def criticalkv_scores(q_win: np.ndarray, k: np.ndarray, v: np.ndarray, w_o: np.ndarray,
                      pool: int, eps: float, lse: np.ndarray | None = None):
    """Ada-KV score (for the budgets) and the CriticalKV composite per KV head.

    CriticalKV notes, "两阶段贪心选择算法": composite (A_i + eps) * ||V W^O||_1
    of each entry; "作为通用插件融入现有驱逐流水线": window, max pooling and the
    cross-head allocation stay as in Ada-KV.  Under GQA the composite of a KV
    head is the mean over its query heads of (A-bar_i + eps) * nrm_i, the same
    additive group rule Ada-KV uses for attention.
    Returns (score [Hkv, p], composite [Hkv, p], a_heads [Hq, p], nrm [Hq, p]).
    """
    hq = q_win.shape[0]
    hkv, n, _ = k.shape
    p = n - q_win.shape[1]
    a = snapkv_head_scores(q_win, k, pool, lse)
    nrm = projected_value_norms(v, w_o, hq, slice(0, p))
    comp = ((a + eps) * nrm).reshape(hkv, hq // hkv, p).mean(axis=1)
    return group_mean(a, hkv), comp, a, nrm


def projected_value_l2(v: np.ndarray, w_o: np.ndarray, hq: int, rows: slice | np.ndarray | None = None) -> np.ndarray:
    """||(V W^O_i)[k, :]||_2 for every query head i and the chosen keys, [Hq, keys].

    LaProx page, Section 4.1, Algorithm 1: H = V W_O and the factor
    ||H[i, :]||_2 of token i.  W^O_i is the d-row block i of the [Hq*d, D]
    output projection, as in projected_value_norms; the product is formed in
    row chunks, which changes no arithmetic of any output element.
    """
    hkv, n, d = v.shape
    G = hq // hkv
    keys = np.arange(n)[rows] if rows is not None else np.arange(n)
    out = np.empty((hq, keys.size), dtype=np.float64)
    for i in range(hq):
        g = i // G
        wi = w_o[i * d:(i + 1) * d]
        for s in range(0, keys.size, 2048):
            kk = keys[s:s + 2048]
            h = v[g, kk] @ wi
            out[i, s:s + 2048] = np.sqrt((h * h).sum(axis=1))
    return out


def laprox_attention_l2(q_win: np.ndarray, k: np.ndarray, lse: np.ndarray | None = None) -> np.ndarray:
    """||A_i[:, t]||_2 over the w window rows for every query head i and prefix
    token t, [Hq, p].

    LaProx page, Section 4.1, Algorithm 1: A = Softmax(Q[-w:, ] K^T / sqrt(d_k))
    over the cached keys, as printed: every window row over all n keys, no
    mask.  The norm runs down column t of A, i.e. over the window rows.  With
    `lse` [Hq, w] given, row r's weights are exp(z - lse[i, r]).
    """
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    p = n - w
    out = np.empty((hq, p), dtype=np.float64)
    for i in range(hq):
        g = i // G
        z = (q_win[i] @ k[g].T) / math.sqrt(d)
        A = softmax_rows(z) if lse is None else np.exp(z - np.asarray(lse, dtype=np.float64)[i][:, None])
        out[i] = np.sqrt((A[:, :p] ** 2).sum(axis=0))
    return out


def laprox_head_scores(q_win: np.ndarray, k: np.ndarray, v: np.ndarray, w_o: np.ndarray,
                       lse: np.ndarray | None = None, keys: np.ndarray | None = None) -> np.ndarray:
    """LaProx token score per query head, p_i[t] = ||A_i[:, t]||_2 * ||(V W^O_i)[t, :]||_2,
    [Hq, p] (or [Hq, len(keys)] for a subset of prefix tokens).

    LaProx page, Section 4.1, Algorithm 1, "评分 token": tokens of the window
    (t >= T - w) score infinity and are always kept, so only the prefix is
    scored here.  Section 4 opening: the layer output splits exactly into per-
    head contributions, and p_i[t] is the Frobenius norm of head i's rank-one
    contribution A_i[:, t] (V W^O_i)[t, :] of token t.
    """
    hq, w, d = q_win.shape
    hkv, n, _ = k.shape
    p = n - w
    a = laprox_attention_l2(q_win, k, lse)
    if keys is None:
        keys = np.arange(p)
    return a[:, keys] * projected_value_l2(v, w_o, hq, np.asarray(keys))


def laprox_scores(q_win: np.ndarray, k: np.ndarray, v: np.ndarray, w_o: np.ndarray,
                  lse: np.ndarray | None = None, keys: np.ndarray | None = None) -> np.ndarray:
    """LaProx score per KV head, [Hkv, p]: the mean of p_i over the query heads
    of the group.  The page describes multi-head attention only; a GQA KV entry
    serves its G query heads, and the group takes the mean of their scores as
    the Ada-KV and CriticalKV scorers do (for a fixed G the mean ranks as the
    sum does, also across layers)."""
    return group_mean(laprox_head_scores(q_win, k, v, w_o, lse, keys), k.shape[0])
