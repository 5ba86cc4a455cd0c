"""Loss bounds and the renormalisation identity (oracle; float64; test infrastructure only).

All checks use one decode query per query head and its full attention A_i over
the n cached entries of its KV head, and a keep-mask T [Hkv, n] (True = kept)
shared by the query heads of a group.  W^O has the pages' shape [Hq*d, D].
"""
from __future__ import annotations

import math

import numpy as np


def attention(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """A_i = softmax(q_i K_g^T / sqrt(d)) over all n entries, [Hq, n]."""
    hq, d = q.shape
    hkv = k.shape[0]
    G = hq // hkv
    A = np.empty((hq, k.shape[1]))
    for i in range(hq):
        z = (k[i // G] @ q[i]) / math.sqrt(d)
        e = np.exp(z - z.max())
        A[i] = e / e.sum()
    return A


def masked_attention(q: np.ndarray, k: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """softmax(-inf * (1 - T) + q K^T / sqrt(d)): the post-eviction weights of
    the Ada-KV notes, "Top-k方法的理论基础与驱逐损失上界"."""
    hq, d = q.shape
    G = hq // k.shape[0]
    A = np.zeros((hq, k.shape[1]))
    for i in range(hq):
        g = i // G
        z = (k[g] @ q[i]) / math.sqrt(d)
        z = np.where(keep[g], z, -np.inf)
        e = np.exp(z - z[keep[g]].max())
        A[i] = e / e.sum()
    return A


def layer_output(A: np.ndarray, v: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """y = sum_i A_i V_i W^O_i  (Ada-KV notes, the multi-head output formula)."""
    hq = A.shape[0]
    hkv, n, d = v.shape
    G = hq // hkv
    y = np.zeros(w_o.shape[1])
    for i in range(hq):
        y += (A[i] @ v[i // G]) @ w_o[i * d:(i + 1) * d]
    return y


def renormalisation_gap(q, k, keep) -> float:
    """Largest gap between the masked softmax and T*A / ||A (.) T||_1
    (Ada-KV notes, proof of Theorem 3.1, the first derived identity)."""
    A = attention(q, k)
    G = q.shape[0] // k.shape[0]
    T = np.repeat(keep, G, axis=0).astype(np.float64)
    ren = (T * A) / (T * A).sum(axis=1, keepdims=True)
    return float(np.abs(masked_attention(q, k, keep) - ren).max())


def adakv_theorem31(q, k, v, w_o, keep):
    """(L1 loss, epsilon) of the Ada-KV notes, Theorem 3.1:
    ||y - y_hat||_1 <= 2 h C - 2 C sum_i sum_j T_i^j A_i^j, with
    C = max over heads and entries of the L1 norm of a row of V_i W^O_i
    (the row norm the proof's triangle-inequality step needs)."""
    hq, d = q.shape
    G = hq // k.shape[0]
    A = attention(q, k)
    Ah = masked_attention(q, k, keep)
    loss = float(np.abs(layer_output(A, v, w_o) - layer_output(Ah, v, w_o)).sum())
    C = max(float(np.abs(v[i // G] @ w_o[i * d:(i + 1) * d]).sum(axis=1).max()) for i in range(hq))
    T = np.repeat(keep, G, axis=0)
    eps = 2 * hq * C - 2 * C * float((A * T).sum())
    return loss, eps


def lava_theorem1(q, k, v, w_o, keep):
    """(L1 loss, bound) of the LAVa notes, Theorem 1:
    ||y - y_hat||_1 <= 2 C_hat sum_h sum_i A_h[i] V_bar_h (1 - T_h[i]) with
    C_hat = ||W^O^T||_1 (largest absolute row sum of W^O) and
    V_bar_h = max_k ||V_h[k]||_1."""
    hq, d = q.shape
    G = hq // k.shape[0]
    A = attention(q, k)
    Ah = masked_attention(q, k, keep)
    loss = float(np.abs(layer_output(A, v, w_o) - layer_output(Ah, v, w_o)).sum())
    c_hat = float(np.abs(w_o).sum(axis=1).max())
    vbar = np.abs(v).sum(axis=2).max(axis=1)
    T = np.repeat(keep, G, axis=0)
    bound = 2 * c_hat * float(sum((A[i] * (1 - T[i])).sum() * vbar[i // G] for i in range(hq)))
    return loss, bound


def criticalkv_theta(q, k, v, w_o, keep):
    """Per-head (L1 loss, theta) of the CriticalKV notes, "输出扰动的可解析上界":
    L <= theta = C - (2 - 1/sum N A) * sum_i N_i A_i ||(V W^O)_i||_1.
    The page gives C only as a constant independent of N; setting N = 1
    (nothing evicted, loss 0) forces C = sum_i A_i ||(V W^O)_i||_1, which is
    the value used here (parity unpinned for the page's own C)."""
    hq, d = q.shape
    G = hq // k.shape[0]
    A = attention(q, k)
    Ah = masked_attention(q, k, keep)
    res = []
    for i in range(hq):
        g = i // G
        vw = v[g] @ w_o[i * d:(i + 1) * d]
        loss = float(np.abs(A[i] @ vw - Ah[i] @ vw).sum())
        nrm = np.abs(vw).sum(axis=1)
        C = float((A[i] * nrm).sum())
        sig = float((A[i] * keep[g]).sum())
        theta = C - (2 - 1 / sig) * float((keep[g] * A[i] * nrm).sum())
        res.append((loss, theta))
    return res
