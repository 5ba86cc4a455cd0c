"""Retained cache and decode attention (oracle; float64; test infrastructure only)."""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np


def compact(kv: np.ndarray, sel: Sequence[np.ndarray], w: int) -> List[np.ndarray]:
    """Retained rows of every KV head: the selected prefix rows in ascending
    token order, then the w window rows.

    Ada-KV notes, Algorithm 2, steps 10-11 (select by the eviction decision,
    then concatenate with the window cache).  Works on any array [Hkv, n, d]
    (keys or values); the copy is exact.
    """
    hkv, n, _ = kv.shape
    p = n - w
    return [np.concatenate([kv[g, np.asarray(sel[g], dtype=np.int64)], kv[g, p:]], axis=0) for g in range(hkv)]


def flat_layout(budgets: Sequence[int], w: int, reserve: int):
    """Offsets of the flat cache: one segment per (instance, KV head) holding
    B_g + w retained rows followed by `reserve` empty rows for appends.

    The Ada-KV paper ("Variable-length Attention with Variable-sized Cache
    Elements") concatenates all heads' caches into one tensor; the segment
    offsets are the plainest index for it (an exclusive prefix sum).
    Returns (seg_start [S+1], seg_len [S]).
    """
    b = np.asarray(budgets, dtype=np.int64).ravel()
    seg_len = b + w
    start = np.zeros(b.size + 1, dtype=np.int64)
    np.cumsum(seg_len + reserve, out=start[1:])
    return start, seg_len


def decode(q: np.ndarray, k_hat: Sequence[np.ndarray], v_hat: Sequence[np.ndarray]) -> np.ndarray:
    """Decode attention over per-KV-head retained caches.

    Ada-KV notes, "多头自注意力层的形式化描述": A_i = softmax(q_i K_i^T) and the
    head output A_i V_i; the logits are divided by sqrt(d_h) (Ada-KV paper,
    Section 3.1 footnote 5; LAVa notes, "解码过程的残差流视角").  After eviction the
    softmax runs over the retained entries only (the masked form of the
    eviction-decision output).  q: [Hq, d]; k_hat[g], v_hat[g]: [len_g, d].
    Returns o [Hq, d].
    """
    hq, d = q.shape
    hkv = len(k_hat)
    G = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for i in range(hq):
        g = i // G
        z = (k_hat[g] @ q[i]) / math.sqrt(d)
        z = z - z.max()
        a = np.exp(z)
        a /= a.sum()
        out[i] = a @ v_hat[g]
    return out


def append(k_hat: Sequence[np.ndarray], v_hat: Sequence[np.ndarray], k_new: np.ndarray, v_new: np.ndarray):
    """Concatenate one new key and value per KV head before attending
    (Ada-KV notes, the cache update K_i = Cat[K_i : k_i] before the output)."""
    return ([np.concatenate([k_hat[g], k_new[g][None]], axis=0) for g in range(len(k_hat))],
            [np.concatenate([v_hat[g], v_new[g][None]], axis=0) for g in range(len(v_hat))])
