"""Tree-verify attention and partial-cache draft attention, plain float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (TokenSwift tool listing, "How it works"): verification runs
the target model once over all draft tokens against its complete KV cache, and
the tree mask lets every candidate see, among the drafts, only itself and its
ancestors. With
``A(t) = {t} U ancestors(t)`` along ``parent[]``, for draft row t and query
head h of KV group g = h // G:

    s_j = scale * <q[t,h], Kc[g,j]>   for every cached token j in [0, L)
    s_a = scale * <q[t,h], Kd[g,a]>   for every draft a in A(t)
    M   = max s,  Z = sum exp(s - M)
    out[t,h] = sum exp(s - M) * v / Z,   lse[t,h] = M + ln Z

Readings where the pages are silent: contiguous GQA groups (g = h // G),
scale = 1/sqrt(D), natural-log LSE of the scaled logits, draft K/V held apart
from the cache (the cache is updated only after verification), and no
visibility between different roots of the forest (tree vs 4-gram chains).
"""
from __future__ import annotations

import numpy as np


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of the values a kernel reads: bf16 bits or fp32."""
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    raise ValueError(dtype)


def ancestor_mask(parent: np.ndarray) -> np.ndarray:
    """Boolean [T][T]: entry (t, a) is True iff a is t or an ancestor of t.

    ``parent[t]`` in [-1, t); -1 marks a root (the drafts form a forest).
    """
    parent = np.asarray(parent, dtype=np.int64)
    T = len(parent)
    vis = np.zeros((T, T), dtype=bool)
    for t in range(T):
        a = t
        while a >= 0:
            if vis[t, a]:
                raise ValueError("cycle in parent array")
            vis[t, a] = True
            p = int(parent[a])
            if p >= a:
                raise ValueError("parent[t] must be < t")
            a = p
    return vis


def verify_attn_ref(q, k_cache, v_cache, k_draft, v_draft, parent, scale, dtype, heads=None):
    """Masked softmax attention of T draft rows; returns (out, lse) in float64.

    q [T][Hq][D]; k_cache, v_cache [Hkv][L][D]; k_draft, v_draft [Hkv][T][D].
    ``heads``: optional iterable of KV heads to evaluate (others left NaN), used
    to bound the CPU time of very large cases.
    """
    q = widen(q, dtype)
    T, Hq, D = q.shape
    Hkv = k_cache.shape[0]
    G = Hq // Hkv
    vis = ancestor_mask(parent)
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    for g in (range(Hkv) if heads is None else heads):
        kc = widen(k_cache[g], dtype)            # [L][D]
        vc = widen(v_cache[g], dtype)
        kd = widen(k_draft[g], dtype)            # [T][D]
        vd = widen(v_draft[g], dtype)
        for h in range(g * G, (g + 1) * G):
            qh = q[:, h, :]                      # [T][D]
            s_cache = scale * (qh @ kc.T)        # [T][L]
            s_draft = scale * (qh @ kd.T)        # [T][T]
            s_draft = np.where(vis, s_draft, -np.inf)
            s = np.concatenate([s_cache, s_draft], axis=1)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            v_all = np.concatenate([vc, vd], axis=0)
            out[:, h, :] = (e @ v_all) / z
            lse[:, h] = m[:, 0] + np.log(z[:, 0])
    return out, lse


def draft_attn_ref(q, k_part, v_part, k_new, v_new, scale, dtype, heads=None):
    """Self-drafting attention over the partial cache (TokenSwift tool listing,
    "How it works"): Tq new tokens see every gathered token and, among
    themselves, their predecessors (a single causal chain)."""
    Tq = q.shape[0]
    chain = np.arange(-1, Tq - 1, dtype=np.int32)
    return verify_attn_ref(q, k_part, v_part, k_new, v_new, chain, scale, dtype, heads=heads)
