"""Dynamic partial KV cache: importance, top-k chunk selection, gather.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The TokenSwift summary page ("Approach") drafts over a reduced KV cache that
is re-selected as generation proceeds, by how strongly queries attend to its
keys; the model card CLI example sets that budget to 4096 tokens. The pages give no formula, so these readings
hold (each is a plain definition, not an algorithm):

* importance of chunk c of KV head g (tokens c*chunk .. c*chunk+chunk-1),
  from R recent queries:
      u[r, j]  = max over heads h of group g of  scale * <q[r,h], K[g,j]>
      score    = mean over (r, j in chunk) of u[r, j]
* selection: per KV head, the k chunks of highest score; between equal scores
  the lower chunk index ranks higher; returned in ascending chunk order, so the
  gathered cache keeps time order.
* gather: chunk i of the partial cache is chunk idx[g][i] of the full cache,
  copied bit for bit, for K and for V.
"""
from __future__ import annotations

import numpy as np

from .attention import widen


def importance_ref(q_recent, k_cache, scale, chunk, dtype, heads=None):
    """float64 scores [Hkv][L // chunk]. q_recent [R][Hq][D], k_cache [Hkv][L][D]."""
    q = widen(q_recent, dtype)
    R, Hq, D = q.shape
    Hkv, L, _ = k_cache.shape
    G = Hq // Hkv
    n_chunks = L // chunk
    scores = np.full((Hkv, n_chunks), np.nan)
    for g in (range(Hkv) if heads is None else heads):
        k = widen(k_cache[g, :n_chunks * chunk], dtype)          # [L][D]
        qg = q[:, g * G:(g + 1) * G, :]                          # [R][G][D]
        s = scale * (qg.reshape(R * G, D) @ k.T).reshape(R, G, -1)  # [R][G][L]
        u = s.max(axis=1)                                        # [R][L]
        scores[g] = u.reshape(R, n_chunks, chunk).mean(axis=(0, 2))
    return scores


def topk_ref(scores, k):
    """int32 [Hkv][k]: per row, the k best chunks (score desc, index asc on ties),
    listed in ascending chunk index. Also returns their scores in that order."""
    scores = np.asarray(scores)
    Hkv, n = scores.shape
    idx = np.empty((Hkv, k), dtype=np.int32)
    val = np.empty((Hkv, k), dtype=scores.dtype)
    for g in range(Hkv):
        order = np.lexsort((np.arange(n), -scores[g]))   # primary: -score, then index
        chosen = np.sort(order[:k])
        idx[g] = chosen
        val[g] = scores[g, chosen]
    return idx, val


def gather_ref(k_cache, v_cache, chunk_idx, chunk):
    """Partial caches [Hkv][k*chunk][D], same element type as the inputs."""
    Hkv, _, D = k_cache.shape
    k = chunk_idx.shape[1]
    kp = np.empty((Hkv, k * chunk, D), dtype=k_cache.dtype)
    vp = np.empty((Hkv, k * chunk, D), dtype=v_cache.dtype)
    for g in range(Hkv):
        for i in range(k):
            c = int(chunk_idx[g, i])
            kp[g, i * chunk:(i + 1) * chunk] = k_cache[g, c * chunk:(c + 1) * chunk]
            vp[g, i * chunk:(i + 1) * chunk] = v_cache[g, c * chunk:(c + 1) * chunk]
    return kp, vp
