"""Seeded synthetic inputs for the tree-verify and partial-KV workloads.

This module only draws random numbers and lays out index structures. It holds
none of the attention, scoring or selection arithmetic: the GPU path and the
CPU oracle both receive the arrays built here and nothing else.

Workloads (the pages measure on PG-19 with real LLaMA activations; neither the
data nor the weights exist here, so Gaussian tensors at the real layer shapes
stand in for them):

* ``tiny``       fp32, Hq=4, Hkv=1, D=64, L=512, 40-node [1,3,3,3] tree, N(0,1).
* ``llama8b_20k``  bf16, Hq=32, Hkv=8, D=128, L=20480, tree + 20 four-token
  chains (T=120), Q ~ N(0,1), K,V ~ N(0,1)/sqrt(128).
* ``llama8b_100k`` as above with L=102400 (the ultra-long endpoint).
* ``partial_100k`` the partial-KV draft pass: 4 recent queries, 102400-token
  cache, 64-token chunks, budget of 64 chunks, 8 chunks per KV head with keys
  scaled by 3 before rounding.
* ``llama2_mha_100k`` bf16, Hq=Hkv=32, D=128, L=102400, same 120-query mask.
* ``make_sample``  target-token sampling over the verify rows: logits
  [121][128256] ~ N(0, 3^2) with 64 "hot" token ids raised by 8 in every row
  (so that a handful of tokens pass min-p 0.1 and the repetition penalty
  changes draws), 4096 committed tokens half drawn from the hot ids, draft
  tokens from the hot ids on the tree + chains forest, u ~ U[0, 1) in fp32.
* ``make_text``    a committed text for the 4-gram table: Zipf(1.2) token ids
  over the vocabulary, with 30% of the 32-token blocks copied from earlier in
  the text.

bf16 tensors are carried as ``np.uint16`` bit patterns (round to nearest even
from the fp32 draw); fp32 tensors as ``np.float32``.

Page references: the [1,3,3,3] tree and the 4-gram candidates come from the
TokenSwift tool listing ("How it works") and the ablation table of the
TokenSwift summary page (tree rows); ``--ngram_topk 20``, ``--gamma 4`` and
``--retrival_max_budget 4096`` from the TokenSwift-Qwen2.5-7B model card
("Example using TokenSwift command line").
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Constants the pages fix (model card CLI example; summary-page ablation table).
TREE_SHAPE = (1, 3, 3, 3)   # per-depth top-k of the candidate tree
NGRAM_TOPK = 20             # retrieved 4-gram candidates
GAMMA = 4                   # draft length: 4 logits, 4-grams, 4 recent queries
RETRIEVAL_BUDGET = 4096     # tokens kept in the partial KV cache
CHUNK = 64                  # tokens per importance chunk (budget = 64 chunks)
MIN_P = 0.1                 # sampling: min-p
TEMPERATURE = 1.0           # sampling: temperature
PENALTY = 1.2               # contextual penalty theta
PENALTY_WINDOW = 1024       # contextual penalty window W (tokens)
VOCAB = 128256              # LLaMA3.1 vocabulary


# --------------------------------------------------------------------------
# random streams and bf16 rounding
# --------------------------------------------------------------------------
def _streams(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("only finite values are rounded here")
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)          # finite inputs: u + 0x8000 < 2^32
    lsb += np.uint32(0x7FFF)
    lsb += u
    lsb >>= np.uint32(16)
    return lsb.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for test tolerances/plots)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, np.float32)


# --------------------------------------------------------------------------
# draft structures
# --------------------------------------------------------------------------
def tree_parents(shape: Sequence[int], rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Parent array of the per-depth top-k candidate tree ``shape``.

    Level 0 holds ``shape[0]`` roots; every node of level d has ``shape[d+1]``
    children. Nodes are numbered level by level (so parent[t] < t). With
    ``rng`` the order inside each level is shuffled and the parents remapped,
    so the numbering is not a canonical layout.
    """
    levels: List[List[int]] = []   # per level: list of parent *positions in previous level*
    sizes = []
    for d, width in enumerate(shape):
        n_prev = 1 if d == 0 else sizes[-1]
        lvl = [(-1 if d == 0 else p) for p in range(n_prev) for _ in range(width)]
        levels.append(lvl)
        sizes.append(len(lvl))
    parent = []
    offset_prev = 0
    new_pos_prev = None
    offset = 0
    for d, lvl in enumerate(levels):
        n = len(lvl)
        perm = rng.permutation(n) if rng is not None else np.arange(n)
        # perm[new_slot] = old index inside the level
        new_pos = np.empty(n, dtype=np.int64)
        new_pos[perm] = np.arange(n)
        level_par = [0] * n
        for old in range(n):
            p_old = lvl[old]
            p = -1 if p_old < 0 else offset_prev + int(new_pos_prev[p_old])
            level_par[int(new_pos[old])] = p
        parent.extend(level_par)
        offset_prev, new_pos_prev = offset, new_pos
        offset += n
    return np.asarray(parent, dtype=np.int32)


def chain_parents(n_chains: int, length: int, base: int) -> np.ndarray:
    """``n_chains`` causal chains of ``length`` nodes numbered from ``base``:
    node base+length*c+j has parent -1 when j == 0 and its predecessor otherwise."""
    out = np.empty(n_chains * length, dtype=np.int32)
    for c in range(n_chains):
        for j in range(length):
            t = c * length + j
            out[t] = -1 if j == 0 else base + t - 1
    return out


def tree_plus_chains_parents(rng: np.random.Generator, shape: Sequence[int] = TREE_SHAPE) -> np.ndarray:
    """The candidate tree `shape` (shuffled within levels) followed by the
    4-gram chains; [1,9,9,9] gives 820 + 80 = 900 drafts."""
    tree = tree_parents(shape, rng)
    chains = chain_parents(NGRAM_TOPK, GAMMA, base=len(tree))
    return np.concatenate([tree, chains]).astype(np.int32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class VerifyCase:
    name: str
    dtype: str
    T: int
    Hq: int
    Hkv: int
    D: int
    L: int
    scale: float
    parent: np.ndarray      # int32 [T]
    q: np.ndarray           # [T][Hq][D]
    k_cache: np.ndarray     # [Hkv][L][D]
    v_cache: np.ndarray
    k_draft: np.ndarray     # [Hkv][T][D]
    v_draft: np.ndarray

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes(self) -> int:
        return 2 * self.k_cache.nbytes


@dataclasses.dataclass
class PartialCase:
    name: str
    dtype: str
    R: int                  # recent queries used for scoring (= draft queries)
    Hq: int
    Hkv: int
    D: int
    L: int
    chunk: int
    k: int                  # chunks kept per KV head
    scale: float
    q: np.ndarray           # [R][Hq][D]
    k_cache: np.ndarray     # [Hkv][L][D]
    v_cache: np.ndarray
    k_new: np.ndarray       # [Hkv][R][D]
    v_new: np.ndarray
    boosted: np.ndarray     # int32 [Hkv][8] chunk ids whose keys were scaled by 3

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_chunks(self) -> int:
        return self.L // self.chunk


def make_verify(name: str, *, dtype: str, Hq: int, Hkv: int, D: int, L: int,
                seed: int, with_chains: bool, q_std: float = 1.0,
                kv_std: Optional[float] = None, parent: Optional[np.ndarray] = None) -> VerifyCase:
    rq, rk, rv, rkd, rvd, rp = _streams(seed, 6)
    if parent is None:
        parent = tree_plus_chains_parents(rp) if with_chains else tree_parents(TREE_SHAPE, rp)
    T = int(len(parent))
    if kv_std is None:
        kv_std = 1.0 / np.sqrt(D) if dtype == BF16 else 1.0
    q = _encode(_normal(rq, (T, Hq, D), q_std), dtype)
    kc = _encode(_normal(rk, (Hkv, L, D), kv_std), dtype)
    vc = _encode(_normal(rv, (Hkv, L, D), kv_std), dtype)
    kd = _encode(_normal(rkd, (Hkv, T, D), kv_std), dtype)
    vd = _encode(_normal(rvd, (Hkv, T, D), kv_std), dtype)
    return VerifyCase(name, dtype, T, Hq, Hkv, D, L, float(1.0 / np.sqrt(D)),
                      np.ascontiguousarray(parent, np.int32), q, kc, vc, kd, vd)


def make_partial(name: str = "partial_100k", *, Hq: int = 32, Hkv: int = 8, D: int = 128,
                 L: int = 102400, R: int = GAMMA, chunk: int = CHUNK,
                 k: int = RETRIEVAL_BUDGET // CHUNK, n_boost: int = 8, boost: float = 3.0,
                 seed: int = 3) -> PartialCase:
    rq, rk, rv, rkn, rvn, rb = _streams(seed, 6)
    std = 1.0 / np.sqrt(D)
    n_chunks = L // chunk
    q = _normal(rq, (R, Hq, D), 1.0)
    kc = _normal(rk, (Hkv, L, D), std)
    boosted = np.stack([np.sort(rb.choice(n_chunks, size=n_boost, replace=False))
                        for _ in range(Hkv)]).astype(np.int32) if n_boost else \
        np.zeros((Hkv, 0), np.int32)
    for g in range(Hkv):
        for c in boosted[g]:
            kc[g, c * chunk:(c + 1) * chunk, :] *= np.float32(boost)
    vc = _normal(rv, (Hkv, L, D), std)
    kn = _normal(rkn, (Hkv, R, D), std)
    vn = _normal(rvn, (Hkv, R, D), std)
    return PartialCase(name, BF16, R, Hq, Hkv, D, L, chunk, k, float(1.0 / np.sqrt(D)),
                       f32_to_bf16_bits(q), f32_to_bf16_bits(kc), f32_to_bf16_bits(vc),
                       f32_to_bf16_bits(kn), f32_to_bf16_bits(vn), boosted)


@dataclasses.dataclass
class SampleCase:
    name: str
    dtype: str
    R: int
    V: int
    logits: np.ndarray       # [R][V] fp32, or bf16 bit patterns
    hist: np.ndarray         # int32 [n_hist] committed tokens, oldest first
    parent: np.ndarray       # int32 [T], T = R - 1
    draft_tok: np.ndarray    # int32 [T]
    u: np.ndarray            # fp32 [R] uniforms in [0, 1)


def make_sample(name: str = "sample_llama8b", *, dtype: str = F32, V: int = VOCAB, n_hist: int = 4096,
                parent: Optional[np.ndarray] = None, logit_std: float = 3.0, n_hot: int = 64,
                hot_boost: float = 8.0, seed: int = 5) -> SampleCase:
    rl, rh, rd, ru, rp, rhot = _streams(seed, 6)
    if parent is None:
        parent = tree_plus_chains_parents(rp)
    T = int(len(parent))
    R = T + 1
    x = _normal(rl, (R, V), logit_std)
    hot = rhot.choice(V, size=min(n_hot, V), replace=False)
    x[:, hot] += np.float32(hot_boost)
    from_hot = rh.random(n_hist) < 0.5
    hist = np.where(from_hot, rh.choice(hot, n_hist), rh.integers(0, V, n_hist)).astype(np.int32)
    draft_tok = rd.choice(hot, size=T).astype(np.int32)
    u = ru.random(R, dtype=np.float32)
    return SampleCase(name, dtype, R, V, _encode(x, dtype), hist,
                      np.ascontiguousarray(parent, np.int32), draft_tok, u)


def make_text(n: int, *, V: int = VOCAB, zipf: float = 1.2, copy_prob: float = 0.3, block: int = 32,
              seed: int = 7) -> np.ndarray:
    """A committed text of n tokens: Zipf-distributed ids (id = rank - 1, past V
    folded back), and with probability `copy_prob` a 32-token block copied
    from an earlier place in the text (the repetition that 4-gram retrieval
    reuses)."""
    rz, rc = _streams(seed, 2)
    out = np.empty(n, np.int32)
    pos = 0
    while pos < n:
        m = min(block, n - pos)
        if pos >= block and rc.random() < copy_prob:
            src = int(rc.integers(0, pos - m + 1))
            out[pos:pos + m] = out[src:src + m]
        else:
            out[pos:pos + m] = (rz.zipf(zipf, m) - 1) % V
        pos += m
    return out


def workload(name: str, *, L: Optional[int] = None, seed: Optional[int] = None):
    """The named workloads; ``L`` shrinks the cache for quick tests."""
    if name == "tiny":
        return make_verify(name, dtype=F32, Hq=4, Hkv=1, D=64, L=512 if L is None else L,
                           seed=0 if seed is None else seed, with_chains=False)
    if name == "llama8b_20k":
        return make_verify(name, dtype=BF16, Hq=32, Hkv=8, D=128, L=20480 if L is None else L,
                           seed=1 if seed is None else seed, with_chains=True)
    if name == "llama8b_100k":
        return make_verify(name, dtype=BF16, Hq=32, Hkv=8, D=128, L=102400 if L is None else L,
                           seed=2 if seed is None else seed, with_chains=True)
    if name == "partial_100k":
        return make_partial(name, L=102400 if L is None else L, seed=3 if seed is None else seed)
    if name == "llama2_mha_100k":
        return make_verify(name, dtype=BF16, Hq=32, Hkv=32, D=128, L=102400 if L is None else L,
                           seed=4 if seed is None else seed, with_chains=True)
    raise KeyError(name)


WORKLOADS = ("tiny", "llama8b_20k", "llama8b_100k", "partial_100k", "llama2_mha_100k")
