"""Target-token sampling with the windowed contextual penalty, by definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

TokenSwift pages: the model card's CLI example samples with min-p 0.1,
temperature 1.0 and a penalty of 1.2 over the last 1024 tokens; the summary
page's "Approach" adds a windowed contextual penalty against repetition, and
its ablation table sets theta = 1.2, W = 1024 and varies W from 20 to 2048.
The tool listing's "How it works" checks drafts against the target's tokens,
which are these samples.

Readings (the pages name the knobs, not the formulas):

* Row layout follows verification: row 0 is the position after the committed
  context, row t+1 the position after draft t (``parent``/``draft_tok`` as in
  the acceptance step), so R = T + 1 rows.
* The penalty window of row r is the last W tokens of its own context: the
  committed tokens ``hist`` followed, for r > 0, by the draft tokens on the
  root path of draft r-1 (root first). A token counts once however often it
  appears in the window.
* Penalty (the sign-aware repetition penalty in common use): a logit x of a
  windowed token becomes x / theta when x > 0 and x * theta otherwise, so that
  it loses probability whatever its sign. Dividing negative logits as well
  would raise their probability.
* Then temperature tau: y = z / tau. tau = 0 means greedy: the highest
  penalised logit, ties to the lower token id.
* Min-p: with p = softmax(y), token i is kept when p_i >= min_p * max p, i.e.
  when y_i - max y >= ln(min_p); min_p = 0 keeps every token.
* Top-p (nucleus; the summary page's temperature ablation samples "with
  top-p"): on the same distribution p, token i is kept when the total
  probability of the tokens strictly more probable than i is below top_p.
  The kept set is the smallest run of the most probable values whose mass
  reaches top_p, and tokens of equal probability are kept or dropped
  together (no token-order tie break inside a probability). top_p >= 1 keeps
  every token of non-zero probability. Both filters look at the same p and a
  token must pass both (the intersection; applying top-p first and min-p to
  the renormalised remainder gives the same set, as the largest probability
  always survives top-p).
* The draw: with the kept probabilities renormalised, the sampled token is the
  smallest id whose cumulative probability (token-id order) exceeds the
  caller's uniform u in [0, 1); past the last boundary (rounding) it is the
  last kept token. The random number is drawn by the caller and passed in.
* Logits may be -inf (a token that can never be drawn), not NaN, and every
  row needs one finite logit.
"""
from __future__ import annotations

import numpy as np

from .accept import _root_path


def penalty_window(hist, parent, draft_tok, row, window):
    """Tokens of row `row`'s window: the last `window` tokens of its context."""
    seq = [int(x) for x in hist]
    if row > 0:
        seq += [int(draft_tok[a]) for a in _root_path(np.asarray(parent), row - 1)]
    return seq[max(0, len(seq) - window):] if window > 0 else []


def penalize(x, tokens, theta):
    """Penalised logits: each distinct windowed token's logit shrinks (x > 0) or grows in magnitude."""
    z = np.array(x, dtype=np.float64, copy=True)
    for i in sorted(set(int(t) for t in tokens)):
        if 0 <= i < len(z):
            z[i] = z[i] / theta if z[i] > 0 else z[i] * theta
    return z


def mass_above(p):
    """For every token, the total probability of the tokens strictly more probable than it."""
    vals, inv = np.unique(p, return_inverse=True)           # distinct values, ascending
    mass = np.bincount(inv, weights=p, minlength=len(vals))  # probability held by each value
    suffix = np.cumsum(mass[::-1])[::-1]                     # mass at or above each value
    return np.concatenate([suffix[1:], [0.0]])[inv]


def kept_probs(z, temperature, min_p, top_p=1.0):
    """Renormalised probabilities after temperature, the min-p and the top-p
    filters (temperature > 0)."""
    y = z / temperature
    w = np.exp(y - y.max())                       # p_i / p_max
    keep = (w >= min_p) & (w > 0)
    if top_p < 1.0:
        keep &= mass_above(w / w.sum()) < top_p
    q = np.where(keep, w, 0.0)
    return q / q.sum(), keep, y


def sample_row(x, tokens, theta, temperature, min_p, u, top_p=1.0):
    """(token, diagnostics) for one row of logits."""
    z = penalize(x, tokens, theta)
    if temperature == 0:
        return int(np.argmax(z)), {"greedy": True, "z": z}
    q, keep, y = kept_probs(z, temperature, min_p, top_p)
    cdf = np.cumsum(q)
    idx = int(np.searchsorted(cdf, u, side="right"))        # first i with cdf[i] > u
    last_kept = int(np.nonzero(keep)[0][-1])
    tok = min(idx, last_kept)
    # how far the draw and the filters sit from a decision boundary
    u_margin = float(np.min(np.abs(cdf[keep] - u)))
    # tokens at the maximum are kept whatever min_p is, so they sit at no boundary
    below = y < y.max()
    keep_margin = float(np.min(np.abs((y[below] - y.max()) - np.log(min_p)), initial=np.inf)) \
        if min_p > 0 else np.inf
    # top-p: how close top_p comes to the mass above a probability value that
    # passes min-p (where a value's tokens switch between kept and dropped),
    # and the kept set with that nearest value's decision flipped
    topp_margin, keep_alt = np.inf, keep
    if top_p < 1.0:
        w = np.exp(y - y.max())
        above = mass_above(w / w.sum())
        cand = (w >= min_p) & (w > 0) & (above > 0)
        if cand.any():
            gap = np.abs(above - top_p)
            topp_margin = float(gap[cand].min())
            a_near = above[cand][np.argmin(gap[cand])]
            flip = cand & (above == a_near)
            keep_alt = keep ^ flip
    return tok, {"greedy": False, "z": z, "q": q, "keep": keep, "cdf": cdf, "u_margin": u_margin,
                 "keep_margin": keep_margin, "topp_margin": topp_margin, "keep_alt": keep_alt}


def sample_ref(logits, hist, parent, draft_tok, *, window, penalty, temperature, min_p, u, top_p=1.0):
    """Sampled token per row of `logits` [R][V] (R = T + 1), plus per-row diagnostics."""
    logits = np.asarray(logits, dtype=np.float64)
    R = logits.shape[0]
    T = 0 if parent is None else len(parent)
    assert R == T + 1
    toks, diags = [], []
    for r in range(R):
        win = penalty_window(hist, parent, draft_tok, r, window)
        t, d = sample_row(logits[r], win, penalty, temperature, min_p, float(u[r]), top_p)
        d["window"] = win
        toks.append(t)
        diags.append(d)
    return np.array(toks, np.int64), diags
