"""GPU parity of ts_sample_tokens (target-token sampling with the windowed
repetition penalty, temperature and min-p) against the oracle.

The sampled token is an integer decided by floating point: the GPU sums the
kept weights in fp32 in its own order, the oracle in fp64. So a row must match
the oracle exactly whenever its draw u sits more than 1e-4 (of the kept mass)
from a cumulative boundary and no logit sits within 1e-4 of the min-p cut;
closer to a boundary, the GPU's token must still be a valid draw within 2e-5
of it (either neighbour of the boundary). Greedy rows must match exactly
unless the two best penalised logits are within 1e-6 relative."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV, say, to_dev
from long_context_kv_ts_amd import inputs, ops
from oracle import sample_ref, widen

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sample_example.json")
EXACT_MARGIN = 1e-4
VALID_TOL = 2e-5


def _i32(a):
    a = np.asarray(a, np.int32)
    return to_dev(a, "i32") if a.size else None


def _is_draw(g, u, q, cdf, keep, border):
    """Token g is the inverse-CDF draw at u of the kept distribution q (within VALID_TOL)."""
    lo, hi = cdf[g] - q[g], cdf[g]
    return (q[g] > 0 or border) and lo - VALID_TOL <= u < hi + VALID_TOL


def run(logits, dtype, hist, parent, draft, *, window, penalty, temperature, min_p, u, label,
        workspace=None, top_p=1.0):
    R = logits.shape[0]
    u = np.asarray(u, np.float32)
    tok = ops.sample_tokens(to_dev(logits, dtype), hist=_i32(hist), parent=_i32(parent) if len(parent) else None,
                            draft_tok=_i32(draft) if len(draft) else None, window=window, penalty=penalty,
                            temperature=temperature, min_p=min_p, top_p=top_p, u=to_dev(u, "f32"),
                            workspace=workspace)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    ref, diags = sample_ref(widen(logits, dtype), hist, parent if len(parent) else None, draft,
                            window=window, penalty=penalty, temperature=temperature, min_p=min_p,
                            u=u.astype(np.float64), top_p=top_p)
    near = 0
    for r in range(R):
        g, e, d = int(got[r]), int(ref[r]), diags[r]
        if d["greedy"]:
            z = d["z"]
            if g != e:
                assert 0 <= g < len(z) and z[g] >= z.max() - 1e-6 * abs(z.max()), f"{label} row {r}: {g} != {e}"
                near += 1
            continue
        if d["u_margin"] > EXACT_MARGIN and d["keep_margin"] > EXACT_MARGIN and d["topp_margin"] > EXACT_MARGIN:
            assert g == e, f"{label} row {r}: token {g} != oracle {e} (u={u[r]})"
            continue
        near += 1
        assert 0 <= g < len(d["q"]), f"{label} row {r}: token {g} out of range"
        y = d["z"] / temperature
        border = abs((y[g] - y.max()) - np.log(min_p)) < VALID_TOL if min_p > 0 else False
        ok = _is_draw(g, u[r], d["q"], d["cdf"], d["keep"], border)
        if not ok and d["topp_margin"] <= EXACT_MARGIN:
            # top-p within rounding of a cumulative boundary: the nearest
            # probability value may be kept or dropped
            w = np.where(d["keep_alt"], np.exp(y - y.max()), 0.0)
            q2 = w / w.sum()
            ok = _is_draw(g, u[r], q2, np.cumsum(q2), d["keep_alt"], border)
        assert ok, f"{label} row {r}: token {g} (oracle {e}) is not a draw at u={u[r]}"
    say(f"  {label}: {R} rows, {near} near a boundary, tokens {got[:6].tolist()}...")
    return got


def test_hand_worked_example():
    ex = json.load(open(GOLDEN))
    x = np.array(ex["logits"], np.float32)
    kw = dict(window=ex["window"], penalty=ex["penalty"], min_p=ex["min_p"])
    g = run(x, "f32", ex["hist"], ex["parent"], ex["draft_tok"], temperature=0.0, u=[0.5] * 3,
            label="golden greedy", **kw)
    assert g.tolist() == ex["greedy"]
    for d in ex["draws"]:
        g = run(x, "f32", ex["hist"], ex["parent"], ex["draft_tok"], temperature=1.0, u=d["u"],
                label=f"golden u={d['u']}", **kw)
        assert g.tolist() == d["tok"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_rows_full_vocabulary(dtype):
    """The pages' settings (min-p 0.1, temperature 1, theta 1.2, W 1024) on the
    121 rows of the tree + chains verify pass over the LLaMA3.1 vocabulary."""
    c = inputs.make_sample(dtype=dtype)
    run(c.logits, dtype, c.hist, c.parent, c.draft_tok, window=inputs.PENALTY_WINDOW, penalty=inputs.PENALTY,
        temperature=inputs.TEMPERATURE, min_p=inputs.MIN_P, u=c.u, label=f"121x128256 {dtype}")


@pytest.mark.parametrize("window,penalty,temperature,min_p", [
    (1024, 1.2, 0.0, 0.1),        # greedy
    (0, 1.2, 1.0, 0.1),           # no window
    (1024, 1.0, 1.0, 0.1),        # no penalty
    (1024, 1.2, 1.0, 0.0),        # min-p off: every token kept
    (20, 1.2, 0.5, 0.05),         # the ablation's shortest window
    (2048, 1.2, 1.5, 0.2),        # and its longest
    (1024, 1.2, 1.0, 1.0),        # only the maximum survives
    (1024, 1.2, 1e-3, 0.1),       # near-greedy
])
def test_knobs(window, penalty, temperature, min_p):
    c = inputs.make_sample(dtype="bf16", seed=6)
    run(c.logits, "bf16", c.hist, c.parent, c.draft_tok, window=window, penalty=penalty,
        temperature=temperature, min_p=min_p, u=c.u, label=f"W={window} theta={penalty} tau={temperature} "
                                                          f"min_p={min_p}")


@pytest.mark.parametrize("V", [1, 3, 7, 9, 1023, 1024, 1025, 4095, 4096, 4097, 8200, 16385, 128257])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_vocabularies_and_edges(V, dtype):
    """Vocabularies around the 1024-logit sub-slices and the 4096-token ranges of
    one scanning workgroup, odd row lengths (misaligned
    rows), window ids outside [0, V), -inf logits, u = 0 and u just below 1."""
    rng = np.random.default_rng(V)
    parent = np.array([-1, 0, 1, -1, 3], np.int32)
    draft = rng.integers(0, V, 5).astype(np.int32)
    hist = np.concatenate([rng.integers(0, V, 300), [-5, V + 3, V]]).astype(np.int32)
    x = (rng.standard_normal((6, V)) * 2).astype(np.float32)
    if V > 2:
        x[1, ::3] = -np.inf
        x[2, 1:] = -np.inf
    if dtype == "bf16":
        fin = np.isfinite(x)
        b = inputs.f32_to_bf16_bits(np.where(fin, x, 0))
        b[~fin] = 0xFF80                                   # bf16 -inf
        x = b
    u = rng.random(6, dtype=np.float32)
    u[0], u[3] = 0.0, np.float32(np.nextafter(np.float32(1), np.float32(0)))
    for tau, mp in ((1.0, 0.1), (0.7, 0.0), (0.0, 0.1)):
        run(x, dtype, hist, parent, draft, window=64, penalty=1.3, temperature=tau, min_p=mp, u=u,
            label=f"V={V} {dtype} tau={tau} min_p={mp}")


@pytest.mark.parametrize("V", [128256, 100003])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_kept_sets_reread_every_sub_slice(V, dtype):
    """Flat logits with min-p on: every 1024-logit sub-slice keeps more tokens
    than its 32-entry list, so each one is read again at the row's cut (one a
    wave) and the token comes from the chosen sub-slice's logits, with the
    window bits the scan stored. V = 100003 takes element loads."""
    parent = np.array([-1, 0, 0, 1], np.int32)
    c = inputs.make_sample(dtype=dtype, V=V, parent=parent, logit_std=0.3, hot_boost=0.5, seed=21)
    for tau, mp in ((2.0, 0.05), (1.0, 0.3)):
        run(c.logits, dtype, c.hist, c.parent, c.draft_tok, window=1024, penalty=1.2, temperature=tau,
            min_p=mp, u=c.u, label=f"wide V={V} {dtype} tau={tau} min_p={mp}")


@pytest.mark.parametrize("V", [1048576, 1048575])
def test_largest_vocabulary(V):
    """V = 2^20 (1024 sub-slices a row, four a picking thread) and one less."""
    parent = np.array([-1, 0], np.int32)
    for dtype in ("f32", "bf16"):
        c = inputs.make_sample(dtype=dtype, V=V, parent=parent, n_hist=3000, seed=22)
        for tau, mp in ((1.0, 0.1), (3.0, 0.02), (0.0, 0.1)):
            run(c.logits, dtype, c.hist, c.parent, c.draft_tok, window=2048, penalty=1.2, temperature=tau,
                min_p=mp, u=c.u, label=f"V={V} {dtype} tau={tau} min_p={mp}")


def test_single_row_no_drafts_no_history():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((1, 50000)) * 3).astype(np.float32)
    for u in (0.0, 0.25, 0.999):
        run(x, "f32", [], [], [], window=1024, penalty=1.2, temperature=1.0, min_p=0.1, u=[u],
            label=f"T=0 u={u}")


def test_deep_chain_window_from_the_path():
    """A 256-draft chain with W = 64: late rows' windows hold only draft tokens."""
    T = 256
    parent = np.arange(-1, T - 1, dtype=np.int32)
    c = inputs.make_sample(dtype="f32", V=5000, parent=parent, n_hot=40, seed=8)
    run(c.logits, "f32", c.hist, c.parent, c.draft_tok, window=64, penalty=1.5, temperature=1.0,
        min_p=0.05, u=c.u, label="chain 256, W=64")


def test_901_rows_of_the_largest_tree():
    """The [1,9,9,9] tree with 20 chains: 900 drafts, 901 rows to sample."""
    parent = inputs.tree_plus_chains_parents(np.random.default_rng(2), shape=(1, 9, 9, 9))
    c = inputs.make_sample(dtype="bf16", V=32000, parent=parent, seed=13)
    assert c.R == 901
    run(c.logits, "bf16", c.hist, c.parent, c.draft_tok, window=1024, penalty=1.2, temperature=1.0,
        min_p=0.1, u=c.u, label="901 rows")


def test_reused_workspace_with_garbage():
    ws = ops.alloc_workspace(int(ops.lib().ts_sample_workspace(257, 300000)), DEV)
    ws.fill_(0x7F)
    for V, dtype, seed in ((300000, "f32", 1), (128256, "bf16", 2), (1000, "f32", 3)):
        c = inputs.make_sample(dtype=dtype, V=V, seed=seed)
        run(c.logits, dtype, c.hist, c.parent, c.draft_tok, window=1024, penalty=1.2, temperature=1.0,
            min_p=0.1, u=c.u, label=f"shared workspace V={V}", workspace=ws)


# ---------------------------------------------------------------------------
# top-p (nucleus)
# ---------------------------------------------------------------------------
TOPP_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "top_p_example.json")


def test_top_p_hand_worked_example():
    ex = json.load(open(TOPP_GOLDEN))
    x = np.array([ex["logits"]], np.float32)
    for c in ex["cases"]:
        for u, tok in c["draws"]:
            g = run(x, "f32", [], [], [], window=0, penalty=1.2, temperature=c["temperature"], min_p=c["min_p"],
                    top_p=c["top_p"], u=[u], label=f"golden top_p={c['top_p']} u={u}")
            assert g.tolist() == [tok]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("temperature,min_p,top_p", [
    (1.0, 0.1, 0.9),              # the CLI's min-p with a nucleus on top (min-p binds: no crossing bin sought)
    (1.0, 0.001, 0.5),            # both filters, the nucleus binding (the crossing bin's key passes)
    (0.4, 0.0, 0.9),              # the temperature ablation's range, top-p alone
    (0.8, 0.0, 0.95),
    (1.2, 0.0, 0.9),
    (1.0, 0.0, 0.5),
])
def test_top_p_verify_rows_full_vocabulary(dtype, temperature, min_p, top_p):
    """121 rows over the 128,256-token vocabulary with the pages' penalty."""
    c = inputs.make_sample(dtype=dtype)
    run(c.logits, dtype, c.hist, c.parent, c.draft_tok, window=inputs.PENALTY_WINDOW, penalty=inputs.PENALTY,
        temperature=temperature, min_p=min_p, top_p=top_p, u=c.u,
        label=f"top-p 121x128256 {dtype} tau={temperature} min_p={min_p} top_p={top_p}")


@pytest.mark.parametrize("top_p", [1e-6, 0.3, 0.999])
def test_top_p_flat_and_tied_logits(top_p):
    """Logits that take few distinct values: whole groups of equal
    probability are kept or dropped together (all tied: every token kept)."""
    rng = np.random.default_rng(31)
    V = 40000
    x = np.zeros((4, V), np.float32)                     # row 0: all equal
    x[1] = rng.integers(0, 4, V).astype(np.float32)      # four values
    x[2] = np.round(rng.standard_normal(V) * 2, 1)       # many ties
    x[3] = rng.standard_normal(V).astype(np.float32) * 0.01
    u = rng.random(4, dtype=np.float32)
    for tau in (1.0, 0.5):
        parent = np.array([-1, 0, 1], np.int32)
        run(x, "f32", [], parent, np.array([5, 6, 7], np.int32), window=4, penalty=1.2, temperature=tau,
            min_p=0.0, top_p=top_p, u=u, label=f"tied tau={tau} top_p={top_p}")


@pytest.mark.parametrize("temperature,top_p", [
    (1e-8, 0.9),                  # near-greedy: z * log2e / tau passes the coarse levels' clamp
    (1e-3, 0.5),
    (0.3, 0.9999999),             # the nucleus nearly the whole mass: the cut lies in the deepest bins
    (5.0, 0.999),                 # hot: weight spread over most of the vocabulary
])
def test_top_p_extreme_temperatures_and_deep_cuts(temperature, top_p):
    """16 rows over the 128,256-token vocabulary (logits N(0, 3^2) with 64 hot
    tokens, the pages' penalty) at temperatures and nuclei that put the cut at
    the ends of the coarse binning."""
    c = inputs.make_sample(dtype="f32", parent=np.arange(-1, 14, dtype=np.int32), seed=41)
    run(c.logits, "f32", c.hist, c.parent, c.draft_tok, window=inputs.PENALTY_WINDOW, penalty=inputs.PENALTY,
        temperature=temperature, min_p=0.0, top_p=top_p, u=c.u,
        label=f"top-p 16x128256 tau={temperature} top_p={top_p}")


@pytest.mark.parametrize("V", [7, 1025, 4097, 128257])
def test_top_p_ragged_vocabularies(V):
    rng = np.random.default_rng(V + 1)
    parent = np.array([-1, 0, 1], np.int32)
    draft = rng.integers(0, V, 3).astype(np.int32)
    hist = rng.integers(0, V, 200).astype(np.int32)
    x = (rng.standard_normal((4, V)) * 2).astype(np.float32)
    x[1, ::5] = -np.inf
    u = rng.random(4, dtype=np.float32)
    for dtype in ("f32", "bf16"):
        xx = x
        if dtype == "bf16":
            fin = np.isfinite(x)
            xx = inputs.f32_to_bf16_bits(np.where(fin, x, 0))
            xx[~fin] = 0xFF80
        for tau, mp, tp in ((1.0, 0.0, 0.8), (0.6, 0.05, 0.7)):
            run(xx, dtype, hist, parent, draft, window=64, penalty=1.3, temperature=tau, min_p=mp, top_p=tp,
                u=u, label=f"top-p V={V} {dtype} tau={tau} min_p={mp} top_p={tp}")


def test_top_p_same_tokens_on_every_call():
    """The top-p path lists the crossing bin's tokens in the order their slot
    reservations land, but adds their weights as integers: ten calls on the
    same rows (fp32 and bf16, with and without min-p) give the same tokens."""
    for dtype, min_p in (("f32", 0.0), ("bf16", 0.05)):
        c = inputs.make_sample(dtype=dtype, seed=43)
        kw = dict(hist=_i32(c.hist), parent=_i32(c.parent), draft_tok=_i32(c.draft_tok), window=inputs.PENALTY_WINDOW,
                  penalty=inputs.PENALTY, temperature=0.8, min_p=min_p, top_p=0.9, u=to_dev(c.u, "f32"))
        x = to_dev(c.logits, dtype)
        first = ops.sample_tokens(x, **kw).cpu()
        for _ in range(9):
            assert torch.equal(ops.sample_tokens(x, **kw).cpu(), first), f"{dtype} min_p={min_p}"
        say(f"  top-p {dtype} min_p={min_p}: 10 calls, identical tokens {first[:6].tolist()}...")
