"""GPU parity of the 4-gram table (ts_ngram_init / _update / _retrieve)
against the oracle: bit-exact 4-grams, counts, ranking and match count,
with the table grown the way generation grows it (a prefill, then a few
tokens per verification), plus repetitive texts, absent first tokens and an
overfull table."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV, say, to_dev
from long_context_kv_ts_amd import inputs, ops
from oracle import ngram_table, ngram_update, retrieve_ref

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_example.json")


def check(table, ref_table, firsts, k, label):
    ws = ops.alloc_workspace(int(ops.lib().ts_ngram_retrieve_workspace(table.max_entries, k)), DEV)
    for f in firsts:
        ft = torch.tensor([int(f)], dtype=torch.int32, device=DEV)
        tok, cnt, nf = table.retrieve(ft, k, workspace=ws)
        torch.cuda.synchronize()
        grams, counts, _ = retrieve_ref(ref_table, int(f), k)
        m = len(grams)
        got_t, got_c, got_n = tok.cpu().numpy(), cnt.cpu().numpy(), int(nf.item())
        assert got_n == m, f"{label} first={f}: n_found {got_n} != {m}"
        assert np.array_equal(got_t[:m], grams) and (got_t[m:] == -1).all(), f"{label} first={f}: 4-grams"
        assert np.array_equal(got_c[:m], counts) and (got_c[m:] == 0).all(), f"{label} first={f}: counts"


def test_hand_worked_example():
    ex = json.load(open(GOLDEN))
    t = ops.NgramTable(DEV, capacity_log2=6, max_entries=64)
    toks = to_dev(np.array(ex["tokens"], np.int32), "i32")
    t.update(toks, 0, len(ex["tokens"]))
    h = t.header()
    assert h["n_entries"] == ex["distinct"] and h["dropped"] == 0
    for q in ex["queries"]:
        tok, cnt, nf = t.retrieve(torch.tensor([q["first"]], dtype=torch.int32, device=DEV), q["k"])
        m = len(q["grams"])
        assert int(nf.item()) == m
        assert tok.cpu().numpy()[:m].tolist() == q["grams"] and cnt.cpu().numpy()[:m].tolist() == q["counts"]


def test_generation_like_growth_100k():
    """A 4096-token prefill, then 1-6 tokens per step for 2000 steps, then the
    rest of a 102,400-token text in one update; retrieval of the 20 best for
    frequent, rare and absent first tokens at three points."""
    text = inputs.make_text(102400)
    tokens = to_dev(text, "i32")
    t = ops.NgramTable(DEV, capacity_log2=18, max_entries=131072)
    ref = {}
    rng = np.random.default_rng(3)
    n0 = 0
    plan = [4096] + list(4096 + np.cumsum(rng.integers(1, 7, 2000)))
    for i, n1 in enumerate(plan + [len(text)]):
        t.update(tokens, n0, int(n1))
        ngram_update(ref, text, n0, int(n1))
        n0 = int(n1)
        if i in (0, len(plan) - 1, len(plan)):
            torch.cuda.synchronize()
            h = t.header()
            assert h["n_entries"] == len(ref) and h["dropped"] == 0, (h, len(ref))
            freq = np.bincount(text[:n0]).argsort()[::-1]
            firsts = list(freq[:12]) + list(freq[200:204]) + [int(text[n0 - 1]), 128255]
            check(t, ref, firsts, 20, f"n={n0}")
            say(f"  n={n0}: {len(ref)} distinct 4-grams")
    check(t, ref, [0, 1, 2], 64, "k=64")
    check(t, ref, [0, 5], 1, "k=1")


@pytest.mark.parametrize("pattern", ["constant", "period2", "period5"])
def test_repetitive_texts(pattern):
    """Every chunk of 1024 positions repeats the same few 4-grams: the chunk's
    multiplicity and last position carry the counts."""
    n = 5000
    base = {"constant": [7], "period2": [3, 9], "period5": [1, 2, 3, 4, 5]}[pattern]
    text = np.array((base * (n // len(base) + 1))[:n], np.int32)
    t = ops.NgramTable(DEV, capacity_log2=8, max_entries=64)
    tokens = to_dev(text, "i32")
    t.update(tokens, 0, 1500)
    t.update(tokens, 1500, n)
    ref = ngram_table(text)
    assert t.header()["n_entries"] == len(ref)
    check(t, ref, sorted(set(base)) + [0], 20, pattern)


def test_noop_updates_reset_and_absent():
    t = ops.NgramTable(DEV, capacity_log2=8, max_entries=200)
    text = np.arange(50, dtype=np.int32) % 11
    tokens = to_dev(text, "i32")
    t.update(tokens, 0, 3)                       # no 4-gram ends before position 3
    t.update(tokens, 10, 10)
    assert t.header()["n_entries"] == 0
    t.update(tokens, 0, 50)
    check(t, ngram_table(text), [0, 4, 10, 11, 99], 20, "period 11")
    t.reset()
    assert t.header()["n_entries"] == 0
    check(t, {}, [0, 4], 20, "after reset")


def test_overfull_table_reports_drops():
    """More distinct 4-grams than entries: the header counts the ones that found
    no room, and every 4-gram that is returned carries its exact count, in
    ranking order."""
    text = inputs.make_text(20000, V=300, copy_prob=0.0, seed=9)
    t = ops.NgramTable(DEV, capacity_log2=12, max_entries=1000)
    tokens = to_dev(text, "i32")
    for a in range(0, 20000, 2500):
        t.update(tokens, a, a + 2500)
    ref = ngram_table(text)
    h = t.header()
    assert h["dropped"] > 0 and min(h["n_entries"], 1000) == 1000
    for f in (0, 1, 2, 3):
        tok, cnt, nf = t.retrieve(torch.tensor([f], dtype=torch.int32, device=DEV), 64)
        m = int(nf.item())
        got = [tuple(r) for r in tok.cpu().numpy()[:m].tolist()]
        keys = [(ref[g][0], ref[g][1]) for g in got]
        assert all(g[0] == f for g in got)
        assert cnt.cpu().numpy()[:m].tolist() == [k[0] for k in keys]
        assert keys == sorted(keys, reverse=True)
