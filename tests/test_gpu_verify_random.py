"""GPU parity of ts_tree_verify_attn against the CPU oracle over a seeded
random sweep of shapes, so that the combinations the named cases do not pin
(draft count x grouped heads x head_dim x cache length x split count x dtype)
still meet the contract. The shapes reach every kernel form: the wave-per-split
kernel (at most 16 grouped rows per KV head), the 128-row and 256-row
matrix-core kernels with one to several row groups, and the fp32 vector-ALU
kernel; cache lengths are ragged and include the empty cache. Each case is
small enough for the oracle to finish within a second or two."""
import numpy as np
import pytest

from long_context_kv_ts_amd import inputs, ops
import oracle
from gpu_util import check_attn, say, to_dev
import torch

pytestmark = pytest.mark.gpu


def _random_forest(rng, T):
    """A forest whose nodes have parents among the previous 12 nodes (or none),
    so that chains, trees and roots mix."""
    return np.array([-1 if t == 0 or rng.random() < 0.15 else int(rng.integers(max(0, t - 12), t))
                     for t in range(T)], np.int32)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    dtype = "f32" if i % 6 == 5 else "bf16"
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    # draft counts per kernel form: <= 16 rows, <= 128 rows, several row groups
    form = i % 3
    if form == 0:
        T = int(rng.integers(1, max(2, 16 // G + 1)))
    elif form == 1:
        T = int(rng.integers(max(1, 17 // G), max(2, 128 // G + 1)))
    else:
        T = int(rng.integers(max(1, 129 // G), max(2, 600 // G + 1)))
    T = min(T, 300)
    L = int(rng.choice([0, 1, 33, int(rng.integers(100, 3000)), int(rng.integers(3000, 9000)),
                        64 * int(rng.integers(2, 140))]))
    splits = int(rng.choice([0, 0, 1, 3, 7]))
    return dict(dtype=dtype, D=D, Hkv=Hkv, Hq=Hkv * G, T=T, L=L, splits=splits, seed=2000 + i)


CASES = [_case(i) for i in range(30)]


@pytest.mark.parametrize("case", CASES, ids=[f"{c['dtype']}-T{c['T']}-G{c['Hq'] // c['Hkv']}-Hkv{c['Hkv']}-D{c['D']}-"
                                              f"L{c['L']}-S{c['splits']}" for c in CASES])
def test_random_shapes(case):
    say(f"[random] {case}")
    rng = np.random.default_rng(case["seed"])
    parent = _random_forest(rng, case["T"])
    c = inputs.make_verify("random", dtype=case["dtype"], Hq=case["Hq"], Hkv=case["Hkv"], D=case["D"], L=case["L"],
                           seed=case["seed"], with_chains=False, parent=parent)
    ro, rl = oracle.verify_attn_ref(c.q, c.k_cache, c.v_cache, c.k_draft, c.v_draft, c.parent, c.scale, c.dtype)
    dt = c.dtype
    out, lse = ops.tree_verify_attn(to_dev(c.q, dt), to_dev(c.k_cache, dt), to_dev(c.v_cache, dt),
                                    to_dev(c.k_draft, dt), to_dev(c.v_draft, dt), to_dev(c.parent, "i32"),
                                    scale=c.scale, num_splits=case["splits"])
    torch.cuda.synchronize()
    check_attn(out, lse, ro, rl, dt, str(case))
