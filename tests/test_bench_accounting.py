"""CPU: the benchmark's accounting of credited work.

`bench.visible_pairs` counts the (query, key) pairs a layer's mask leaves
visible, the quantity every credited FLOP figure rests on.  It is checked
against a pair-by-pair count from the mask's definition (keys in the query's
document; causal: key <= query; window: query - key <= left and
key - query <= right when those are >= 0) on random document sets, and against
closed forms; the S=131072 workload's per-launch dK/dV figure is checked
against its closed form."""
import random

import pytest

import bench
from ulysses_inputs import WORKLOADS


def _brute(docs, causal, wl, wr):
    n = 0
    for L in docs:
        for i in range(L):
            for j in range(L):
                if causal and j > i:
                    continue
                if wl >= 0 and i - j > wl:
                    continue
                if wr >= 0 and j - i > wr:
                    continue
                n += 1
    return n


@pytest.mark.parametrize("seed", range(6))
def test_visible_pairs_match_pair_by_pair_count(seed):
    rnd = random.Random(seed)
    docs = [rnd.randint(1, 90) for _ in range(rnd.randint(1, 4))]
    for causal in (False, True):
        for wl in (-1, 0, 3, 17, 200):
            for wr in (-1, 0, 5, 40):
                assert bench.visible_pairs(docs, causal, wl, wr) == _brute(docs, causal, wl, wr), \
                    (docs, causal, wl, wr)


def test_visible_pairs_closed_forms():
    L = 4097
    assert bench.visible_pairs([L], False, -1, -1) == L * L
    assert bench.visible_pairs([L], True, -1, -1) == L * (L + 1) // 2
    # a causal window of W keys (the query included): min(t + 1, W) keys for query t
    W = 128
    assert bench.visible_pairs([L], True, W - 1, -1) == W * (W + 1) // 2 + (L - W) * W
    # documents are independent
    assert bench.visible_pairs([100, 200], True, -1, -1) == 100 * 101 // 2 + 200 * 201 // 2


def test_s131072_dkdv_credit_per_launch():
    """One rank call of the S=131072 causal layer: 7 query heads, 6*D FLOPs per
    visible pair credited to dK/dV (dP, dV, dK), 12*D to the whole step."""
    case = WORKLOADS[5]
    credit = bench.kernel_credit(case, [case.S] * case.B)  # one sequence per batch row
    S, D, hq = case.S, case.D, case.hq
    pairs = hq * S * (S + 1) // 2
    (layer,) = credit.values()
    assert layer["pairs"] == pairs
    assert layer["attn_bwd_dkdv"] == 6 * D * pairs == 46179840688128
    assert layer["attn_fwd"] + layer["attn_bwd_dkdv"] + layer["attn_bwd_dq"] == 12 * D * pairs


def test_host_cpu_counts():
    c = bench.host_cpus()
    assert c["logical_cpus"] >= 1
    assert 1 <= c.get("usable_cpus", 1) <= c["logical_cpus"]
    assert 1 <= c.get("physical_cores", 1) <= c["logical_cpus"]


@pytest.mark.parametrize("seed", range(4))
def test_visible_counts_per_row_and_key(seed):
    """The CPU baseline credits its sampled rows and keys with these counts."""
    rnd = random.Random(100 + seed)
    docs = [rnd.randint(1, 60) for _ in range(rnd.randint(1, 3))]
    T = sum(docs)
    doc_of = [d for d, L in enumerate(docs) for _ in range(L)]
    idx = sorted(rnd.sample(range(T), min(T, 12)))
    for causal in (False, True):
        for wl, wr in ((-1, -1), (4, -1), (9, 3), (-1, 2)):
            def vis(i, j):
                if doc_of[i] != doc_of[j]:
                    return False
                if causal and j > i:
                    return False
                if wl >= 0 and i - j > wl:
                    return False
                return not (wr >= 0 and j - i > wr)
            rows = bench._visible_counts(docs, T, causal, wl, wr, idx, False)
            keys = bench._visible_counts(docs, T, causal, wl, wr, idx, True)
            assert rows == [sum(vis(i, j) for j in range(T)) for i in idx], (docs, causal, wl, wr)
            assert keys == [sum(vis(i, j) for i in range(T)) for j in idx], (docs, causal, wl, wr)
