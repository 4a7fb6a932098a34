"""Pins of the alignment oracle against what the pages and mathematics fix.

Each check is independent of the oracle's own code path: hand-worked fixtures,
closed forms, a library stable sort, and a brute-force second formulation
(a Python stable sort of (id, slot) pairs plus a pairwise rank count).
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "align_worked_examples.json")


def _second_formulation(ids, E, BS):
    """Tables from a different construction: a stable sort of (id, slot) pairs
    for the order, and the pages' pairwise rank (#earlier slots with the same id)
    for the within-expert position."""
    n = len(ids)
    valid = [i for i in range(n) if 0 <= ids[i] < E]
    order = sorted(valid, key=lambda i: (ids[i], i))
    counts = [sum(1 for i in valid if ids[i] == e) for e in range(E)]
    padded = [-(-c // BS) * BS for c in counts]
    offsets = [0]
    for p in padded:
        offsets.append(offsets[-1] + p)
    bound = min(n * BS, n + E * (BS - 1))
    mt = -(-bound // BS) * BS
    table = [n] * mt
    perm = [-1] * n
    for i in valid:
        rank = sum(1 for j in range(i) if ids[j] == ids[i])
        table[offsets[ids[i]] + rank] = i
        perm[i] = offsets[ids[i]] + rank
    # the order within each segment must be the stable sort's order
    seg = [i for e in range(E) for i in table[offsets[e]:offsets[e] + counts[e]]]
    assert seg == order
    blocks = []
    for b in range(mt // BS):
        owner = [e for e in range(E) if offsets[e] <= b * BS < offsets[e + 1]]
        blocks.append(owner[0] if owner else -1)
    active = [e for e in range(E) if counts[e] > 0]
    active += [-1] * (min(n, E) - len(active))
    return dict(expert_counts=counts, expert_offsets=offsets, total=offsets[-1],
                max_total=mt, sorted_token_ids=table, block_expert_ids=blocks,
                token_to_perm=perm, active_experts=active, active_count=sum(c > 0 for c in counts))


def _check_equal(got, want):
    for key, val in want.items():
        g = got[key]
        if isinstance(val, list):
            assert list(np.asarray(g).tolist()) == val, key
        else:
            assert int(g) == int(val), key


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    got = oracle.align(np.array(case["topk_ids"], dtype=np.int64), case["E"], case["BS"])
    want = {k: v for k, v in case.items() if k not in ("name", "derivation", "E", "BS", "topk_ids")}
    _check_equal(got, want)


def test_brute_force_tiny():
    """Every id vector over {-1, 0..E} (one invalid id on each side) for E<=3,
    n<=6 and BS in 1..5."""
    checked = 0
    for E in (1, 2, 3):
        for n in range(1, 7):
            for ids in itertools.product(range(-1, E + 1), repeat=n):
                for BS in (1, 2, 3, 4, 5):
                    got = oracle.align(np.array(ids, dtype=np.int64), E, BS)
                    _check_equal(got, _second_formulation(list(ids), E, BS))
                    checked += 1
    assert checked == 5 * sum((E + 2) ** n for E in (1, 2, 3) for n in range(1, 7))


def test_bs1_is_library_stable_argsort():
    rng = np.random.default_rng(7)
    for E in (1, 5, 64):
        ids = rng.integers(-2, E + 2, size=300)
        t = oracle.align(ids, E, 1)
        valid = ids[(ids >= 0) & (ids < E)]
        keep = np.flatnonzero((ids >= 0) & (ids < E))
        lib = keep[np.argsort(valid, kind="stable")]
        assert t["total"] == valid.size
        assert np.array_equal(t["sorted_token_ids"][: t["total"]], lib)


@pytest.mark.parametrize("seed", range(6))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 300))
    BS = int(rng.choice([1, 2, 3, 16, 64]))
    n = int(rng.integers(1, 2000))
    ids = rng.integers(-1, E + 1, size=n)
    t = oracle.align(ids, E, BS)
    valid = (ids >= 0) & (ids < E)
    c = t["expert_counts"]
    # conservation
    assert c.sum() == valid.sum()
    # closed-form total, multiple of BS, within the worst case
    assert t["total"] == sum(-(-int(x) // BS) * BS for x in c)
    assert t["total"] % BS == 0 and t["total"] <= t["max_total"]
    # identity of the worst case: n + min(n, E)*(BS-1), rounded up to BS
    assert t["max_total"] == -(-(n + min(n, E) * (BS - 1)) // BS) * BS
    # segments: [off, off+count) hold expert e's slots ascending, then sentinels
    off = t["expert_offsets"]
    st = t["sorted_token_ids"]
    for e in range(E):
        seg = st[off[e]:off[e] + c[e]]
        assert np.all(ids[seg] == e)
        assert np.all(np.diff(seg) > 0)
        assert np.all(st[off[e] + c[e]:off[e + 1]] == n)
    assert np.all(st[t["total"]:] == n)
    # mutual inverse on valid slots
    perm = t["token_to_perm"]
    assert np.all(perm[~valid] == -1)
    assert np.array_equal(st[perm[valid]], np.flatnonzero(valid))
    # active list strictly ascending, equal to the experts with a slot, within the cap
    a = t["active_experts"][: t["active_count"]]
    assert np.array_equal(a, np.flatnonzero(c > 0))
    assert np.all(t["active_experts"][t["active_count"]:] == -1)
    assert t["active_experts"].size == min(n, E)
    # blocks: owner covers the block start
    for b, e in enumerate(t["block_expert_ids"]):
        if b * BS < t["total"]:
            assert off[e] <= b * BS < off[e + 1]
        else:
            assert e == -1


def test_bound_attained_when_distinct():
    for E, n, BS in ((8, 8, 16), (128, 64, 16), (5, 3, 7)):
        ids = np.random.default_rng(n).permutation(E)[:n]
        t = oracle.align(ids, E, BS)
        assert t["total"] == n * BS == t["max_total"]


def test_dtype_independent():
    ids = np.random.default_rng(3).integers(0, 40, size=(50, 4))
    a = oracle.align(ids.astype(np.int64), 40, 8)
    b = oracle.align(ids.astype(np.int32), 40, 8)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k]))


def test_max_total_and_cap_formulas():
    # the page's worst case: min(n*BS, n+E*(BS-1)) rounded up to BS
    assert oracle.max_total(8, 128, 16) == 128
    assert oracle.max_total(64, 128, 16) == 1024
    assert oracle.max_total(1024, 128, 16) == 2944
    assert oracle.max_total(32768, 256, 64) == 48896
    assert oracle.max_total(512, 256, 64) == 16640
    assert oracle.max_total(5, 2, 4) == 12
    assert oracle.active_cap(64, 128) == 64
    assert oracle.active_cap(32768, 256) == 256
