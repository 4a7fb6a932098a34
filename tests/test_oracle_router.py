"""Pins of the router oracle.

Independent checks: brute force over every k-subset on tiny inputs, the full
softmax renormalised over the chosen experts (a second way to the weights),
exact integer arithmetic and one-hot gate rows for the logits, shift
invariance, ties, and the workload generator's own routing recipe (softmax
over N(0,1) logits, stable top-k, renormalised), which is separate code.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads
from workloads import bf16_bits_from_f32
from workloads.gen import _TAG_LOGITS, _rng


def _brute_topk(row, k):
    """The unique k-subset every member of which beats every non-member
    (larger logit, or equal logit and lower index), ordered the same way."""
    E = len(row)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)  # noqa: E731
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [f for f in range(E) if f not in S]
        if all(beats(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    S = found[0]
    return sorted(S, key=lambda a: sum(beats(b, a) for b in S))  # rank = members that beat it


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    E, k = 7, 3
    logits = rng.integers(-3, 4, size=(12, E)).astype(np.float64)  # many ties
    ids, w = oracle.topk_softmax(logits, k)
    for t in range(logits.shape[0]):
        S = _brute_topk(list(logits[t]), k)
        assert list(ids[t]) == S
        e = np.exp(logits[t, S])
        assert np.allclose(w[t], e / e.sum(), rtol=1e-15, atol=0)


def test_weights_are_the_renormalised_full_softmax():
    rng = np.random.default_rng(11)
    logits = rng.normal(0, 2, size=(20, 32))
    ids, w = oracle.topk_softmax(logits, 6)
    p = np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)
    chosen = np.take_along_axis(p, ids, axis=1)
    assert np.allclose(w, chosen / chosen.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)  # larger logits first, so weights do not grow


def test_shift_invariance_and_ties():
    rng = np.random.default_rng(12)
    logits = rng.normal(size=(9, 16))
    ids, w = oracle.topk_softmax(logits, 4)
    ids2, w2 = oracle.topk_softmax(logits + 37.25, 4)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w, w2, rtol=1e-12, atol=0)
    ids3, w3 = oracle.topk_softmax(np.zeros((3, 10)), 4)
    assert np.array_equal(ids3, np.tile(np.arange(4), (3, 1)))
    assert np.array_equal(w3, np.full((3, 4), 0.25))


def test_top_k_equal_to_e_is_a_sorted_full_softmax():
    logits = np.array([[0.5, -1.0, 2.0, 2.0, 0.0]])
    ids, w = oracle.topk_softmax(logits, 5)
    assert list(ids[0]) == [2, 3, 0, 4, 1]
    p = np.exp(logits[0]) / np.exp(logits[0]).sum()
    assert np.allclose(w[0], p[ids[0]], rtol=1e-15)


@pytest.mark.parametrize("name", ["decode", "verify", "tiny"])
def test_matches_the_workload_routing_recipe(name):
    """The configs' routings are softmax top-k of seeded logits, renormalised;
    the oracle on those logits gives the same ids and weights."""
    cfg = workloads.CONFIGS[name]
    logits = _rng(cfg, _TAG_LOGITS).standard_normal((cfg.M, cfg.E))
    if cfg.routing == "softmax_bias":
        from workloads.gen import _TAG_BIAS
        logits = logits + _rng(cfg, _TAG_BIAS).normal(0.0, cfg.bias_std, size=cfg.E)[None, :]
    ids, w = workloads.routing(cfg)
    o_ids, o_w = oracle.topk_softmax(logits, cfg.top_k)
    assert np.array_equal(ids, o_ids)
    assert np.allclose(w, o_w, rtol=1e-6, atol=0)


def test_logits_exact_integers():
    """Small integers are exact in bf16 and their dot products are exact in
    float64: compare with Python integer arithmetic."""
    rng = np.random.default_rng(13)
    M, E, H = 5, 7, 40
    xi = rng.integers(-8, 9, size=(M, H))
    wi = rng.integers(-8, 9, size=(E, H))
    x = bf16_bits_from_f32(xi.astype(np.float32))
    w = bf16_bits_from_f32(wi.astype(np.float32))
    got = oracle.router_logits(x, w)
    for t in range(M):
        for e in range(E):
            assert got[t, e] == sum(int(a) * int(b) for a, b in zip(xi[t], wi[e]))


def test_logits_one_hot_rows_pick_columns():
    rng = np.random.default_rng(14)
    M, E, H = 4, 6, 24
    x = bf16_bits_from_f32(rng.normal(size=(M, H)).astype(np.float32))
    cols = [3, 0, 23, 3, 11, 7]
    wf = np.zeros((E, H), dtype=np.float32)
    wf[np.arange(E), cols] = 1.0
    got = oracle.router_logits(x, bf16_bits_from_f32(wf))
    assert np.array_equal(got, oracle.bf16_to_f64(x)[:, cols])
