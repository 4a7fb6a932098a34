"""Pins of the FFN/blend oracle.

Independent checks: torch's float8_e4m3fn and bfloat16 decodes (library),
a per-token dense evaluation with torch float64 ops (the layer is a dense
per-token sum over the token's top-k experts plus the shared expert), exact
integer arithmetic, closed forms of SiLU, and the special cases where a term
must vanish.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import bf16_bits_from_f32


def _torch_dequant(bits, scales, wdt):
    if wdt == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
    w = torch.from_numpy(bits).view(torch.float8_e4m3fn).double()
    s = torch.from_numpy(scales).double()
    return w * torch.kron(s, torch.ones(128, 128, dtype=torch.float64))


def _rand_fp8(rng, N, K):
    codes = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38     # no NaN codes in weights
    scales = rng.uniform(0.001, 0.01, size=(N // 128, K // 128)).astype(np.float32)
    return codes, scales


def _rand_bf16(rng, N, K, std=0.1):
    return bf16_bits_from_f32(rng.normal(0, std, size=(N, K)).astype(np.float32)), None


def test_dequant_matches_torch_float8():
    rng = np.random.default_rng(0)
    codes, scales = _rand_fp8(rng, 256, 384)
    ours = oracle.dequant(codes, scales, "fp8")
    ref = _torch_dequant(codes, scales, "fp8").numpy()
    assert np.array_equal(ours, ref)


def test_dequant_block_locality():
    rng = np.random.default_rng(1)
    codes, scales = _rand_fp8(rng, 256, 256)
    base = oracle.dequant(codes, scales, "fp8")
    s2 = scales.copy()
    s2[1, 0] *= 2
    moved = oracle.dequant(codes, s2, "fp8")
    diff = moved != base
    blk = np.zeros_like(diff)
    blk[128:256, 0:128] = True
    assert not np.any(diff & ~blk)
    assert np.array_equal(moved[128:, :128], 2 * base[128:, :128])


def test_bf16_dequant_matches_torch():
    rng = np.random.default_rng(2)
    bits, _ = _rand_bf16(rng, 32, 48)
    assert np.array_equal(oracle.dequant(bits, None, "bf16"), _torch_dequant(bits, None, "bf16").numpy())


def test_silu_closed_form():
    g = np.array([-3.0, -1.0, 0.0, 0.5, 2.0])
    want = [x / (1 + math.exp(-x)) for x in g]
    assert np.allclose(oracle.silu(g), want, rtol=1e-15, atol=0)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # torch's SiLU, a library routine
    assert np.allclose(oracle.silu(g), F.silu(torch.from_numpy(g)).numpy(), rtol=1e-15, atol=1e-300)


def test_expert_ffn_exact_integers():
    """Integer activations and weights: the two projections are exact, and the
    orientation (W is [out, in]) is fixed by non-square shapes."""
    rng = np.random.default_rng(3)
    r, H, I = 3, 7, 5
    x = rng.integers(-4, 5, size=(r, H)).astype(np.float64)
    Wg = rng.integers(-3, 4, size=(I, H)).astype(np.float64)
    Wu = rng.integers(-3, 4, size=(I, H)).astype(np.float64)
    Wd = rng.integers(-3, 4, size=(H, I)).astype(np.float64)
    act, y = oracle.expert_ffn(x, Wg, Wu, Wd)
    for a in range(r):
        for i in range(I):
            g = sum(int(x[a, h]) * int(Wg[i, h]) for h in range(H))
            u = sum(int(x[a, h]) * int(Wu[i, h]) for h in range(H))
            want = g / (1 + math.exp(-g)) * u
            assert act[a, i] == pytest.approx(want, rel=1e-14, abs=1e-300)
    assert y.shape == (r, H)
    assert np.allclose(y, act @ Wd.T, rtol=0, atol=0)


def _dense_reference(x_bits, ids, w, E, wdt, routed, shared):
    """Per token: sum_k w[t,k] * MLP_{ids[t,k]}(x_t) + MLP_shared(x_t), torch float64."""
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double()
    M, top_k = ids.shape
    out = torch.zeros(M, x.shape[1], dtype=torch.float64)

    def mlp(m, xt):
        Wg = _torch_dequant(*m("gate"), wdt)
        Wu = _torch_dequant(*m("up"), wdt)
        Wd = _torch_dequant(*m("down"), wdt)
        return torch.mv(Wd, F.silu(torch.mv(Wg, xt)) * torch.mv(Wu, xt))

    for t in range(M):
        for k in range(top_k):
            e = int(ids[t, k])
            if 0 <= e < E:
                out[t] += float(w[t, k]) * mlp(lambda which: routed(which, e), x[t])
        if shared is not None:
            out[t] += mlp(shared, x[t])
    return out.numpy()


def _make_model(rng, E, H, I, S, wdt):
    mk = _rand_fp8 if wdt == "fp8" else _rand_bf16
    mats = {(which, e): mk(rng, *((I, H) if which != "down" else (H, I)))
            for e in range(E) for which in ("gate", "up", "down")}
    sh = None
    if S:
        shm = {which: mk(rng, *((S, H) if which != "down" else (H, S))) for which in ("gate", "up", "down")}
        sh = lambda which: shm[which]  # noqa: E731
    return (lambda which, e: mats[(which, e)]), sh


@pytest.mark.parametrize("wdt,E,H,I,S,M,top_k,BS", [
    ("bf16", 1, 24, 40, 0, 3, 1, 4),       # dense special case: one expert, top-1
    ("bf16", 3, 16, 8, 12, 5, 2, 4),       # shared expert of another width
    ("fp8", 4, 256, 128, 0, 6, 2, 16),
    ("fp8", 3, 128, 256, 128, 4, 3, 8),
])
def test_layer_equals_dense_per_token_sum(wdt, E, H, I, S, M, top_k, BS):
    rng = np.random.default_rng(10 + E + H)
    routed, shared = _make_model(rng, E, H, I, S, wdt)
    x_bits = bf16_bits_from_f32(rng.normal(0, 1, size=(M, H)).astype(np.float32))
    ids = np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int64)
    w = rng.uniform(0.1, 1.0, size=(M, top_k)).astype(np.float32)
    if E == 1:
        w[:] = 1.0
    got = oracle.moe_layer(x_bits, ids, w, E, BS, wdt, routed, shared)["out"]
    ref = _dense_reference(x_bits, ids, w, E, wdt, routed, shared)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_out_of_range_slots_add_nothing():
    rng = np.random.default_rng(20)
    E, H, I, M, top_k = 3, 16, 8, 4, 2
    routed, _ = _make_model(rng, E, H, I, 0, "bf16")
    x_bits = bf16_bits_from_f32(rng.normal(0, 1, size=(M, H)).astype(np.float32))
    ids = np.array([[0, 1], [2, -1], [E, 1], [0, 2]], dtype=np.int64)
    w = rng.uniform(0.1, 1.0, size=(M, top_k)).astype(np.float32)
    got = oracle.moe_layer(x_bits, ids, w, E, 4, "bf16", routed)["out"]
    # same routing with the bad slots pointed at expert 0 but given weight 0
    ids2, w2 = ids.copy(), w.copy()
    bad = (ids < 0) | (ids >= E)
    ids2[bad] = 0
    w2[bad] = 0.0
    ref = oracle.moe_layer(x_bits, ids2, w2, E, 4, "bf16", routed)["out"]
    assert np.array_equal(got, ref)


def test_zero_gate_leaves_shared_only():
    rng = np.random.default_rng(21)
    E, H, I, S, M = 2, 16, 8, 8, 3
    routed, shared = _make_model(rng, E, H, I, S, "bf16")
    zero = (np.zeros((I, H), dtype=np.uint16), None)
    routed0 = lambda which, e: zero if which == "gate" else routed(which, e)  # noqa: E731
    x_bits = bf16_bits_from_f32(rng.normal(0, 1, size=(M, H)).astype(np.float32))
    ids = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int64)
    w = np.full((M, 2), 0.5, dtype=np.float32)
    res = oracle.moe_layer(x_bits, ids, w, E, 4, "bf16", routed0, shared)
    assert np.array_equal(res["out"], res["sh_out"])
    assert all(np.all(a == 0) for a in res["act_pos"].values())


def test_closed_form_example():
    """Two tokens, two experts, top-2, H=2, I=1, values exact in bf16; the
    expected outputs are written with the SiLU closed form g/(1+e^-g)."""
    def b(v):
        return bf16_bits_from_f32(np.array(v, dtype=np.float32))
    mats = {
        ("gate", 0): b([[1, 0]]), ("up", 0): b([[0, 1]]), ("down", 0): b([[1], [-1]]),
        ("gate", 1): b([[0, 1]]), ("up", 1): b([[1, 1]]), ("down", 1): b([[2], [0.5]]),
    }
    routed = lambda which, e: (mats[(which, e)], None)  # noqa: E731
    x = b([[1, 2], [-1, 0.5]])
    ids = np.array([[1, 0], [0, 1]], dtype=np.int64)
    w = np.array([[0.75, 0.25], [0.5, 0.5]], dtype=np.float32)
    s = lambda g: g / (1 + math.exp(-g))  # noqa: E731
    a01 = s(2) * 3          # token 0, expert 1: g = 2, u = 3
    a00 = s(1) * 2          # token 0, expert 0: g = 1, u = 2
    a10 = s(-1) * 0.5       # token 1, expert 0: g = -1, u = 0.5
    a11 = s(0.5) * -0.5     # token 1, expert 1: g = 0.5, u = -0.5
    want = np.array([
        [0.75 * 2 * a01 + 0.25 * a00, 0.75 * 0.5 * a01 - 0.25 * a00],
        [0.5 * a10 + 0.5 * 2 * a11, -0.5 * a10 + 0.5 * 0.5 * a11],
    ])
    got = oracle.moe_layer(x, ids, w, 2, 2, "bf16", routed)["out"]
    assert np.allclose(got, want, rtol=1e-15, atol=1e-15)


def test_blend_special_cases():
    rng = np.random.default_rng(22)
    M, top_k, H = 5, 3, 8
    rows = rng.normal(size=(M * top_k + 4, H))
    perm = rng.permutation(M * top_k + 4)[: M * top_k]
    w = rng.uniform(0.1, 1, size=(M, top_k)).astype(np.float32)
    base = oracle.blend(rows, w, perm, None)
    # doubling every weight doubles the output exactly
    assert np.array_equal(oracle.blend(rows, 2 * w, perm, None), 2 * base)
    # top-1 with weight 1 and no shared expert copies the slot's row
    one = oracle.blend(rows, np.ones((M, 1), np.float32), perm[:M], None)
    assert np.array_equal(one, rows[perm[:M]])
    # a dropped slot (-1) adds nothing; the shared output adds once
    p2 = perm.copy()
    p2[1] = -1
    sh = rng.normal(size=(M, H))
    got = oracle.blend(rows, w, p2, sh)
    want0 = w[0, 0] * rows[perm[0]].astype(np.float64) + w[0, 2] * rows[perm[2]] + sh[0]
    assert np.allclose(got[0], want0, rtol=1e-15, atol=0)


def test_intermediates_keyed_by_sorted_position():
    rng = np.random.default_rng(23)
    E, H, I, M, top_k, BS = 4, 16, 8, 6, 2, 4
    routed, _ = _make_model(rng, E, H, I, 0, "bf16")
    x_bits = bf16_bits_from_f32(rng.normal(0, 1, size=(M, H)).astype(np.float32))
    ids = np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int64)
    w = np.full((M, top_k), 0.5, np.float32)
    res = oracle.moe_layer(x_bits, ids, w, E, BS, "bf16", routed)
    t = res["tables"]
    valid_pos = set(int(p) for p in t["token_to_perm"] if p >= 0)
    assert set(res["act_pos"]) == valid_pos == set(res["y_pos"])
    # the row at position p is slot sorted_token_ids[p]'s expert output
    x = oracle.bf16_to_f64(x_bits)
    for p in valid_pos:
        i = int(t["sorted_token_ids"][p])
        e = int(ids.reshape(-1)[i])
        Wg, Wu, Wd = (oracle.dequant(*routed(m, e), "bf16") for m in ("gate", "up", "down"))
        act, y = oracle.expert_ffn(x[i // top_k][None], Wg, Wu, Wd)
        assert np.allclose(res["y_pos"][p], y[0], rtol=1e-13, atol=1e-13)


def test_token_subset_matches_full():
    rng = np.random.default_rng(24)
    E, H, I, S, M, top_k = 4, 16, 8, 8, 6, 2
    routed, shared = _make_model(rng, E, H, I, S, "bf16")
    x_bits = bf16_bits_from_f32(rng.normal(0, 1, size=(M, H)).astype(np.float32))
    ids = np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int64)
    w = rng.uniform(0.1, 1, size=(M, top_k)).astype(np.float32)
    full = oracle.moe_layer(x_bits, ids, w, E, 4, "bf16", routed, shared)["out"]
    part = oracle.moe_layer(x_bits, ids, w, E, 4, "bf16", routed, shared, tokens=[4, 1])["out"]
    assert np.allclose(part, full[[4, 1]], rtol=1e-14, atol=1e-14)


# ------------------------------------------------------- gated shared expert --

def test_shared_gate_special_values_and_symmetry():
    rng = np.random.default_rng(21)
    M, H = 6, 64
    x = bf16_bits_from_f32(rng.normal(size=(M, H)).astype(np.float32))
    zero = bf16_bits_from_f32(np.zeros(H, dtype=np.float32))
    assert np.array_equal(oracle.shared_gate(x, zero), np.full(M, 0.5))
    g = bf16_bits_from_f32(rng.normal(0, 0.2, size=H).astype(np.float32))
    neg = bf16_bits_from_f32(-oracle.bf16_to_f64(g).astype(np.float32))
    assert np.allclose(oracle.shared_gate(x, g) + oracle.shared_gate(x, neg), 1.0, rtol=0, atol=1e-15)
    big = bf16_bits_from_f32(np.full(H, 64.0, dtype=np.float32))
    ones = bf16_bits_from_f32(np.ones((1, H), dtype=np.float32))
    assert oracle.shared_gate(ones, big)[0] == 1.0
    assert oracle.shared_gate(ones, bf16_bits_from_f32(np.full(H, -64.0, dtype=np.float32)))[0] < 1e-300
    ref = torch.sigmoid(torch.from_numpy(oracle.bf16_to_f64(x)) @ torch.from_numpy(oracle.bf16_to_f64(g)))
    assert np.allclose(oracle.shared_gate(x, g), ref.numpy(), rtol=1e-14, atol=0)


def test_blend_gate_scales_only_the_shared_term():
    rng = np.random.default_rng(22)
    M, top_k, E, H = 7, 3, 5, 16
    ids = np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int64)
    w = rng.uniform(0.1, 1, size=(M, top_k)).astype(np.float32)
    t = oracle.align(ids, E, 4)
    eo = rng.normal(size=(int(t["total"]), H))
    sh = rng.normal(size=(M, H))
    gate = rng.uniform(0, 1, size=M)
    plain = oracle.blend(eo, w, t["token_to_perm"], None, H=H)
    gated = oracle.blend(eo, w, t["token_to_perm"], sh, H=H, sh_gate=gate)
    assert np.allclose(gated, plain + gate[:, None] * sh, rtol=1e-14, atol=1e-14)
    assert np.array_equal(oracle.blend(eo, w, t["token_to_perm"], sh, H=H, sh_gate=np.ones(M)),
                          oracle.blend(eo, w, t["token_to_perm"], sh, H=H))


# ------------------------------------------------------- per-row FP8 scales --

def test_dequant_row_scales_match_torch_and_stay_in_their_row():
    rng = np.random.default_rng(31)
    codes, _ = _rand_fp8(rng, 256, 384)
    s = rng.uniform(0.001, 0.01, size=256).astype(np.float32)
    ours = oracle.dequant(codes, s, "fp8_rows")
    ref = (torch.from_numpy(codes).view(torch.float8_e4m3fn).double() * torch.from_numpy(s).double()[:, None])
    assert np.array_equal(ours, ref.numpy())
    s2 = s.copy()
    s2[17] *= 4
    moved = oracle.dequant(codes, s2, "fp8_rows")
    diff = np.any(moved != ours, axis=1)
    assert np.array_equal(np.flatnonzero(diff), [17]) or not np.any(codes[17] & 0x7F)
    assert np.array_equal(moved[17], 4 * ours[17])


def test_row_scaled_generator_fills_each_row_to_448():
    """The fp8_rows workload: every row's largest code is 448 (its row scale is
    the row's amax / 448) and no dequantised value leaves the draw range
    [-1/sqrt(K), 1/sqrt(K)]."""
    import workloads
    cfg = workloads.MoeConfig("rows", 2, 256, 2, 1, 128, 0, 16, "fp8_rows", "softmax", seed=5)
    bits, sc = workloads.expert_matrix(cfg, "gate", 0)
    assert sc.shape == (cfg.I,)
    w = oracle.dequant(bits, sc, "fp8_rows")
    assert np.allclose(np.abs(w).max(axis=1), 448.0 * sc, rtol=1e-7)
    bound = 1.0 / np.sqrt(cfg.H)
    assert np.all(np.abs(w) <= bound * (1 + 1e-6))
