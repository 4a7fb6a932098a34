"""MXFP4 (4-bit) experts on the GPU: exact decode of every code through the
down projection (both nibbles, every position of a 128-deep chunk, scale
bytes across the documented range), the tiled layout against its documented
order, layer parity against the float64 oracle on decode, verify and odd
shapes, and the bit-exact properties (tiled = row-major, single pass = steps
path = the separate calls, row invariance)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_testlib import (DeviceModel, bf16_to_np, compare_tables, device_inputs, log, oracle_layer,
                         separate_steps, tolerance_ok)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_routing_align_amd as m

    return m


def _mx(name):
    return workloads.CONFIGS[name].replace(wdt="mxfp4", name=name + "_mxfp4")


MX = {
    "tiny": _mx("tiny"),
    "decode": _mx("decode"),
    "verify": _mx("verify"),
    # a shared expert narrower than the routed one, 36 slots (tiled: the single pass)
    "small": workloads.MoeConfig("mxfp4_small", 9, 256, 16, 4, 384, 128, 8, "mxfp4", "softmax_bias",
                                 bias_std=2.0, seed=18),
    # 130 tokens: many 16-row passes per expert (the steps path either way)
    "wide": workloads.MoeConfig("mxfp4_wide", 130, 256, 8, 2, 256, 128, 8, "mxfp4", "softmax_bias",
                                bias_std=2.0, seed=19),
    # one token over a 1024-wide layer: tiled, the 8-wave single pass
    "narrow": workloads.MoeConfig("mxfp4_narrow", 1, 1024, 16, 4, 256, 128, 8, "mxfp4", "softmax", seed=20),
}

_MODELS = {}


def model_for(key):
    if key not in _MODELS:
        log(f"generating MXFP4 weights for {MX[key].name}")
        _MODELS[key] = DeviceModel(MX[key], threads=16)
    return _MODELS[key]


# ------------------------------------------------------------ exact decode --

@pytest.mark.parametrize("tiled", [False, True])
def test_mxfp4_decode_exhaustive_through_down(moe, tiled):
    """One expert, 128 tokens on it, act row p one-hot at depth p: the down
    projection's output row p is column p of the weights, decoded.  Random
    codes (each of the 16 codes in both nibbles of every byte position) and
    scale bytes from 2 to 252 (both ends included) must come out as the OCP
    E2M1 value times 2^(scale - 127), exactly."""
    H, I = 256, 128
    rng = np.random.default_rng(41)
    packed = rng.integers(0, 256, size=(1, H, I // 2)).astype(np.uint8)
    packed[0, :16, :] = (np.arange(16, dtype=np.uint8)[:, None] * 17)  # row r: code r in both nibbles
    scales = rng.integers(2, 253, size=(1, H, I // 32)).astype(np.uint8)
    scales[0, 16, :] = 2
    scales[0, 17, :] = 252
    expect = oracle.mxfp4_decode(packed[0], scales[0])  # [H, I] float64
    M = 128
    ids = torch.zeros(M, 1, dtype=torch.int64, device="cuda")
    t = moe.moe_align(ids, 1, 16)
    sorted_ids = t.sorted_token_ids.cpu().numpy()
    assert np.array_equal(sorted_ids[:M], np.arange(M))  # one expert: positions in slot order
    act = torch.zeros(sorted_ids.size, I, dtype=torch.float32, device="cuda")
    act[torch.arange(M), torch.arange(M)] = 1.0
    weight = (torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda())
    if tiled:
        weight = moe.moe_tile_weights(weight)
    out = torch.full((sorted_ids.size, H), 7.0, dtype=torch.float32, device="cuda")
    log(f"MXFP4 exhaustive decode through down, tiled={tiled}")
    moe.moe_grouped_down(act, weight, t, out, M, 1, 16)
    torch.cuda.synchronize()
    got = out[:M].cpu().double().numpy().T  # [H, I]
    bad = np.argwhere(got != expect)
    assert bad.size == 0, (bad[:8].tolist(), got[tuple(bad[0])], expect[tuple(bad[0])])


# ------------------------------------------------------------- tiled layout --

def _tiled_reference_mxfp4(packed: np.ndarray) -> np.ndarray:
    """The documented MXFP4 tiled layout, rebuilt on the host: per expert,
    16-row tiles; per tile, 128-deep chunks; per chunk two 512-byte halves; in
    half h, lane l's 8 bytes are row 16t + l%16 at k = 128c + 64h + 16(l/16)
    .. +15, as they lie in the row-major row."""
    E, N, KB = packed.shape
    K = 2 * KB
    out = np.zeros((E, N // 16, K // 128, 2, 64, 8), dtype=np.uint8)
    for t in range(N // 16):
        for c in range(K // 128):
            for h in range(2):
                for lane in range(64):
                    row, qd = 16 * t + lane % 16, lane // 16
                    b0 = (c * 128 + 64 * h + 16 * qd) // 2
                    out[:, t, c, h, lane] = packed[:, row, b0:b0 + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("E,N,K", [(2, 256, 384), (1, 48, 128), (3, 16, 256)])
def test_mxfp4_tiled_layout_matches_documented_order(moe, E, N, K):
    rng = np.random.default_rng(31)
    packed = rng.integers(0, 256, size=(E, N, K // 2)).astype(np.uint8)
    scales = rng.integers(100, 140, size=(E, N, K // 32)).astype(np.uint8)
    tw = moe.moe_tile_weights((torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda()))
    torch.cuda.synchronize()
    assert tw.wdt == moe.MOE_W_MXFP4_TILED and tuple(tw.shape) == (E, N, K)
    assert np.array_equal(tw.w.cpu().numpy(), _tiled_reference_mxfp4(packed))


# ---------------------------------------------------------- layer parity --

def _run(moe, layer, xt, it, wt):
    ws = layer.alloc_workspace(xt.shape[0])
    out = layer.forward(xt, it, wt, workspace=ws)
    torch.cuda.synchronize()
    return out, layer.workspace_views(ws, xt.shape[0])


def _single_fits(moe, model, M):
    try:
        return model.tiled_layer().with_path(moe.MOE_LAYER_PATH_SINGLE_PASS).path(M) == moe.MOE_LAYER_PATH_SINGLE_PASS
    except moe.MoeError:
        return False


@pytest.mark.parametrize("key", list(MX))
def test_mxfp4_layer_parity(moe, key):
    """Row-major weights (the steps path), tiled weights under AUTO (the steps
    for MXFP4) and tiled weights forced onto the single pass where the shape
    fits: tables bit-exact, output within the bound of the oracle, and the runs
    equal bit for bit."""
    model = model_for(key)
    cfg = model.cfg
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    log(f"MXFP4 layer parity: {cfg}")
    layer = model.layer()
    tiled = model.tiled_layer()
    assert tiled.path(cfg.M) == moe.MOE_LAYER_PATH_STEPS
    a, views = _run(moe, layer, xt, it, wt)
    b, tviews = _run(moe, tiled, xt, it, wt)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    compare_tables(tviews, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(a), ref["out"])
    log(f"  out: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    if _single_fits(moe, model, cfg.M):
        c, sviews = _run(moe, tiled.with_path(moe.MOE_LAYER_PATH_SINGLE_PASS), xt, it, wt)
        compare_tables(sviews, ref["tables"])
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
        log("  single pass: the same bits")
    pos = sorted(ref["act_pos"])
    act = views["act"][pos].cpu().double().numpy()
    ok, err, bound = tolerance_ok(act, np.stack([ref["act_pos"][p] for p in pos]))
    assert ok, ("act", err, bound)
    y = views["expert_out"][pos].cpu().double().numpy()
    ok, err, bound = tolerance_ok(y, np.stack([ref["y_pos"][p] for p in pos]))
    assert ok, ("expert_out", err, bound)


def test_mxfp4_decode_steps_match_single_pass(moe):
    """The decode layer with tiled MXFP4 weights runs the steps under AUTO;
    forced onto the single pass it gives the same bits, and so do the four
    separate calls."""
    model = model_for("decode")
    _, (xt, it, wt) = device_inputs(model.cfg)
    tiled = model.tiled_layer()
    assert tiled.path(model.cfg.M) == moe.MOE_LAYER_PATH_STEPS
    a = tiled.with_path(moe.MOE_LAYER_PATH_SINGLE_PASS).forward(xt, it, wt)
    b = tiled.forward(xt, it, wt)
    c, _ = separate_steps(moe, tiled, xt, it, wt)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("key,ms", [("decode", [1, 2, 3, 5, 7]), ("verify", [1, 9, 64, 127]),
                                    ("wide", [1, 17, 64, 128, 129])])
def test_mxfp4_row_invariance(moe, key, ms):
    """Rows of a run on the first m tokens equal the full run's rows bit for
    bit: tiled weights (AUTO), row-major, and (decode) tiled weights forced
    onto the single pass."""
    model = model_for(key)
    _, (xt, it, wt) = device_inputs(model.cfg)
    layers = [model.tiled_layer(), model.layer()]
    if key == "decode":
        layers.append(model.tiled_layer().with_path(moe.MOE_LAYER_PATH_SINGLE_PASS))
    for layer in layers:
        full = layer.forward(xt, it, wt)
        for m in ms:
            part = layer.forward(xt[:m].contiguous(), it[:m].contiguous(), wt[:m].contiguous())
            torch.cuda.synchronize()
            assert torch.equal(part.view(torch.int16), full[:m].view(torch.int16)), m
