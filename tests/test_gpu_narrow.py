"""The narrow path (a few tokens, FP8 tiled weights) on the GPU: the same bits
as the single pass and the steps path, parity with the float64 oracle, the
alignment tables, repeated and out-of-range ids, two row tiles per expert,
a gated shared expert, and graph replay with new routings."""

import numpy as np
import pytest
import torch

import workloads
from moe_testlib import (DeviceModel, bf16_to_np, compare_tables, device_inputs, log, oracle_layer,
                         separate_steps, tolerance_ok)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_routing_align_amd as m

    return m


_MODELS = {}


def model_for(cfg):
    if cfg.name not in _MODELS:
        log(f"generating weights for {cfg.name}")
        _MODELS[cfg.name] = DeviceModel(cfg, threads=16)
    return _MODELS[cfg.name]


DECODE = workloads.CONFIGS["decode"]
# one token over a 1024-wide layer, row-scaled FP8, a shared expert
ROWS_NARROW = workloads.MoeConfig("fp8_rows_narrow", 1, 1024, 16, 4, 256, 128, 8, "fp8_rows", "softmax", seed=17)
# four tokens at top-8 over a small layer: 32 slots, the narrow path's limit
SMALL32 = workloads.MoeConfig("fp8_small32", 4, 1024, 16, 8, 256, 128, 8, "fp8", "softmax_bias", bias_std=2.0,
                              seed=23)


def _paths(moe, layer, M):
    return {p: layer.with_path(p) for p in (moe.MOE_LAYER_PATH_NARROW, moe.MOE_LAYER_PATH_SINGLE_PASS,
                                            moe.MOE_LAYER_PATH_STEPS)}


def _all_paths_equal(moe, model, xt, it, wt, sh_expert_gate=None):
    layer = model.tiled_layer() if sh_expert_gate is None else model.layer(sh_expert_gate).tiled()
    outs = {}
    for p, lay in _paths(moe, layer, xt.shape[0]).items():
        outs[p] = lay.forward(xt, it, wt)
    torch.cuda.synchronize()
    ref = outs[moe.MOE_LAYER_PATH_NARROW]
    for p, o in outs.items():
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), p
    return ref


@pytest.mark.parametrize("M", [1, 2, 3])
def test_narrow_decode_parity_and_bits(moe, M):
    """The decode layer (FP8 block scales) at 1-3 tokens: AUTO takes the
    narrow path; its tables are the oracle's, its output within the bound,
    and the single pass, the steps path and the separate calls give its bits."""
    cfg = DECODE.replace(M=M, name=f"decode_m{M}")
    model = model_for(DECODE)
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    tiled = model.tiled_layer()
    assert tiled.path(M) == moe.MOE_LAYER_PATH_NARROW
    log(f"narrow decode parity, M={M}")
    ws = tiled.alloc_workspace(M)
    out = tiled.forward(xt, it, wt, workspace=ws)
    torch.cuda.synchronize()
    views = tiled.workspace_views(ws, M)
    assert "act" in views and "expert_out" not in views and "part" not in views
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    log(f"  out: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)
    # act by slot against the oracle's act at the slot's sorted position
    perm = ref["tables"]["token_to_perm"]
    slots = [s for s in range(perm.size) if perm[s] >= 0]
    ok, err, bound = tolerance_ok(views["act"][slots].cpu().double().numpy(),
                                  np.stack([ref["act_pos"][perm[s]] for s in slots]))
    assert ok, ("act", err, bound)
    a = _all_paths_equal(moe, model, xt, it, wt)
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))
    sep, _ = separate_steps(moe, tiled, xt, it, wt)
    assert torch.equal(sep.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("gated", [False, True])
def test_narrow_rows_shared_expert(moe, gated):
    """Row-scaled FP8 with a shared expert (ungated and gated), one token."""
    model = model_for(ROWS_NARROW)
    cfg = model.cfg
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    assert model.tiled_layer().path(cfg.M) == moe.MOE_LAYER_PATH_NARROW
    g = None
    gbits = None
    if gated:
        gbits = workloads.shared_gate_bf16(cfg)
        g = torch.from_numpy(gbits.view(np.int16)).view(torch.bfloat16).cuda()
    out = _all_paths_equal(moe, model, xt, it, wt, sh_expert_gate=g)
    ref = oracle_layer(model, x, ids, w, sh_gate_bits=gbits)
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    log(f"  rows narrow gated={gated}: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)


def test_narrow_32_slots_two_row_tiles(moe):
    """32 slots (the limit), forced narrow: the skewed routing, then every slot
    on one expert (32 rows: two row tiles), then out-of-range ids; each against
    the single pass's bits and the oracle."""
    model = model_for(SMALL32)
    cfg = model.cfg
    (x, ids0, w), (xt, it0, wt) = device_inputs(cfg)
    tiled = model.tiled_layer()
    assert tiled.path(cfg.M) == moe.MOE_LAYER_PATH_STEPS  # AUTO at 4 tokens of top-8
    narrow = tiled.with_path(moe.MOE_LAYER_PATH_NARROW)
    single = tiled.with_path(moe.MOE_LAYER_PATH_SINGLE_PASS)
    one = np.full((cfg.M, cfg.top_k), 5, dtype=np.int64)
    bad = ids0.copy()
    bad[0, 1] = -1
    bad[2, 3] = cfg.E + 4
    bad[3, :] = 7
    for name, ids in (("routing", ids0), ("one expert", one), ("out of range", bad)):
        log(f"narrow, 32 slots: {name}")
        it = torch.from_numpy(ids).cuda()
        ws = narrow.alloc_workspace(cfg.M)
        a = narrow.forward(xt, it, wt, workspace=ws)
        b = single.forward(xt, it, wt)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        ref = oracle_layer(model, x, ids, w)
        compare_tables(narrow.workspace_views(ws, cfg.M), ref["tables"])
        ok, err, bound = tolerance_ok(bf16_to_np(a), ref["out"])
        assert ok, (name, err, bound)


def test_narrow_repeated_ids_one_token(moe):
    """One token whose 8 slots all name the same expert (8 rows of one
    group), and one with a repeated pair: narrow = single pass bits, oracle."""
    model = model_for(DECODE)
    cfg = DECODE.replace(M=1, name="decode_m1")
    (x, _, w), (xt, _, wt) = device_inputs(cfg)
    for ids in (np.full((1, 8), 3, dtype=np.int64), np.array([[4, 9, 4, 100, 9, 0, 127, 5]], dtype=np.int64)):
        it = torch.from_numpy(ids).cuda()
        out = _all_paths_equal(moe, model, xt, it, wt)
        ref = oracle_layer(model, x, ids, w)
        ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
        assert ok, (ids.tolist(), err, bound)


def test_narrow_graph_replay_follows_new_routing(moe):
    """Capture the one-token layer once; overwrite ids and weights in place
    between replays; every replay equals the eager call and the oracle."""
    model = model_for(DECODE)
    cfg = DECODE.replace(M=1, name="decode_m1")
    layer = model.tiled_layer()
    (x, _, _), (xt, it, wt) = device_inputs(cfg)
    ws = layer.alloc_workspace(1)
    out = torch.empty(1, cfg.H, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        layer.forward(xt, it, wt, out=out, workspace=ws)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        layer.forward(xt, it, wt, out=out, workspace=ws)
    for r in range(3):
        ids, w = workloads.routing(cfg.replace(seed=cfg.seed + 200 + r))
        it.copy_(torch.from_numpy(ids))
        wt.copy_(torch.from_numpy(w))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        eager = layer.forward(xt, it, wt)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
        ref = oracle_layer(model, x, ids, w)
        ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
        assert ok, (r, err, bound)
