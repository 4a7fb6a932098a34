"""The wide-pass grouped kernels on the GPU (FP8 and MXFP4 layers whose experts
hold many rows): parity with the float64 oracle, and the same bits as the
16-row pass kernels (a run on the first 16 tokens takes those; its rows must
equal the wide run's), on shapes that exercise the cases of the wide kernels:
experts with several 32-row passes, every slot on a few experts, out-of-range
ids, a shared expert whose tokens end mid-pass and whose depth ends mid-round,
per-row scales, an output width that ends inside a 256-row group, and a depth
of 3 chunks that the gate+up pads to a round of 6."""

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


CONFIGS = {
    # 96 tokens at top-4 over 8 experts, skewed: experts of up to 96 rows (three passes)
    "heavy": workloads.MoeConfig("wide_heavy", 96, 512, 8, 4, 256, 0, 16, "fp8", "softmax_bias", bias_std=3.0,
                                 seed=61),
    # row scales and a shared expert: 40 tokens (shared passes of 32 + 8 tokens),
    # shared depth 384 (6 halves: down pads to rounds of 4)
    "shared_rows": workloads.MoeConfig("wide_shared_rows", 40, 512, 8, 2, 128, 384, 16, "fp8_rows", "softmax",
                                       seed=62),
    # hidden 384: gate+up depth of 3 chunks (padded to a round of 6), down's
    # second 256-row group half full
    "mixed": workloads.MoeConfig("wide_mixed", 48, 384, 4, 2, 256, 0, 16, "fp8", "softmax", seed=63),
    # MXFP4: experts of up to 96 rows
    "mx_heavy": workloads.MoeConfig("wide_mx_heavy", 96, 512, 8, 4, 256, 0, 16, "mxfp4", "softmax_bias",
                                    bias_std=3.0, seed=64),
    # MXFP4, hidden 384 (gate+up depth 3 chunks, down's second 256-row group
    # half full), routed down depth 128 (2 halves, padded to 4), a shared
    # expert of 384 (6 halves) over 40 tokens (passes of 32 + 8)
    "mx_shared": workloads.MoeConfig("wide_mx_shared", 40, 384, 8, 2, 128, 384, 16, "mxfp4", "softmax", seed=65),
    # intermediate 1152: 18 gate+up column groups, so the XCD lanes hold 2 or 3
    # columns of an expert; down depth 9 chunks (18 halves, padded to 20)
    "many_groups": workloads.MoeConfig("wide_many_groups", 64, 256, 16, 4, 1152, 0, 16, "fp8", "softmax_bias",
                                       bias_std=2.0, seed=67),
    "mx_many_groups": workloads.MoeConfig("wide_mx_many_groups", 64, 256, 16, 4, 1152, 0, 16, "mxfp4",
                                          "softmax_bias", bias_std=2.0, seed=68),
}

_MODELS = {}


def model_for(key):
    if key not in _MODELS:
        log(f"generating weights for {CONFIGS[key].name}")
        _MODELS[key] = DeviceModel(CONFIGS[key], threads=16)
    return _MODELS[key]


def _check(moe, model, x, ids, w, xt, it, wt, label):
    cfg = model.cfg
    ref = oracle_layer(model, x, ids, w)
    outs = []
    for layer in (model.layer(), model.tiled_layer().with_path(moe.MOE_LAYER_PATH_STEPS)):
        ws = layer.alloc_workspace(cfg.M)
        out = layer.forward(xt, it, wt, workspace=ws)
        torch.cuda.synchronize()
        compare_tables(layer.workspace_views(ws, cfg.M), ref["tables"])
        ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
        log(f"  {label}: max err {err:.3e} bound {bound:.3e}")
        assert ok, (label, err, bound)
        views = layer.workspace_views(ws, cfg.M)
        pos = sorted(ref["act_pos"])
        ok, err, bound = tolerance_ok(views["act"][pos].cpu().double().numpy(),
                                      np.stack([ref["act_pos"][p] for p in pos]))
        assert ok, (label, "act", err, bound)
        ok, err, bound = tolerance_ok(views["expert_out"][pos].cpu().double().numpy(),
                                      np.stack([ref["y_pos"][p] for p in pos]))
        assert ok, (label, "expert_out", err, bound)
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), label
    return outs[1]


@pytest.mark.parametrize("key", list(CONFIGS))
def test_wide_parity_and_pass_kernel_bits(moe, key):
    """Oracle parity (tables, act, expert_out, output), row-major = tiled, the
    separate calls = the layer, and rows equal to a 16-token run's (the pass
    kernels) and to runs on 17 and 33 tokens (wide again, other pass splits)."""
    model = model_for(key)
    cfg = model.cfg
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    log(f"wide parity: {cfg}")
    full = _check(moe, model, x, ids, w, xt, it, wt, key)
    tiled = model.tiled_layer()
    sep, _ = separate_steps(moe, tiled, xt, it, wt)
    assert torch.equal(sep.view(torch.int16), full.view(torch.int16))
    # 16 tokens: the 16-row pass kernels (row-major) and the library's choice
    # for tiled weights (the single pass); 17 and 33: wide, other pass splits
    for m in (16, 17, 33, cfg.M):
        for layer in (model.layer(), tiled):
            part = layer.forward(xt[:m].contiguous(), it[:m].contiguous(), wt[:m].contiguous())
            torch.cuda.synchronize()
            assert torch.equal(part.view(torch.int16), full[:m].view(torch.int16)), (m, layer.path(m))


@pytest.mark.parametrize("key", ["heavy", "mx_heavy"])
def test_wide_every_slot_on_few_experts(moe, key):
    """Every token names experts 0..3 (96 rows each: three passes per expert),
    then a routing with out-of-range ids and a token whose slots are all
    dropped: oracle parity and pass-kernel bits."""
    model = model_for(key)
    cfg = model.cfg
    (x, ids0, w), (xt, _, wt) = device_inputs(cfg)
    few = np.tile(np.arange(4, dtype=np.int64), (cfg.M, 1))
    bad = ids0.copy()
    bad[3, 1] = -1
    bad[10, :] = cfg.E + 2
    bad[50, 2] = 1 << 20
    for label, ids in (("experts 0..3", few), ("out of range", bad)):
        it = torch.from_numpy(ids).cuda()
        full = _check(moe, model, x, ids, w, xt, it, wt, label)
        part = model.layer().forward(xt[:16].contiguous(), it[:16].contiguous(), wt[:16].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int16), full[:16].view(torch.int16)), label


def test_wide_graph_replay(moe):
    """The verify-width layer captured once; ids and weights rewritten in place
    between replays; each replay equals the eager call."""
    model = model_for("heavy")
    cfg = model.cfg
    (_, _, _), (xt, it, wt) = device_inputs(cfg)
    layer = model.tiled_layer()
    assert layer.path(cfg.M) == moe.MOE_LAYER_PATH_STEPS
    ws = layer.alloc_workspace(cfg.M)
    out = torch.empty(cfg.M, cfg.H, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        layer.forward(xt, it, wt, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward(xt, it, wt, out=out, workspace=ws)
    for r in range(3):
        ids, w = workloads.routing(cfg.replace(seed=cfg.seed + 100 + r))
        it.copy_(torch.from_numpy(ids))
        wt.copy_(torch.from_numpy(w))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = layer.forward(xt, it, wt)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
