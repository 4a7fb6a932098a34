"""GPU parity of the grouped expert FFN, the blend and the fused layer against
the float64 oracle, plus the bit-exact properties (row invariance, run-to-run
determinism, blend invariants, exact FP8 decode)."""

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


_MODELS = {}


def model_for(name, **kw):
    if name not in _MODELS:
        cfg = workloads.CONFIGS[name]
        log(f"generating weights for {name}")
        _MODELS[name] = DeviceModel(cfg, keep_host=(name != "large"), threads=16)
    return _MODELS[name]


def _run_layer(moe, model, xt, it, wt, tiled=False, path=None):
    layer = model.tiled_layer() if tiled else model.layer()
    if path is not None:
        layer = layer.with_path(path)
    ws = layer.alloc_workspace(xt.shape[0], moe.MOE_IDX_I64 if it.dtype == torch.int64 else moe.MOE_IDX_I32)
    out = layer.forward(xt, it, wt, workspace=ws)
    torch.cuda.synchronize()
    return out, layer.workspace_views(ws, xt.shape[0], moe.MOE_IDX_I64 if it.dtype == torch.int64 else
                                      moe.MOE_IDX_I32)


# ------------------------------------------------------------ FP8 decode --

@pytest.mark.parametrize("scale", [1.0, 0.375])
def test_fp8_decode_exhaustive_through_down(moe, scale):
    """Row c of a one-expert down projection holds code c at input column j and
    zeros elsewhere; act is one-hot at j.  expert_out[c] must equal the OCP e4m3
    value of c times the block scale exactly, for every code and several j."""
    H, I = 256, 128
    ids = torch.zeros(1, 1, dtype=torch.int64, device="cuda")
    t = moe.moe_align(ids, 1, 1)
    table = oracle.e4m3_table() * scale
    for j in (0, 1, 5, 8, 9, 15, 16, 31, 63, 64, 100, 127):
        w = torch.zeros(1, H, I, dtype=torch.uint8)
        w[0, :, j] = torch.arange(256, dtype=torch.int32).to(torch.uint8)
        s = torch.full((1, H // 128, I // 128), scale, dtype=torch.float32)
        act = torch.zeros(1, I, dtype=torch.float32, device="cuda")
        act[0, j] = 1.0
        out = torch.full((1, H), 7.0, dtype=torch.float32, device="cuda")
        moe.moe_grouped_down(act, (w.cuda(), s.cuda()), t, out, 1, 1, 1)
        torch.cuda.synchronize()
        got = out[0].cpu().double().numpy()
        nan = np.isnan(table)
        assert np.array_equal(np.isnan(got), nan), j
        assert np.array_equal(got[~nan], table[~nan]), (j, np.flatnonzero(got[~nan] != table[~nan])[:8])


# ------------------------------------------------------- full-layer parity --

def _check_layer(moe, name, tokens=None):
    model = model_for(name)
    cfg = model.cfg
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    log(f"layer parity: config {name} M={cfg.M} H={cfg.H} E={cfg.E} top_k={cfg.top_k} I={cfg.I} S={cfg.S}")
    out, views = _run_layer(moe, model, xt, it, wt)
    ref = oracle_layer(model, x, ids, w, tokens=tokens)
    compare_tables(views, ref["tables"])
    got = bf16_to_np(out)
    rows = ref["tokens"]
    ok, err, bound = tolerance_ok(got[rows], ref["out"])
    log(f"  out: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)
    # intermediates (debug aid): act and expert_out rows at every slot position computed
    pos = sorted(ref["act_pos"])
    act = views["act"][pos].cpu().double().numpy()
    ok, err, bound = tolerance_ok(act, np.stack([ref["act_pos"][p] for p in pos]))
    assert ok, ("act", err, bound)
    y = views["expert_out"][pos].cpu().double().numpy()
    ok, err, bound = tolerance_ok(y, np.stack([ref["y_pos"][p] for p in pos]))
    assert ok, ("expert_out", err, bound)
    if cfg.S:
        ok, err, bound = tolerance_ok(views["sh_act"][rows].cpu().double().numpy(), ref["sh_act"])
        assert ok, ("sh_act", err, bound)
        ok, err, bound = tolerance_ok(views["sh_out"][rows].cpu().double().numpy(), ref["sh_out"])
        assert ok, ("sh_out", err, bound)
    return out


def test_layer_tiny(moe):
    _check_layer(moe, "tiny")


def test_layer_decode(moe):
    _check_layer(moe, "decode")


def test_layer_verify(moe):
    _check_layer(moe, "verify")


# the large layer's oracle sample: 4 tokens from each 16-token row group of the
# shared expert (its passes), first and last token included
LARGE_TOKENS = [0, 5, 10, 15, 16, 22, 27, 31, 32, 37, 42, 47, 48, 53, 58, 63]


def test_layer_large_sampled(moe):
    # full size; the oracle computes a sample of tokens one by one
    _check_layer(moe, "large", tokens=LARGE_TOKENS)


def test_layer_large_tiled(moe):
    """The large layer with tiled weights (the form the benchmark times): its
    gate+up stages x 128 deep at a time (the 7168-deep rows do not stay
    resident in LDS).  Bit-identical to the row-major run, and within the
    tolerance of the oracle on the sampled tokens."""
    model = model_for("large")
    cfg = model.cfg
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    log(f"large layer, tiled weights: M={cfg.M} H={cfg.H} E={cfg.E} I={cfg.I} S={cfg.S}")
    a, views = _run_layer(moe, model, xt, it, wt)
    b, tviews = _run_layer(moe, model, xt, it, wt, tiled=True)
    assert model.tiled_layer().path(cfg.M) == moe.MOE_LAYER_PATH_STEPS
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle_layer(model, x, ids, w, tokens=LARGE_TOKENS)
    compare_tables(tviews, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(b)[LARGE_TOKENS], ref["out"])
    log(f"  out: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)


def test_layer_int32_ids_same_bits(moe):
    model = model_for("decode")
    _, (xt, it, wt) = device_inputs(model.cfg)
    a, _ = _run_layer(moe, model, xt, it, wt)
    b, _ = _run_layer(moe, model, xt, it.to(torch.int32), wt)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------ single-pass decode layer --

@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_single_pass_layer_parity(moe, name):
    """Tiled weights at decode width on the single-pass path (AUTO's choice for
    the BF16 tiny layer; forced for the FP8 decode layer, where AUTO takes the
    steps): tables bit-exact, output and each slot's expert output (the sum of
    its slices) within tolerance."""
    model = model_for(name)
    cfg = model.cfg
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    single = moe.MOE_LAYER_PATH_SINGLE_PASS
    assert model.tiled_layer().path(cfg.M) == (single if name == "tiny" else moe.MOE_LAYER_PATH_STEPS)
    log(f"single-pass parity: config {name}")
    out, views = _run_layer(moe, model, xt, it, wt, tiled=True, path=single)
    assert "act" not in views and "part" in views
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    log(f"  out: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)
    perm = ref["tables"]["token_to_perm"]
    slots = [i for i in range(perm.size) if perm[i] >= 0]
    y = views["part"].double().sum(dim=0)[slots].cpu().numpy()
    ok, err, bound = tolerance_ok(y, np.stack([ref["y_pos"][perm[i]] for i in slots]))
    assert ok, ("expert output", err, bound)


def test_single_pass_stages_equal_forward(moe):
    """moe_layer_partials then moe_layer_blend_partials give moe_layer_forward's bits."""
    model = model_for("decode")
    _, (xt, it, wt) = device_inputs(model.cfg)
    layer = model.tiled_layer().with_path(moe.MOE_LAYER_PATH_SINGLE_PASS)
    a = layer.forward(xt, it, wt)
    ws = layer.alloc_workspace(xt.shape[0])
    moe.moe_layer_partials(layer, xt, it, ws)
    b = moe.moe_layer_blend_partials(layer, it, wt, torch.empty_like(a), ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_single_pass_large_m_takes_steps(moe):
    """More than 256 slots (verify: 1024) keeps the separate kernels even with tiled weights."""
    model = model_for("verify")
    assert model.tiled_layer().path(model.cfg.M) == moe.MOE_LAYER_PATH_STEPS


# ------------------------------------------------ odd shapes, many passes --

ODD = [
    # BF16, N not a multiple of the 64-column tile, K with a partial 128 chunk, shared expert
    workloads.MoeConfig("bf16_odd", 5, 96, 6, 3, 160, 96, 4, "bf16", "softmax", seed=7),
    # FP8, shared expert narrower than the routed one
    workloads.MoeConfig("fp8_small", 9, 256, 16, 4, 384, 128, 8, "fp8", "softmax_bias", bias_std=2.0, seed=8),
    # 70 tokens -> 16-row passes spread over 5 workgroup rows; the skew puts > 64 rows on some
    # experts, so a workgroup row runs several passes
    workloads.MoeConfig("bf16_many_rows", 70, 128, 4, 2, 64, 0, 16, "bf16", "softmax_bias", bias_std=4.0, seed=9),
    # >= 128 tokens: nine or more 16-row passes per expert, ~75 rows per expert, a partial
    # 128-deep chunk and a shared expert
    workloads.MoeConfig("bf16_wide", 150, 96, 4, 2, 160, 96, 4, "bf16", "softmax_bias", bias_std=4.0, seed=10),
    workloads.MoeConfig("fp8_wide", 130, 256, 8, 2, 256, 128, 8, "fp8", "softmax_bias", bias_std=2.0, seed=11),
    # one token over a 1024-wide layer: the single pass's 8-wave kernel, bf16, with a shared expert
    workloads.MoeConfig("bf16_narrow", 1, 1024, 16, 4, 192, 128, 8, "bf16", "softmax", seed=12),
    # FP8 with one scale per weight row: 36 slots (tiled: the single pass), many passes
    # (steps path only), one token over a 1024-wide layer (tiled: the 8-wave single pass)
    workloads.MoeConfig("fp8_rows_small", 9, 256, 16, 4, 384, 128, 8, "fp8_rows", "softmax_bias", bias_std=2.0,
                        seed=15),
    workloads.MoeConfig("fp8_rows_wide", 130, 256, 8, 2, 256, 128, 8, "fp8_rows", "softmax_bias", bias_std=2.0,
                        seed=16),
    workloads.MoeConfig("fp8_rows_narrow", 1, 1024, 16, 4, 256, 128, 8, "fp8_rows", "softmax", seed=17),
]


@pytest.mark.parametrize("cfg", ODD, ids=lambda c: c.name)
def test_layer_odd_shapes(moe, cfg):
    model = DeviceModel(cfg, threads=4)
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    log(f"odd-shape parity: {cfg}")
    out, views = _run_layer(moe, model, xt, it, wt)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    assert ok, (err, bound)


@pytest.mark.parametrize("tiled", [False, True])
def test_layer_prefill_width_two_launch_align(moe, tiled):
    """4800 slots: past the fused align and past 4096 slots, so the layer aligns
    in two launches with the blocks' counts in its workspace (the expert_out
    region, written later by the down projection); tables bit-exact, output
    within the bound."""
    cfg = workloads.MoeConfig("bf16_prefill", 600, 96, 32, 8, 64, 0, 16, "bf16", "softmax_bias", bias_std=2.0,
                              seed=21)
    assert cfg.M * cfg.top_k >= 4096
    model = DeviceModel(cfg, threads=4)
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    log(f"prefill-width layer parity: {cfg} tiled={tiled}")
    out, views = _run_layer(moe, model, xt, it, wt, tiled=tiled)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    assert ok, (err, bound)


@pytest.mark.parametrize("tiled", [False, True])
def test_layer_repeated_ids_multi_pass(moe, tiled):
    """Every slot of every token on one expert (ids repeat within a token): 96
    rows on expert 2, more than one pass of row tiles for M=48 (tiled: the
    single-pass layer, 64 rows per pass)."""
    cfg = workloads.MoeConfig("repeat", 48, 128, 4, 2, 32, 0, 8, "bf16", "softmax", seed=11)
    model = DeviceModel(cfg, threads=4)
    (x, _, w), (xt, _, wt) = device_inputs(cfg)
    ids = np.full((cfg.M, cfg.top_k), 2, dtype=np.int64)
    it = torch.from_numpy(ids).cuda()
    if tiled:
        assert model.tiled_layer().path(cfg.M) == moe.MOE_LAYER_PATH_SINGLE_PASS
    out, views = _run_layer(moe, model, xt, it, wt, tiled=tiled)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    assert ok, (err, bound)


def test_layer_out_of_range_ids(moe):
    model = model_for("tiny")
    cfg = model.cfg
    (x, ids, w), (xt, _, wt) = device_inputs(cfg)
    ids = ids.copy()
    ids[0, 1] = -1
    ids[2, 0] = cfg.E + 3
    it = torch.from_numpy(ids).cuda()
    out, views = _run_layer(moe, model, xt, it, wt)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    assert ok, (err, bound)


# ------------------------------------------------------ bit-exact properties --

@pytest.mark.parametrize("name,ms,tiled", [("decode", [1, 2, 3, 5, 7], False),
                                           ("verify", [1, 9, 16, 33, 64, 100, 127], False),
                                           ("decode", [1, 2, 3, 5, 7], True)])
def test_row_invariance(moe, name, ms, tiled):
    """Rows 0..m-1 of a run on the first m tokens equal the full run's rows bit for bit."""
    model = model_for(name)
    _, (xt, it, wt) = device_inputs(model.cfg)
    full, _ = _run_layer(moe, model, xt, it, wt, tiled=tiled)
    for m in ms:
        part, _ = _run_layer(moe, model, xt[:m].contiguous(), it[:m].contiguous(), wt[:m].contiguous(),
                             tiled=tiled)
        assert torch.equal(part.view(torch.int16), full[:m].view(torch.int16)), m


@pytest.mark.parametrize("cfg", [c for c in ODD if c.M >= 128], ids=lambda c: c.name)
def test_row_invariance_across_pass_shapes(moe, cfg):
    """Rows of a run on the first m tokens equal the full run's rows bit for bit
    for m that change the number of row passes and workgroup rows."""
    model = DeviceModel(cfg, threads=4)
    _, (xt, it, wt) = device_inputs(cfg)
    full, _ = _run_layer(moe, model, xt, it, wt)
    for m in (1, 17, 64, 127, 128, cfg.M - 1):
        part, _ = _run_layer(moe, model, xt[:m].contiguous(), it[:m].contiguous(), wt[:m].contiguous())
        assert torch.equal(part.view(torch.int16), full[:m].view(torch.int16)), m


def test_run_to_run_bit_exact(moe):
    model = model_for("verify")
    _, (xt, it, wt) = device_inputs(model.cfg)
    first, _ = _run_layer(moe, model, xt, it, wt)
    for _ in range(5):
        again, _ = _run_layer(moe, model, xt, it, wt)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


# ------------------------------------------------------------------ blend --

def test_blend_parity_and_invariants(moe):
    rng = np.random.default_rng(5)
    M, top_k, E, BS, H = 37, 4, 16, 8, 512
    ids = np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int64)
    ids[3, 2] = -1
    ref_t = oracle.align(ids, E, BS)
    mt = ref_t["max_total"]
    eo = rng.normal(size=(mt, H)).astype(np.float32)
    w = rng.uniform(0.05, 1, size=(M, top_k)).astype(np.float32)
    sh = rng.normal(size=(M, H)).astype(np.float32)
    t = moe.moe_align(torch.from_numpy(ids).cuda(), E, BS)
    eo_d, w_d, sh_d = (torch.from_numpy(a).cuda() for a in (eo, w, sh))
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    moe.moe_blend(out, eo_d, w_d, t.token_to_perm, sh_d)
    ref = oracle.blend(eo, w, ref_t["token_to_perm"], sh.astype(np.float64))
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref)
    assert ok, (err, bound)
    # no shared expert: doubling every weight doubles the output exactly
    a = torch.empty_like(out)
    b = torch.empty_like(out)
    moe.moe_blend(a, eo_d, w_d, t.token_to_perm)
    moe.moe_blend(b, eo_d, 2 * w_d, t.token_to_perm)
    torch.cuda.synchronize()
    assert torch.equal(b.float(), 2 * a.float())
    # top-1, weight 1, no shared: the output is the row rounded to bf16
    ids1 = ids[:, :1].copy()
    ids1[3, 0] = 1
    t1 = moe.moe_align(torch.from_numpy(ids1).cuda(), E, BS)
    o1 = torch.empty_like(out)
    moe.moe_blend(o1, eo_d, torch.ones(M, 1, device="cuda"), t1.token_to_perm)
    r1 = oracle.align(ids1, E, BS)["token_to_perm"]
    assert torch.equal(o1, torch.from_numpy(eo[r1]).cuda().to(torch.bfloat16))


# ------------------------------------------------------------ graph replay --

@pytest.mark.parametrize("kind", ["rowmajor", "tiled", "single"])
def test_graph_replay_follows_new_routing(moe, kind):
    """Capture the layer once; overwrite ids/weights in place between replays;
    every replay must match the oracle for the routing it saw.  Row-major and
    tiled weights under AUTO (both the steps at this width), and tiled weights
    forced onto the single pass."""
    model = model_for("decode")
    cfg = model.cfg
    layer = {"rowmajor": model.layer(), "tiled": model.tiled_layer(),
             "single": model.tiled_layer().with_path(moe.MOE_LAYER_PATH_SINGLE_PASS)}[kind]
    (x, ids0, w0), (xt, it, wt) = device_inputs(cfg)
    ws = layer.alloc_workspace(cfg.M)
    out = torch.empty(cfg.M, cfg.H, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        layer.forward(xt, it, wt, out=out, workspace=ws)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward(xt, it, wt, out=out, workspace=ws)
    for r in range(3):
        cfg_r = cfg.replace(seed=cfg.seed + 100 + r)
        ids, w = workloads.routing(cfg_r)
        it.copy_(torch.from_numpy(ids))
        wt.copy_(torch.from_numpy(w))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = layer.forward(xt, it, wt)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
        ref = oracle_layer(model, x, ids, w)
        ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
        assert ok, (r, err, bound)


# ------------------------------------------------------------- tiled layout --

def _tiled_reference(bits: np.ndarray, fp8: bool) -> np.ndarray:
    """The documented tiled layout, rebuilt on the host: per expert, 16-row
    tiles; per tile, 128-deep chunks (zero-padded); per chunk, 1 KB fragments
    where lane l's 16 bytes hold row 16t + l%16 at the k its quad l/16 feeds."""
    E, N, K = bits.shape
    esz = 1 if fp8 else 2
    raw = bits.view(np.uint8).reshape(E, N, K * esz)
    kp = -(-K // 128) * 128
    out = np.zeros((E, N // 16, kp // 128, (128 * esz) // 64, 64, 16), dtype=np.uint8)
    for t in range(N // 16):
        for c in range(kp // 128):
            for j in range((128 * esz) // 64):
                for lane in range(64):
                    row, qd = 16 * t + lane % 16, lane // 16
                    kk = c * 128 + (j * 64 + qd * 16 if fp8 else j * 32 + qd * 8)
                    if kk < K:
                        out[:, t, c, j, lane] = raw[:, row, kk * esz:kk * esz + 16]
    return out.reshape(-1)


@pytest.mark.parametrize("fp8,E,N,K", [(True, 2, 256, 384), (False, 3, 48, 96), (False, 1, 32, 256)])
def test_tiled_layout_matches_documented_order(moe, fp8, E, N, K):
    rng = np.random.default_rng(30)
    if fp8:
        bits = rng.integers(0, 256, size=(E, N, K)).astype(np.uint8)
        w = torch.from_numpy(bits).cuda()
        s = torch.ones(E, N // 128, K // 128, device="cuda")
    else:
        bits = rng.integers(0, 2 ** 16, size=(E, N, K)).astype(np.uint16)
        w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        s = None
    tw = moe.moe_tile_weights((w, s))
    torch.cuda.synchronize()
    assert np.array_equal(tw.w.cpu().numpy(), _tiled_reference(bits, fp8))


@pytest.mark.parametrize("name", ["tiny", "decode", "verify"])
def test_tiled_layer_bit_identical(moe, name):
    """The tiled layout changes where weights sit, not what is computed."""
    model = model_for(name)
    (x, ids, w), (xt, it, wt) = device_inputs(model.cfg)
    layer = model.layer()
    tiled = layer.tiled()
    a = layer.forward(xt, it, wt)
    b = tiled.forward(xt, it, wt)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("cfg", ODD, ids=lambda c: c.name)
def test_tiled_odd_shapes_bit_identical(moe, cfg):
    model = DeviceModel(cfg, threads=4)
    _, (xt, it, wt) = device_inputs(cfg)
    layer = model.layer()
    a = layer.forward(xt, it, wt)
    b = layer.tiled().forward(xt, it, wt)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------ fused layer vs the four steps --

@pytest.mark.parametrize("name,ids_dtype", [("tiny", torch.int64), ("decode", torch.int64), ("decode", torch.int32),
                                            ("verify", torch.int64)])
def test_fused_layer_equals_separate_steps(moe, name, ids_dtype):
    """moe_layer_forward aligns inside the gate+up kernel for small slot counts;
    its output and tables equal the four separate calls' bit for bit."""
    model = model_for(name)
    _, (xt, it, wt) = device_inputs(model.cfg)
    it = it.to(ids_dtype)
    for layer in (model.layer(), model.layer().tiled()):
        ws = layer.alloc_workspace(xt.shape[0], moe.MOE_IDX_I64 if ids_dtype == torch.int64 else moe.MOE_IDX_I32)
        fused = layer.forward(xt, it, wt, workspace=ws)
        torch.cuda.synchronize()
        views = layer.workspace_views(ws, xt.shape[0], moe.MOE_IDX_I64 if ids_dtype == torch.int64 else moe.MOE_IDX_I32)
        sep, t = separate_steps(moe, layer, xt, it, wt)
        assert torch.equal(fused.view(torch.int16), sep.view(torch.int16))
        for k in moe.TABLE_FIELDS:
            assert torch.equal(views[k], getattr(t, k)), k


@pytest.mark.parametrize("cfg", ODD, ids=lambda c: c.name)
def test_fused_odd_shapes_equal_separate_steps(moe, cfg):
    model = DeviceModel(cfg, threads=4)
    _, (xt, it, wt) = device_inputs(cfg)
    layer = model.layer()
    fused = layer.forward(xt, it, wt)
    sep, _ = separate_steps(moe, layer, xt, it, wt)
    assert torch.equal(fused.view(torch.int16), sep.view(torch.int16))


def test_fused_layer_with_dropped_and_repeated_ids(moe):
    """Out-of-range ids and an expert repeated within a token, through the fused path."""
    cfg = workloads.MoeConfig("messy", 12, 128, 6, 3, 64, 0, 4, "bf16", "softmax", seed=13)
    model = DeviceModel(cfg, threads=4)
    (x, _, w), (xt, _, wt) = device_inputs(cfg)
    rng = np.random.default_rng(14)
    ids = rng.integers(-2, cfg.E + 2, size=(cfg.M, cfg.top_k)).astype(np.int64)
    ids[3] = [1, 1, 1]
    it = torch.from_numpy(ids).cuda()
    out, views = _run_layer(moe, model, xt, it, wt)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    assert ok, (err, bound)
    sep, _ = separate_steps(moe, model.layer(), xt, it, wt)
    assert torch.equal(out.view(torch.int16), sep.view(torch.int16))


# ---------------------------------------------------- gated shared expert --

@pytest.mark.parametrize("name", ["verify", "bf16_odd", "fp8_small", "bf16_narrow", "fp8_rows_narrow"])
def test_gated_shared_expert(moe, name):
    """The shared expert's output scaled by sigmoid(x . g): parity with the
    oracle on both layouts (row-major: steps path; tiled: the single pass where
    the shape takes it), the two bit-identical, and different from ungated."""
    cfg = workloads.CONFIGS[name] if name in workloads.CONFIGS else next(c for c in ODD if c.name == name)
    model = model_for(name) if name in workloads.CONFIGS else DeviceModel(cfg, threads=4)
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    g_bits = workloads.shared_gate_bf16(cfg)
    g = torch.from_numpy(g_bits.view(np.int16)).view(torch.bfloat16).cuda()
    log(f"gated shared expert: {name}")
    row = model.layer(sh_expert_gate=g)
    tiled = row.tiled()
    a = row.forward(xt, it, wt)
    b = tiled.forward(xt, it, wt)
    ungated = model.layer().forward(xt, it, wt)
    torch.cuda.synchronize()
    ref = oracle_layer(model, x, ids, w, sh_gate_bits=g_bits)
    ok, err, bound = tolerance_ok(bf16_to_np(a), ref["out"])
    assert ok, (err, bound)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), ungated.view(torch.int16))
    if name == "bf16_odd":
        assert tiled.path(cfg.M) == moe.MOE_LAYER_PATH_SINGLE_PASS


@pytest.mark.parametrize("m", [1, 2])
def test_narrow_width_kernel(moe, m):
    """At up to 8 slots of a wide layer the single pass runs its 8-wave kernel
    (gate and up on separate waves; M = 2 stays on 4 waves): oracle parity, and
    the same bits as the steps path."""
    model = model_for("decode")
    (x, ids, w), (xt, it, wt) = device_inputs(model.cfg)
    x, ids, w = x[:m], ids[:m], w[:m]
    xt, it, wt = xt[:m].contiguous(), it[:m].contiguous(), wt[:m].contiguous()
    tiled = model.tiled_layer().with_path(moe.MOE_LAYER_PATH_SINGLE_PASS)  # AUTO takes the narrow path here
    assert tiled.path(m) == moe.MOE_LAYER_PATH_SINGLE_PASS
    a = tiled.forward(xt, it, wt)
    b = model.layer().forward(xt, it, wt)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle_layer(model, x, ids, w)
    ok, err, bound = tolerance_ok(bf16_to_np(a), ref["out"])
    assert ok, (err, bound)


# ------------------------------------------------------ FP8 row scales --

@pytest.mark.parametrize("name", ["fp8_rows_small", "fp8_rows_narrow"])
def test_row_scales_single_pass(moe, name):
    """FP8 with one scale per weight row through the single-pass layer (tiled
    weights; the narrow case on its 8-wave kernel): tables bit-exact, output
    within tolerance of the oracle."""
    cfg = next(c for c in ODD if c.name == name)
    model = DeviceModel(cfg, threads=4)
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    single = moe.MOE_LAYER_PATH_SINGLE_PASS  # the one-token case would take the narrow path under AUTO
    assert model.tiled_layer().with_path(single).path(cfg.M) == single
    assert model.tiled_layer().wdt == moe.MOE_W_FP8_E4M3_ROWS_TILED
    log(f"row-scale single pass: {cfg}")
    out, views = _run_layer(moe, model, xt, it, wt, tiled=True, path=single)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    assert ok, (err, bound)


@pytest.mark.parametrize("name", ["decode", "verify"])
def test_row_scales_full_size(moe, name):
    """The decode and verify layers at full size with per-row FP8 scales:
    row-major weights (the steps path) against the oracle, tables bit-exact,
    and tiled weights (AUTO: the steps; decode also forced onto the single
    pass) with the same bits."""
    cfg = workloads.CONFIGS[name].replace(wdt="fp8_rows", name=name + "_rows")
    log(f"row-scale full size: {cfg}")
    model = DeviceModel(cfg, threads=16)
    (x, ids, w), (xt, it, wt) = device_inputs(cfg)
    out, views = _run_layer(moe, model, xt, it, wt)
    ref = oracle_layer(model, x, ids, w)
    compare_tables(views, ref["tables"])
    ok, err, bound = tolerance_ok(bf16_to_np(out), ref["out"])
    log(f"  out: max err {err:.3e} bound {bound:.3e}")
    assert ok, (err, bound)
    tiled, _ = _run_layer(moe, model, xt, it, wt, tiled=True)
    assert model.tiled_layer().path(cfg.M) == moe.MOE_LAYER_PATH_STEPS
    assert torch.equal(tiled.view(torch.int16), out.view(torch.int16))
    if name == "decode":
        single, _ = _run_layer(moe, model, xt, it, wt, tiled=True, path=moe.MOE_LAYER_PATH_SINGLE_PASS)
        assert torch.equal(single.view(torch.int16), out.view(torch.int16))
