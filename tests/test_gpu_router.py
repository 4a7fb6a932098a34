"""GPU parity of the per-row router against the float64 oracle.

The logits are float32 sums, so they are compared with the exact (float64)
logits within a bound on float32 accumulation: |err| <= H * 2^-23 * sum_h
|W[e,h] x[t,h]|.  The top-k choice is an integer decided by floating point:
the oracle takes it on the kernel's own float32 logits (widened exactly), so
the ids must match bit for bit, and the weights (float32 exp and sums) within
2e-6 relative + 1e-7.  Against the exact logits the choice must be valid: no
unchosen expert beats a chosen one by more than twice the bound, and where the
k-th / (k+1)-th margin exceeds that, the chosen set is the exact one.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_testlib import log

pytestmark = pytest.mark.gpu


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _check(x_bits, w_bits, top_k, ids_dtype=torch.int64):
    import mixture_experts_routing_align_amd as moe

    M, H = x_bits.shape
    E = w_bits.shape[0]
    ids, wts, logits = moe.moe_router_topk(_dev_bf16(x_bits), _dev_bf16(w_bits), top_k, ids_dtype=ids_dtype)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy().astype(np.float64)
    g_ids = ids.cpu().numpy().astype(np.int64)
    g_w = wts.cpu().numpy().astype(np.float64)

    exact = oracle.router_logits(x_bits, w_bits)
    mag = np.abs(oracle.bf16_to_f64(x_bits)) @ np.abs(oracle.bf16_to_f64(w_bits)).T
    bound = H * 2.0 ** -23 * mag + 1e-30
    assert np.all(np.abs(g_logits - exact) <= bound), float(np.max(np.abs(g_logits - exact) - bound))

    o_ids, o_w = oracle.topk_softmax(g_logits, top_k)
    assert np.array_equal(g_ids, o_ids)
    assert np.all(np.abs(g_w - o_w) <= 2e-6 * np.abs(o_w) + 1e-7), float(np.max(np.abs(g_w - o_w)))

    e_ids, _ = oracle.topk_softmax(exact, top_k)
    for t in range(M):
        chosen = set(g_ids[t].tolist())
        rest = [f for f in range(E) if f not in chosen]
        b2 = 2 * bound[t].max()
        if rest:
            assert exact[t, g_ids[t]].min() >= exact[t, rest].max() - b2, t
        srt = np.sort(exact[t])[::-1]
        if top_k < E and srt[top_k - 1] - srt[top_k] > b2:
            assert chosen == set(e_ids[t].tolist()), t
    return g_ids, g_w


@pytest.mark.parametrize("name", ["tiny", "decode", "verify", "large"])
def test_router_configs(name):
    cfg = workloads.CONFIGS[name]
    log(f"router parity: {name} M={cfg.M} H={cfg.H} E={cfg.E} top_k={cfg.top_k}")
    _check(workloads.x_bf16(cfg), workloads.router_weight_bf16(cfg), cfg.top_k)


# (the selection holds ceil(E / 64), rounded up to a power of two, logits per
# lane: 1 for E = 1, 16, 48; 2 for 70; 4 for 256; 8 for 300; 16 for 1024;
# (20, 2040, 48, 6): 16 rounds of H, the last one ragged; (5, 1000, 256, 8): 8
# rounds, the last ragged, over 16 expert tiles)
@pytest.mark.parametrize("M,H,E,k", [(37, 104, 70, 5), (1, 8, 1, 1), (17, 520, 1024, 64), (33, 64, 16, 16),
                                     (20, 2040, 48, 6), (5, 1000, 256, 8), (9, 256, 300, 10)])
def test_router_odd_shapes(M, H, E, k):
    cfg = workloads.MoeConfig("router_odd", M, H, E, k, 0, 0, 16, "bf16", "softmax", seed=M * 1000 + E)
    log(f"router odd shape M={M} H={H} E={E} top_k={k}")
    _check(workloads.x_bf16(cfg), workloads.router_weight_bf16(cfg), k, ids_dtype=torch.int32)


def test_router_ties_go_to_the_lower_expert():
    M, H, E, k = 6, 64, 40, 7
    x = np.zeros((M, H), dtype=np.uint16)  # bf16 zeros: every logit is 0
    rng = np.random.default_rng(3)
    w = workloads.bf16_bits_from_f32(rng.normal(size=(E, H)).astype(np.float32))
    ids, wts = _check(x, w, k)
    assert np.array_equal(ids, np.tile(np.arange(k), (M, 1)))
    assert np.allclose(wts, 1.0 / k, rtol=1e-7, atol=0)


def test_router_feeds_the_layer():
    """Router ids and weights drive the layer: the same output as the layer fed
    the oracle's choice on the router's logits."""
    import mixture_experts_routing_align_amd as moe
    from moe_testlib import DeviceModel

    cfg = workloads.CONFIGS["decode"]
    model = DeviceModel(cfg, keep_host=False, threads=16)
    x_bits = workloads.x_bf16(cfg)
    xt = _dev_bf16(x_bits)
    ids, wts, logits = moe.moe_router_topk(xt, _dev_bf16(workloads.router_weight_bf16(cfg)), cfg.top_k)
    o_ids, o_w = oracle.topk_softmax(logits.cpu().numpy().astype(np.float64), cfg.top_k)
    layer = model.tiled_layer()
    a = layer.forward(xt, ids, wts)
    b = layer.forward(xt, torch.from_numpy(o_ids).cuda(), torch.from_numpy(o_w.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    assert torch.equal(ids.cpu(), torch.from_numpy(o_ids))
    err = (a.float() - b.float()).abs().max().item()
    assert err <= 2e-2 * b.float().pow(2).mean().sqrt().item() + 1e-3, err


def test_router_row_invariance_and_graph_replay():
    """A row's logits, ids and weights do not depend on the other rows (M), and
    a captured router launch replays for new activations."""
    import mixture_experts_routing_align_amd as moe

    cfg = workloads.CONFIGS["verify"]
    x = _dev_bf16(workloads.x_bf16(cfg))
    w = _dev_bf16(workloads.router_weight_bf16(cfg))
    ids, wts, logits = moe.moe_router_topk(x, w, cfg.top_k)
    for m in (1, 7, 16, 17, 100):
        i2, w2, l2 = moe.moe_router_topk(x[:m].contiguous(), w, cfg.top_k)
        torch.cuda.synchronize()
        assert torch.equal(l2, logits[:m]) and torch.equal(i2, ids[:m]) and torch.equal(w2, wts[:m]), m

    xs = x[:16].clone()
    g_ids = torch.empty(16, cfg.top_k, dtype=torch.int64, device="cuda")
    g_w = torch.empty(16, cfg.top_k, dtype=torch.float32, device="cuda")
    g_l = torch.empty(16, cfg.E, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def route():
        moe._check(moe.lib().moe_router_topk(xs.data_ptr(), w.data_ptr(), 16, cfg.H, cfg.E, cfg.top_k, g_l.data_ptr(),
                                             g_ids.data_ptr(), moe.MOE_IDX_I64, g_w.data_ptr(), stream.cuda_stream))

    with torch.cuda.stream(stream):
        route()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        route()
    for start in (16, 48, 80):
        xs.copy_(x[start:start + 16])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_ids, e_w, e_l = moe.moe_router_topk(x[start:start + 16].contiguous(), w, cfg.top_k)
        torch.cuda.synchronize()
        assert torch.equal(g_ids, e_ids) and torch.equal(g_w, e_w) and torch.equal(g_l, e_l), start

