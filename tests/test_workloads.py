"""The seeded input generators: determinism and the stated distributions."""

import numpy as np
import torch

from workloads import CONFIGS, expert_matrix, routing, shared_matrix, x_bf16


def test_configs_shapes():
    c = CONFIGS
    assert (c["tiny"].M, c["tiny"].H, c["tiny"].E, c["tiny"].top_k, c["tiny"].I, c["tiny"].BS) == (4, 256, 8, 2, 128, 16)
    assert (c["decode"].M, c["decode"].H, c["decode"].E, c["decode"].top_k, c["decode"].I) == (8, 2048, 128, 8, 768)
    assert (c["verify"].M, c["verify"].S) == (128, 2048)
    assert (c["align"].n, c["align"].E, c["align"].BS) == (32768, 256, 64)
    assert (c["large"].H, c["large"].E, c["large"].I, c["large"].S, c["large"].BS) == (7168, 256, 2048, 2048, 64)


def test_deterministic():
    cfg = CONFIGS["tiny"]
    assert np.array_equal(x_bf16(cfg), x_bf16(cfg))
    a, b = routing(cfg), routing(cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    w1, _ = expert_matrix(cfg, "gate", 3)
    w2, _ = expert_matrix(cfg, "gate", 3)
    assert np.array_equal(w1, w2)
    assert not np.array_equal(w1, expert_matrix(cfg, "gate", 4)[0])
    assert not np.array_equal(w1, expert_matrix(cfg, "up", 3)[0])


def test_routing_properties():
    for name in ("tiny", "decode", "verify"):
        cfg = CONFIGS[name]
        ids, w = routing(cfg)
        assert ids.shape == (cfg.M, cfg.top_k) and ids.dtype == np.int64
        assert w.dtype == np.float32
        assert np.all((ids >= 0) & (ids < cfg.E))
        assert all(len(set(r)) == cfg.top_k for r in ids.tolist())
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
        assert np.all(np.diff(w, axis=1) <= 1e-7)   # descending probability order


def test_verify_routing_is_skewed():
    ids, _ = routing(CONFIGS["verify"])
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.max() >= 64          # a per-expert bias of std 2 concentrates load
    ids2, _ = routing(CONFIGS["decode"].replace(M=128))
    assert np.bincount(ids2.reshape(-1), minlength=128).max() < counts.max()


def test_zipf_routing():
    cfg = CONFIGS["align"].replace(M=512)
    ids, w = routing(cfg)
    assert ids.shape == (512, 8)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    assert counts.max() > 5 * np.median(counts)


def test_fp8_weights_quantisation():
    cfg = CONFIGS["decode"]
    codes, scales = expert_matrix(cfg, "down", 5)
    assert codes.shape == (2048, 768) and codes.dtype == np.uint8
    assert scales.shape == (16, 6) and scales.dtype == np.float32
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert not np.isnan(vals).any()
    blk = np.abs(vals).reshape(16, 128, 6, 128).max(axis=(1, 3))
    assert np.all(blk == 448.0)              # every block reaches its scale's full range
    bound = 1 / np.sqrt(768)
    assert np.all(scales * 448 <= bound * 1.0001) and np.all(scales * 448 > 0.9 * bound)


def test_shared_matrix():
    assert shared_matrix(CONFIGS["decode"], "gate") is None
    codes, scales = shared_matrix(CONFIGS["verify"], "down")
    assert codes.shape == (2048, 2048) and scales.shape == (16, 16)


def test_bf16_weights():
    bits, sc = expert_matrix(CONFIGS["tiny"], "up", 0)
    assert sc is None and bits.dtype == np.uint16 and bits.shape == (128, 256)
    v = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert 0.015 < v.std() < 0.025


def test_mxfp4_weights_quantisation():
    """Each 32-column block's scale puts the block's largest magnitude at E2M1
    4 or 6 (amax / scale in [4, 8), rounded, saturating at 6), no element
    exceeds 6 times its scale, and the same seed gives the same bits."""
    import oracle
    import workloads

    cfg = workloads.CONFIGS["decode"].replace(wdt="mxfp4", name="decode_mxfp4")
    packed, scales = workloads.expert_matrix(cfg, "gate", 5)
    N, K = workloads.weight_shape(cfg, "gate")
    assert packed.shape == (N, K // 2) and scales.shape == (N, K // 32)
    assert packed.dtype == np.uint8 and scales.dtype == np.uint8
    w = oracle.mxfp4_decode(packed, scales)
    scale = 2.0 ** (scales.astype(np.float64) - 127)
    blocks = np.abs(w).reshape(N, K // 32, 32) / scale[:, :, None]
    assert blocks.max() <= 6.0
    assert np.all(np.isin(blocks.max(axis=2), [4.0, 6.0]))
    bound = 1.0 / np.sqrt(K)
    assert np.abs(w).max() <= 6.0 / 4.0 * bound * 1.0001
    # same seed, same bits
    p2, s2 = workloads.expert_matrix(cfg, "gate", 5)
    assert np.array_equal(p2, packed) and np.array_equal(s2, scales)
