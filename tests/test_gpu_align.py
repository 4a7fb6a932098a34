"""GPU parity of moe_align: every table bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_testlib import compare_tables, log

pytestmark = pytest.mark.gpu


def _gpu_align(ids_np, E, BS, dtype=torch.int64, ws=False):
    """moe_align, or (ws) moe_align_ws with a workspace pre-filled with garbage:
    the tables may not depend on what it held."""
    import mixture_experts_routing_align_amd as moe

    ids = torch.from_numpy(np.ascontiguousarray(ids_np)).to(dtype).cuda()
    if ws:
        M, top_k = ids.shape
        nbytes = moe.moe_align_workspace_bytes(M, top_k, E)
        work = torch.full((max(nbytes, 16) // 4,), -12345, dtype=torch.int32, device="cuda")
        t = moe.moe_align_ws(ids, E, BS, work)
    else:
        t = moe.moe_align(ids, E, BS)
    torch.cuda.synchronize()
    return {k: getattr(t, k) for k in moe.TABLE_FIELDS}


@pytest.mark.parametrize("name", ["tiny", "decode", "verify", "align", "large"])
@pytest.mark.parametrize("dtype", [torch.int64, torch.int32])
@pytest.mark.parametrize("ws", [False, True], ids=["tables_only", "workspace"])
def test_align_configs_bit_exact(name, dtype, ws):
    cfg = workloads.CONFIGS[name]
    log(f"align parity: config {name} n={cfg.n} E={cfg.E} BS={cfg.BS} ids {dtype} workspace={ws}")
    ids, _ = workloads.routing(cfg)
    compare_tables(_gpu_align(ids, cfg.E, cfg.BS, dtype, ws), oracle.align(ids, cfg.E, cfg.BS))


ADVERSARIAL = [
    ("one_expert_all_slots", lambda r: np.full((300, 4), 5), 8, 16),
    ("all_distinct", lambda r: r.permutation(1024)[:1000].reshape(250, 4), 1024, 16),
    ("out_of_range", lambda r: r.integers(-3, 11, size=(77, 3)), 8, 4),
    ("bs1", lambda r: r.integers(0, 64, size=(100, 8)), 64, 1),
    ("single_expert_E1", lambda r: np.zeros((13, 1)), 1, 16),
    ("max_experts", lambda r: r.integers(0, 1024, size=(500, 8)), 1024, 64),
    ("ragged_n", lambda r: r.integers(0, 7, size=(37, 3)), 7, 3),
    ("single_slot", lambda r: np.array([[2]]), 4, 8),
    ("large_bs", lambda r: r.integers(0, 32, size=(64, 2)), 32, 256),
    ("all_invalid", lambda r: np.full((20, 2), -1), 8, 4),
    ("skewed_big", lambda r: np.minimum(r.geometric(0.05, size=(8192, 4)), 300), 300, 32),
    # from 4096 slots on, the alignment runs over blocks of 1024 slots (count, scan, scatter)
    ("blocks_one_expert", lambda r: np.full((5000, 2), 7), 16, 64),
    ("blocks_max_experts", lambda r: r.integers(-1, 1025, size=(1500, 7)), 1024, 8),
    ("blocks_exact_4096", lambda r: r.integers(0, 64, size=(512, 8)), 64, 16),
    ("below_blocks_4095", lambda r: r.integers(0, 64, size=(4095, 1)), 64, 16),
    ("blocks_ragged_tail", lambda r: r.integers(-2, 40, size=(2047, 3)), 37, 5),
    ("blocks_bs1", lambda r: r.integers(0, 200, size=(3000, 4)), 200, 1),
    ("blocks_65536", lambda r: r.integers(-1, 300, size=(8192, 8)), 300, 16),
    ("blocks_1024_experts_20000", lambda r: r.integers(0, 1024, size=(2500, 8)), 1024, 4),
    ("blocks_65537_ragged", lambda r: r.integers(0, 256, size=(65537, 1)), 256, 64),
    ("blocks_skewed_72000", lambda r: np.minimum(r.geometric(0.02, size=(9000, 8)), 255), 256, 64),
]


@pytest.mark.parametrize("case", ADVERSARIAL, ids=lambda c: c[0])
@pytest.mark.parametrize("ws", [False, True], ids=["tables_only", "workspace"])
def test_align_adversarial(case, ws):
    name, make, E, BS = case
    ids = make(np.random.default_rng(99)).astype(np.int64)
    log(f"align adversarial: {name} shape={ids.shape} E={E} BS={BS} workspace={ws}")
    compare_tables(_gpu_align(ids, E, BS, ws=ws), oracle.align(ids, E, BS))


def test_align_ws_past_its_cap():
    """1024 experts over 257 blocks of 1024 slots: E * G^2 passes the workspace
    form's limit, so moe_align_ws runs the three launches; its tables are the
    oracle's (and at 256 blocks, the workspace form's own)."""
    for rows in (32896, 32768):  # 257 and 256 blocks of 1024 slots at top-8
        ids = np.random.default_rng(7).integers(-1, 1025, size=(rows, 8)).astype(np.int64)
        log(f"align ws at its limit: {rows * 8} slots, 1024 experts")
        compare_tables(_gpu_align(ids, 1024, 4, ws=True), oracle.align(ids, 1024, 4))


def test_align_int64_ids_beyond_int32():
    """int64 ids that would alias a valid expert if truncated to 32 bits are dropped."""
    ids = np.array([[2 ** 32 + 1, 1], [3, -(2 ** 40)], [2 ** 33, 0]], dtype=np.int64)
    compare_tables(_gpu_align(ids, 4, 2), oracle.align(ids, 4, 2))


def test_align_deterministic_repeats():
    cfg = workloads.CONFIGS["align"]
    ids, _ = workloads.routing(cfg)
    first = _gpu_align(ids, cfg.E, cfg.BS)
    for _ in range(10):
        again = _gpu_align(ids, cfg.E, cfg.BS)
        for k in first:
            assert torch.equal(first[k], again[k]), k


@pytest.mark.parametrize("seed", range(8))
def test_align_random_shapes(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 1025))
    BS = int(rng.choice([1, 2, 4, 16, 64, 128]))
    M = int(rng.integers(1, 3000 if seed < 4 else 6000))
    top_k = int(rng.integers(1, 9))
    ids = rng.integers(-1, E + 1, size=(M, top_k))
    ws = seed % 4 >= 2
    log(f"align random: seed={seed} M={M} top_k={top_k} E={E} BS={BS} workspace={ws}")
    compare_tables(_gpu_align(ids, E, BS, torch.int32 if seed % 2 else torch.int64, ws), oracle.align(ids, E, BS))


def test_align_ws_graph_replay_and_reuse():
    """The two-launch align captured once and replayed over new ids (the
    workspace keeps the previous call's counts) matches the oracle each time."""
    import mixture_experts_routing_align_amd as moe

    cfg = workloads.CONFIGS["align"]
    M, top_k, E, BS = cfg.M, cfg.top_k, cfg.E, cfg.BS
    routings = [workloads.routing(cfg.replace(seed=cfg.seed + r))[0] for r in range(3)]
    ids = torch.from_numpy(routings[0]).cuda()
    work = torch.empty(moe.moe_align_workspace_bytes(M, top_k, E) // 4, dtype=torch.int32, device="cuda")
    tables = moe.AlignTables.allocate(M, top_k, E, BS)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        moe.moe_align_ws(ids, E, BS, work, tables=tables)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_align_ws(ids, E, BS, work, tables=tables)
    for r in (1, 2, 0, 1):
        ids.copy_(torch.from_numpy(routings[r]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"align workspace graph replay: routing {r}")
        compare_tables({k: getattr(tables, k) for k in moe.TABLE_FIELDS}, oracle.align(routings[r], E, BS))
