"""The C-ABI library on the host: it loads, exports every declared symbol, its
pure sizing functions agree with the oracle, and every host-side check refuses
bad arguments before touching the GPU (no compute call runs here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from mixture_experts_routing_align_amd import _ffi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_mi355x.h")
FAKE = 0x1000  # a non-NULL address no call may dereference: every case below fails before any launch


@pytest.fixture(scope="module")
def lib():
    return _ffi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
        assert name in _ffi.SIGNATURES, name
    assert set(_ffi.SIGNATURES) == set(names)


def test_abi_version(lib):
    assert lib.moe_abi_version() == 11


@pytest.mark.parametrize("seed", range(5))
def test_sizing_matches_oracle(lib, seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        n = int(rng.integers(0, 100000))
        E = int(rng.integers(1, 1025))
        BS = int(rng.integers(1, 129))
        assert lib.moe_align_max_total(n, E, BS) == oracle.max_total(n, E, BS)
        assert lib.moe_active_cap(n, E) == oracle.active_cap(n, E)
    assert lib.moe_align_max_total(-1, 4, 4) == -1
    assert lib.moe_align_max_total(4, 0, 4) == -1
    assert lib.moe_active_cap(-1, 4) == -1


def _tables(ptr=FAKE):
    return _ffi.MoeAlignTables(*([ptr] * 8))


def _err(lib):
    return lib.moe_last_error().decode()


def test_align_refusals(lib):
    t = _tables()
    assert lib.moe_align(FAKE, 1, 4, 2, 1025, 16, ctypes.byref(t), None) == _ffi.MOE_ERR_LIMIT
    assert "1024" in _err(lib)
    assert lib.moe_align(FAKE, 1, 4, 0, 8, 16, ctypes.byref(t), None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_align(FAKE, 1, 4, 2, 8, 0, ctypes.byref(t), None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_align(FAKE, 1, -1, 2, 8, 16, ctypes.byref(t), None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_align(FAKE, 7, 4, 2, 8, 16, ctypes.byref(t), None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_align(None, 1, 4, 2, 8, 16, ctypes.byref(t), None) == _ffi.MOE_ERR_NULL
    bad = _tables()
    bad.token_to_perm = None
    assert lib.moe_align(FAKE, 1, 4, 2, 8, 16, ctypes.byref(bad), None) == _ffi.MOE_ERR_NULL
    assert lib.moe_align(FAKE, 1, 2 ** 30, 4, 8, 16, ctypes.byref(t), None) == _ffi.MOE_ERR_LIMIT
    # worst-case table past 2^31 entries: n = 2^20 slots, 1024 experts, BS = 2^21
    assert oracle.max_total(2 ** 20, 1024, 2 ** 21) >= 2 ** 31
    assert lib.moe_align(FAKE, 1, 2 ** 17, 8, 1024, 2 ** 21, ctypes.byref(t), None) == _ffi.MOE_ERR_LIMIT
    # M = 0: nothing to do, nothing launched
    assert lib.moe_align(None, 1, 0, 2, 8, 16, None, None) == _ffi.MOE_OK


def test_align_ws_refusals(lib):
    t = _tables()
    need = lib.moe_align_workspace_bytes(512, 8, 256)  # 4096 slots: 4 blocks of 1024
    assert need == 4 * 256 * 4
    assert lib.moe_align_workspace_bytes(511, 8, 256) == 0  # one workgroup, no workspace
    assert lib.moe_align_workspace_bytes(-1, 8, 256) == 0
    assert lib.moe_align_workspace_bytes(512, 8, 2000) == 0  # moe_align refuses E > 1024
    assert lib.moe_align_ws(FAKE, 1, 512, 8, 256, 64, ctypes.byref(t), None, need, None) == _ffi.MOE_ERR_NULL
    assert "workspace" in _err(lib)
    assert lib.moe_align_ws(FAKE, 1, 512, 8, 256, 64, ctypes.byref(t), FAKE, need - 1, None) == _ffi.MOE_ERR_WORKSPACE
    assert lib.moe_align_ws(FAKE, 1, 512, 8, 256, 64, ctypes.byref(t), FAKE + 4, need, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_align_ws(FAKE, 1, 512, 8, 1025, 64, ctypes.byref(t), FAKE, need, None) == _ffi.MOE_ERR_LIMIT
    assert lib.moe_align_ws(None, 1, 512, 8, 256, 64, ctypes.byref(t), FAKE, need, None) == _ffi.MOE_ERR_NULL
    assert lib.moe_align_ws(FAKE, 9, 512, 8, 256, 64, ctypes.byref(t), FAKE, need, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_align_ws(None, 1, 0, 8, 256, 64, None, None, 0, None) == _ffi.MOE_OK


def _w(scale=True):
    return _ffi.MoeWeight(FAKE, FAKE if scale else None)


def test_grouped_refusals(lib):
    t = _tables()
    g, u = _w(), _w()
    args = dict(M=4, H=256, I=128, S=0, E=8, top_k=2, BS=16)

    def gu(wdt=1, **kw):
        a = {**args, **kw}
        return lib.moe_grouped_gate_up_silu(FAKE, wdt, ctypes.byref(g), ctypes.byref(u), ctypes.byref(t), FAKE,
                                            None, None, None, a["M"], a["H"], a["I"], a["S"], a["E"], a["top_k"],
                                            a["BS"], None)

    assert gu(H=200) == _ffi.MOE_ERR_SHAPE          # FP8 needs whole 128 blocks
    assert gu(I=64) == _ffi.MOE_ERR_SHAPE
    assert gu(wdt=0, H=48) == _ffi.MOE_ERR_SHAPE    # BF16 needs K % 32
    assert gu(wdt=0, I=24) == _ffi.MOE_ERR_SHAPE    # and N % 16
    assert gu(wdt=8) == _ffi.MOE_ERR_SHAPE          # no such weight dtype
    assert gu(wdt=-1) == _ffi.MOE_ERR_SHAPE
    # FP8 with row scales keeps the 128-multiple shapes, and reads its scales 16 bytes at a time
    assert gu(wdt=_ffi.MOE_W_FP8_E4M3_ROWS, H=200) == _ffi.MOE_ERR_SHAPE
    assert gu(wdt=_ffi.MOE_W_FP8_E4M3_ROWS_TILED, I=64) == _ffi.MOE_ERR_SHAPE
    odd = _ffi.MoeWeight(FAKE, FAKE + 4)
    for wdt in (_ffi.MOE_W_FP8_E4M3_ROWS, _ffi.MOE_W_FP8_E4M3_ROWS_TILED):
        assert lib.moe_grouped_gate_up_silu(FAKE, wdt, ctypes.byref(odd), ctypes.byref(u), ctypes.byref(t), FAKE,
                                            None, None, None, 4, 256, 128, 0, 8, 2, 16, None) == _ffi.MOE_ERR_SHAPE
        assert "16-byte" in _err(lib)
        assert lib.moe_grouped_down(FAKE, wdt, ctypes.byref(odd), ctypes.byref(t), FAKE, None, None, None,
                                    4, 256, 128, 0, 8, 2, 16, None) == _ffi.MOE_ERR_SHAPE
    assert gu(S=128) == _ffi.MOE_ERR_NULL           # shared expert without weights
    assert gu(E=2000) == _ffi.MOE_ERR_LIMIT
    assert gu(M=0) == _ffi.MOE_OK
    nos = _w(scale=False)
    assert lib.moe_grouped_gate_up_silu(FAKE, 1, ctypes.byref(nos), ctypes.byref(u), ctypes.byref(t), FAKE, None,
                                        None, None, 4, 256, 128, 0, 8, 2, 16, None) == _ffi.MOE_ERR_NULL
    d = _w()
    assert lib.moe_grouped_down(FAKE, 1, ctypes.byref(d), ctypes.byref(t), FAKE, None, None, None,
                                4, 256, 100, 0, 8, 2, 16, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_grouped_down(FAKE, 1, ctypes.byref(d), ctypes.byref(t), FAKE, None, None, None,
                                4, 256, 128, 128, 8, 2, 16, None) == _ffi.MOE_ERR_NULL
    assert lib.moe_blend(FAKE, FAKE, FAKE, FAKE, None, None, None, 4, 6, 2, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_blend(None, FAKE, FAKE, FAKE, None, None, None, 4, 8, 2, None) == _ffi.MOE_ERR_NULL
    assert lib.moe_blend(None, None, None, None, None, None, None, 0, 8, 2, None) == _ffi.MOE_OK
    # a shared gate needs x
    assert lib.moe_blend(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 8, 2, None) == _ffi.MOE_ERR_NULL
    assert "gate" in _err(lib)


def _desc(M=8, H=2048, I=768, S=0, E=128, top_k=8, BS=16, wdt=1, idt=1):
    w = _w(wdt == 1)
    none = _ffi.MoeWeight(None, None)
    sh = w if S else none
    return _ffi.MoeLayerDesc(M, H, I, S, E, top_k, BS, wdt, idt, w, w, w, sh, sh, sh)


def _tiled(d):
    d.wdt = _ffi.MOE_W_FP8_E4M3_TILED if d.wdt == _ffi.MOE_W_FP8_E4M3 else _ffi.MOE_W_BF16_TILED
    return d


def _rows_per_pass(M):
    r = 4
    while r < M and r < 128:
        r *= 2
    return r


def _auto_single(M, n, fp8):
    """Where the single pass fits, AUTO's documented choice for tiled FP8
    (block scales) and BF16 weights: FP8 takes the steps when the slots exceed
    6 times the rows of one pass in the 4- and 8-row classes."""
    r = _rows_per_pass(M)
    return not (fp8 and r <= 8 and n > 6 * r)


@pytest.mark.parametrize("tiled", [False, True])
def test_workspace_layout(lib, tiled):
    R = _ffi.MOE_LAYER_WORKSPACE_REGIONS
    for kw in (dict(), dict(M=128, S=2048), dict(M=64, H=7168, E=256, I=2048, S=2048, BS=64),
               dict(M=4, H=256, E=8, top_k=2, I=128, wdt=0), dict(M=5, H=256, S=256, I=384)):
        d = _desc(**kw)
        if tiled:
            d = _tiled(d)
        off = (ctypes.c_size_t * (R + 1))()
        assert lib.moe_layer_workspace_layout(ctypes.byref(d), off) == _ffi.MOE_OK
        a = {k: v for k, v in dict(M=8, H=2048, I=768, S=0, E=128, top_k=8, BS=16).items()}
        a.update({k: v for k, v in kw.items() if k in a})
        n = a["M"] * a["top_k"]
        mt = oracle.max_total(n, a["E"], a["BS"])
        path = lib.moe_layer_path(ctypes.byref(d))
        # the single pass runs tiled weights at decode width (at most 256 slots)
        # where AUTO does not prefer the steps
        single_auto = tiled and n <= 256 and _auto_single(a["M"], n, kw.get("wdt", 1) == 1)
        assert path == (_ffi.MOE_LAYER_PATH_SINGLE_PASS if single_auto else _ffi.MOE_LAYER_PATH_STEPS), kw
        single = path == _ffi.MOE_LAYER_PATH_SINGLE_PASS
        M, H, I, S = a["M"], a["H"], a["I"], a["S"]
        sizes = [mt * 4, mt // a["BS"] * 4, (a["E"] + 1) * 4, a["E"] * 4, n * 4, min(n, a["E"]) * 4, 4, 4,
                 0 if single else mt * I * 4, 0 if single else mt * H * 4,
                 0 if single else M * S * 4, 0 if single else M * H * 4,
                 -(-I // 64) * n * H * 4 if single else 0, -(-S // 64) * M * H * 4 if single else 0]
        assert len(sizes) == R
        for i, s in enumerate(sizes):
            assert off[i] % 256 == 0
            assert off[i + 1] >= off[i] + s, (kw, i)
        total = lib.moe_layer_workspace_bytes(ctypes.byref(d))
        assert total == off[R]


def test_layer_refusals(lib):
    d = _desc()
    need = lib.moe_layer_workspace_bytes(ctypes.byref(d))
    assert need > 0
    rc = lib.moe_layer_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0x100000, need - 1, None)
    assert rc == _ffi.MOE_ERR_WORKSPACE
    rc = lib.moe_layer_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0x100010, need, None)
    assert rc == _ffi.MOE_ERR_WORKSPACE              # not 256-byte aligned
    rc = lib.moe_layer_forward(ctypes.byref(d), None, FAKE, FAKE, FAKE, 0x100000, need, None)
    assert rc == _ffi.MOE_ERR_NULL
    bad = _desc(H=1000)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(bad)) == 0
    assert "128" in _err(lib)
    bad = _desc(S=2048)
    bad.sh_down = _ffi.MoeWeight(None, None)
    rc = lib.moe_layer_forward(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 0x100000, 1 << 40, None)
    assert rc == _ffi.MOE_ERR_NULL
    d0 = _desc(M=0)
    assert lib.moe_layer_forward(ctypes.byref(d0), None, None, None, None, None, 0, None) == _ffi.MOE_OK


def test_fused_align_gate_up_refusals(lib):
    t = _tables()
    g, u = _w(), _w()

    def call(M, top_k=8, idt=1, **kw):
        a = dict(H=256, I=128, S=0, E=8, BS=16)
        a.update(kw)
        return lib.moe_align_gate_up_silu(FAKE, idt, FAKE, 1, ctypes.byref(g), ctypes.byref(u), ctypes.byref(t), FAKE,
                                          None, None, None, M, a["H"], a["I"], a["S"], a["E"], top_k, a["BS"], None)

    assert call(257) == _ffi.MOE_ERR_LIMIT               # 2056 slots > 2048
    assert call(4, idt=9) == _ffi.MOE_ERR_SHAPE
    assert call(4, H=100) == _ffi.MOE_ERR_SHAPE
    assert call(4, E=4096) == _ffi.MOE_ERR_LIMIT
    assert call(0) == _ffi.MOE_OK
    bad = _tables()
    bad.total = None
    assert lib.moe_align_gate_up_silu(FAKE, 1, FAKE, 1, ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad), FAKE,
                                      None, None, None, 4, 256, 128, 0, 8, 8, 16, None) == _ffi.MOE_ERR_NULL


def test_single_pass_stage_refusals(lib):
    """The stage calls refuse a descriptor that takes the steps path (row-major
    weights, more than 256 slots, or AUTO's choice of the steps) and check the
    workspace like the layer."""
    d = _desc()                                   # row-major FP8: steps path
    need = lib.moe_layer_workspace_bytes(ctypes.byref(d))
    assert lib.moe_layer_partials(ctypes.byref(d), FAKE, FAKE, 0x100000, need, None) == _ffi.MOE_ERR_SHAPE
    assert "single-pass" in _err(lib)
    assert lib.moe_layer_blend_partials(ctypes.byref(d), None, FAKE, FAKE, FAKE, 0x100000, need,
                                        None) == _ffi.MOE_ERR_SHAPE
    big = _tiled(_desc(M=128))                    # 1024 slots
    need = lib.moe_layer_workspace_bytes(ctypes.byref(big))
    assert lib.moe_layer_partials(ctypes.byref(big), FAKE, FAKE, 0x100000, need, None) == _ffi.MOE_ERR_SHAPE
    auto8 = _tiled(_desc())                       # decode shape, tiled: AUTO takes the steps
    need = lib.moe_layer_workspace_bytes(ctypes.byref(auto8))
    assert lib.moe_layer_partials(ctypes.byref(auto8), FAKE, FAKE, 0x100000, need, None) == _ffi.MOE_ERR_SHAPE
    t = _tiled(_desc())                           # the same, forced onto the single pass
    t.path = _ffi.MOE_LAYER_PATH_SINGLE_PASS
    need = lib.moe_layer_workspace_bytes(ctypes.byref(t))
    assert lib.moe_layer_partials(ctypes.byref(t), FAKE, FAKE, 0x100000, need - 1, None) == _ffi.MOE_ERR_WORKSPACE
    assert lib.moe_layer_partials(ctypes.byref(t), None, FAKE, 0x100000, need, None) == _ffi.MOE_ERR_NULL
    assert lib.moe_layer_blend_partials(ctypes.byref(t), None, FAKE, None, FAKE, 0x100000, need,
                                        None) == _ffi.MOE_ERR_NULL
    t0 = _tiled(_desc(M=0))
    assert lib.moe_layer_partials(ctypes.byref(t0), None, None, None, 0, None) == _ffi.MOE_OK



def test_path_control(lib):
    """The descriptor's `path` field: AUTO chooses from the shapes, STEPS runs
    every valid descriptor, SINGLE_PASS is refused where it does not fit; the
    workspace follows the chosen path."""
    P = _ffi
    t = _tiled(_desc(M=6))                              # 6 tokens, tiled: AUTO takes the single pass
    assert lib.moe_layer_path(ctypes.byref(t)) == P.MOE_LAYER_PATH_SINGLE_PASS
    auto_bytes = lib.moe_layer_workspace_bytes(ctypes.byref(t))
    t.path = P.MOE_LAYER_PATH_STEPS
    assert lib.moe_layer_path(ctypes.byref(t)) == P.MOE_LAYER_PATH_STEPS
    steps_bytes = lib.moe_layer_workspace_bytes(ctypes.byref(t))
    assert steps_bytes > 0 and steps_bytes != auto_bytes
    need = steps_bytes
    # the stage calls of the single pass refuse a descriptor forced onto the steps path
    assert lib.moe_layer_partials(ctypes.byref(t), FAKE, FAKE, 0x100000, need, None) == P.MOE_ERR_SHAPE
    t.path = P.MOE_LAYER_PATH_SINGLE_PASS
    assert lib.moe_layer_path(ctypes.byref(t)) == P.MOE_LAYER_PATH_SINGLE_PASS
    assert lib.moe_layer_workspace_bytes(ctypes.byref(t)) == auto_bytes
    r = _desc()                                         # row-major: no single pass
    assert lib.moe_layer_path(ctypes.byref(r)) == P.MOE_LAYER_PATH_STEPS
    r.path = P.MOE_LAYER_PATH_SINGLE_PASS
    assert lib.moe_layer_path(ctypes.byref(r)) == P.MOE_ERR_SHAPE
    assert "single-pass" in _err(lib)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(r)) == 0
    rc = lib.moe_layer_forward(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, 0x100000, 1 << 40, None)
    assert rc == P.MOE_ERR_SHAPE
    v = _tiled(_desc(M=128, S=2048))                    # 1024 slots: no single pass even when tiled
    v.path = P.MOE_LAYER_PATH_SINGLE_PASS
    assert lib.moe_layer_path(ctypes.byref(v)) == P.MOE_ERR_SHAPE
    bad = _desc()
    bad.path = 7
    assert lib.moe_layer_path(ctypes.byref(bad)) == P.MOE_ERR_SHAPE
    assert "path" in _err(lib)


def test_auto_path_by_shape_class(lib):
    """Where the single pass fits, AUTO takes the steps where they measured
    faster: block-scaled FP8 past 6 slots per pass row in the 4- and 8-row
    classes (4, 7, 8 tokens at top-8), MXFP4 and per-row FP8 scales at every
    width; BF16 always the single pass.  A forced single pass still runs."""
    P = _ffi
    for M, want in ((4, P.MOE_LAYER_PATH_STEPS), (5, P.MOE_LAYER_PATH_SINGLE_PASS),
                    (6, P.MOE_LAYER_PATH_SINGLE_PASS), (7, P.MOE_LAYER_PATH_STEPS), (8, P.MOE_LAYER_PATH_STEPS),
                    (9, P.MOE_LAYER_PATH_SINGLE_PASS), (12, P.MOE_LAYER_PATH_SINGLE_PASS),
                    (16, P.MOE_LAYER_PATH_SINGLE_PASS), (33, P.MOE_LAYER_PATH_STEPS)):
        assert lib.moe_layer_path(ctypes.byref(_tiled(_desc(M=M)))) == want, M
    for wdt in (P.MOE_W_MXFP4_TILED, P.MOE_W_FP8_E4M3_ROWS_TILED):
        for M in (4, 5, 6, 8, 9, 16):
            d = _desc(M=M)
            d.wdt = wdt
            assert lib.moe_layer_path(ctypes.byref(d)) == P.MOE_LAYER_PATH_STEPS, (wdt, M)
            d.path = P.MOE_LAYER_PATH_SINGLE_PASS
            assert lib.moe_layer_path(ctypes.byref(d)) == P.MOE_LAYER_PATH_SINGLE_PASS, (wdt, M)
    for M in (4, 8, 16):
        assert lib.moe_layer_path(ctypes.byref(_tiled(_desc(M=M, wdt=0)))) == P.MOE_LAYER_PATH_SINGLE_PASS, M


def test_narrow_path_control(lib):
    """AUTO takes the narrow path for tiled FP8 weights and at most
    MOE_NARROW_AUTO_SLOTS slots; forcing it elsewhere (BF16, row-major, more
    than MOE_NARROW_LAYER_MAX_SLOTS slots) is refused; its workspace holds act
    by slot and no expert_out, sh_out or partials."""
    P = _ffi
    for M, want in ((1, P.MOE_LAYER_PATH_NARROW), (2, P.MOE_LAYER_PATH_NARROW), (3, P.MOE_LAYER_PATH_NARROW),
                    (4, P.MOE_LAYER_PATH_STEPS), (5, P.MOE_LAYER_PATH_SINGLE_PASS), (8, P.MOE_LAYER_PATH_STEPS)):
        assert lib.moe_layer_path(ctypes.byref(_tiled(_desc(M=M)))) == want, M
    four = _tiled(_desc(M=4))                           # 32 slots of 768-wide act: past the LDS budget
    four.path = P.MOE_LAYER_PATH_NARROW
    assert lib.moe_layer_path(ctypes.byref(four)) == P.MOE_ERR_SHAPE
    four = _tiled(_desc(M=4, H=1024, I=256))            # 32 slots of a smaller layer: narrow when asked for
    assert lib.moe_layer_path(ctypes.byref(four)) == P.MOE_LAYER_PATH_STEPS
    four.path = P.MOE_LAYER_PATH_NARROW
    assert lib.moe_layer_path(ctypes.byref(four)) == P.MOE_LAYER_PATH_NARROW
    five = _tiled(_desc(M=5, H=1024, I=256))
    five.path = P.MOE_LAYER_PATH_NARROW
    assert lib.moe_layer_path(ctypes.byref(five)) == P.MOE_ERR_SHAPE
    assert "narrow" in _err(lib)
    for d in (_desc(M=1), _tiled(_desc(M=1, wdt=0))):   # row-major FP8; tiled BF16
        d.path = P.MOE_LAYER_PATH_NARROW
        assert lib.moe_layer_path(ctypes.byref(d)) == P.MOE_ERR_SHAPE
    b = _tiled(_desc(M=1, wdt=0))
    assert lib.moe_layer_path(ctypes.byref(b)) == P.MOE_LAYER_PATH_SINGLE_PASS
    s = _tiled(_desc(M=2, S=2048))
    assert lib.moe_layer_path(ctypes.byref(s)) == P.MOE_LAYER_PATH_NARROW
    off = (ctypes.c_size_t * (P.MOE_LAYER_WORKSPACE_REGIONS + 1))()
    assert lib.moe_layer_workspace_layout(ctypes.byref(s), off) == P.MOE_OK
    size = [off[i + 1] - off[i] for i in range(P.MOE_LAYER_WORKSPACE_REGIONS)]
    assert size[8] >= 16 * 768 * 4 and size[8] < 16 * 768 * 4 + 256     # act [n, I] by slot
    assert size[9] == 0 and size[11] == 0 and size[12] == 0 and size[13] == 0
    assert size[10] >= 2 * 2048 * 4                                     # sh_act [M, S]


FORCE_SCRIPT = """
import ctypes, sys
sys.path.insert(0, {root!r})
from mixture_experts_routing_align_amd import _ffi
from tests.test_abi import _desc, _tiled
lib = _ffi.load()
t = _tiled(_desc(M=6))
auto = lib.moe_layer_path(ctypes.byref(t))
t.path = _ffi.MOE_LAYER_PATH_SINGLE_PASS
explicit = lib.moe_layer_path(ctypes.byref(t))
r = _desc()
print(auto, explicit, lib.moe_layer_path(ctypes.byref(r)))
"""


@pytest.mark.parametrize("env,want", [("steps", (1, 2, 1)), ("single_pass", (2, 2, -2)), ("bogus", (2, 2, 1)),
                                      ("narrow", (-2, 2, -2))])
def test_force_path_environment(env, want):
    """MOE_FORCE_PATH replaces AUTO in every descriptor (an explicit path wins;
    a forced single pass that does not fit is refused); read once, so each case
    runs in a fresh process.  Host sizing calls only: no GPU is touched."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    e = dict(os.environ, MOE_FORCE_PATH=env)
    out = subprocess.run([sys.executable, "-c", FORCE_SCRIPT.format(root=root)], env=e, cwd=root,
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert tuple(int(v) for v in out.stdout.split()) == want


def test_stream_read_probe_refusals(lib):
    assert lib.moe_stream_read_probe(FAKE, 24, FAKE, 8, None) == _ffi.MOE_ERR_SHAPE
    assert "multiple of 16" in _err(lib)
    assert lib.moe_stream_read_probe(FAKE, 32, FAKE, 0, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_stream_read_probe(FAKE, 32, FAKE, 65537, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_stream_read_probe(None, 32, FAKE, 8, None) == _ffi.MOE_ERR_NULL
    assert lib.moe_stream_read_probe(FAKE, 32, None, 8, None) == _ffi.MOE_ERR_NULL
    assert lib.moe_stream_read_probe(FAKE + 8, 32, FAKE, 8, None) == _ffi.MOE_ERR_SHAPE
    assert lib.moe_stream_read_probe(None, 0, None, 8, None) == _ffi.MOE_OK


def test_router_refusals(lib):
    r = lib.moe_router_topk
    ok = dict(x=FAKE, w=FAKE, M=4, H=64, E=16, k=2, lg=FAKE, ids=FAKE, idt=1, wts=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return r(a["x"], a["w"], a["M"], a["H"], a["E"], a["k"], a["lg"], a["ids"], a["idt"], a["wts"], None)

    assert call(H=60) == _ffi.MOE_ERR_SHAPE
    assert "multiple of 8" in _err(lib)
    assert call(H=0) == _ffi.MOE_ERR_SHAPE
    assert call(E=0) == _ffi.MOE_ERR_SHAPE
    assert call(E=1025) == _ffi.MOE_ERR_LIMIT
    assert call(k=0) == _ffi.MOE_ERR_SHAPE
    assert call(k=17) == _ffi.MOE_ERR_SHAPE
    assert call(E=128, k=65) == _ffi.MOE_ERR_SHAPE
    assert call(M=-1) == _ffi.MOE_ERR_SHAPE
    assert call(M=1 << 20) == _ffi.MOE_ERR_LIMIT
    assert call(idt=7) == _ffi.MOE_ERR_SHAPE
    for name in ("x", "w", "lg", "ids", "wts"):
        assert call(**{name: None}) == _ffi.MOE_ERR_NULL, name
    assert call(M=0, x=None, w=None, lg=None, ids=None, wts=None) == _ffi.MOE_OK


def test_shared_gate_needs_a_shared_expert(lib):
    d = _desc()                                   # S = 0
    d.sh_expert_gate = FAKE
    need = lib.moe_layer_workspace_bytes(ctypes.byref(d))
    assert lib.moe_layer_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0x100000, need, None) == _ffi.MOE_ERR_SHAPE
    assert "shared gate" in _err(lib)
    t = _tiled(_desc(M=4, H=256, E=8, top_k=2, I=128, S=128))   # single pass, gated: blend needs x
    t.path = _ffi.MOE_LAYER_PATH_SINGLE_PASS
    t.sh_expert_gate = FAKE
    need = lib.moe_layer_workspace_bytes(ctypes.byref(t))
    assert lib.moe_layer_blend_partials(ctypes.byref(t), None, FAKE, FAKE, FAKE, 0x100000, need,
                                        None) == _ffi.MOE_ERR_NULL


def test_row_scaled_fp8_dtypes(lib):
    """Row-scaled FP8 codes tile exactly like block-scaled ones; the binding
    tells the two scale forms apart by the scales' rank."""
    import torch

    import mixture_experts_routing_align_amd as moe

    for E, N, K in ((1, 128, 256), (8, 384, 1024)):
        assert lib.moe_tiled_weight_bytes(_ffi.MOE_W_FP8_E4M3_ROWS, E, N, K) == \
            lib.moe_tiled_weight_bytes(_ffi.MOE_W_FP8_E4M3, E, N, K) == E * N * K
    assert lib.moe_tiled_weight_bytes(_ffi.MOE_W_FP8_E4M3_ROWS_TILED, 1, 128, 128) == 0  # not a source dtype
    assert lib.moe_tiled_weight_bytes(_ffi.MOE_W_FP8_E4M3_ROWS, 1, 128, 100) == 0
    w3 = torch.zeros(4, 256, 128, dtype=torch.uint8)
    w2 = torch.zeros(256, 128, dtype=torch.uint8)
    assert moe.weight_dtype((w3, torch.ones(4, 2, 1))) == _ffi.MOE_W_FP8_E4M3
    assert moe.weight_dtype((w3, torch.ones(4, 256))) == _ffi.MOE_W_FP8_E4M3_ROWS
    assert moe.weight_dtype((w2, torch.ones(2, 1))) == _ffi.MOE_W_FP8_E4M3
    assert moe.weight_dtype((w2, torch.ones(256))) == _ffi.MOE_W_FP8_E4M3_ROWS
    assert moe.weight_dtype((w3.to(torch.bfloat16), None)) == _ffi.MOE_W_BF16
    with pytest.raises(ValueError):
        moe._common_dtype((w3, torch.ones(4, 256)), (w3, torch.ones(4, 2, 1)))


def test_misaligned_pointers_refused(lib):
    """Every pointer the kernels move 16 bytes per lane (the bf16 output: 8) is
    refused off that alignment, before any launch."""
    t = _tables()
    g, u = _w(), _w()
    odd = FAKE + 8    # 8-byte but not 16-byte aligned
    odder = FAKE + 4  # not 8-byte aligned

    def refused(rc, what, bytes_=16):
        msg = _err(lib)
        assert rc == _ffi.MOE_ERR_SHAPE and what in msg and f"{bytes_}-byte" in msg, (rc, msg)

    def gu(x=FAKE, act=FAKE, w=None):
        return lib.moe_grouped_gate_up_silu(x, 1, ctypes.byref(w or g), ctypes.byref(u), ctypes.byref(t), act,
                                            None, None, None, 4, 256, 128, 0, 8, 2, 16, None)

    refused(gu(x=odd), "x")
    refused(gu(act=odd), "act")
    refused(gu(w=_ffi.MoeWeight(odd, FAKE)), "gate weights")
    refused(lib.moe_align_gate_up_silu(FAKE, 1, odd, 1, ctypes.byref(g), ctypes.byref(u), ctypes.byref(t), FAKE,
                                       None, None, None, 4, 256, 128, 0, 8, 2, 16, None), "x")
    d = _w()
    refused(lib.moe_grouped_down(odd, 1, ctypes.byref(d), ctypes.byref(t), FAKE, None, None, None,
                                 4, 256, 128, 0, 8, 2, 16, None), "act")
    refused(lib.moe_grouped_down(FAKE, 1, ctypes.byref(d), ctypes.byref(t), odd, None, None, None,
                                 4, 256, 128, 0, 8, 2, 16, None), "expert_out")
    refused(lib.moe_blend(odder, FAKE, FAKE, FAKE, None, None, None, 4, 8, 2, None), "out", 8)
    refused(lib.moe_blend(FAKE, odd, FAKE, FAKE, None, None, None, 4, 8, 2, None), "expert_out")
    refused(lib.moe_blend(FAKE, FAKE, FAKE, FAKE, odd, None, None, 4, 8, 2, None), "sh_out")

    desc = _desc()
    need = lib.moe_layer_workspace_bytes(ctypes.byref(desc))
    refused(lib.moe_layer_forward(ctypes.byref(desc), odd, FAKE, FAKE, FAKE, 0x100000, need, None), "x")
    refused(lib.moe_layer_forward(ctypes.byref(desc), FAKE, FAKE, FAKE, odder, 0x100000, need, None), "out", 8)
    wodd = _desc()
    wodd.down = _ffi.MoeWeight(odd, FAKE)
    refused(lib.moe_layer_forward(ctypes.byref(wodd), FAKE, FAKE, FAKE, FAKE, 0x100000, need, None), "down weights")
    single = _tiled(_desc())
    single.path = _ffi.MOE_LAYER_PATH_SINGLE_PASS
    need1 = lib.moe_layer_workspace_bytes(ctypes.byref(single))
    assert lib.moe_layer_path(ctypes.byref(single)) == _ffi.MOE_LAYER_PATH_SINGLE_PASS
    refused(lib.moe_layer_partials(ctypes.byref(single), odd, FAKE, 0x100000, need1, None), "x")
    refused(lib.moe_layer_blend_partials(ctypes.byref(single), FAKE, FAKE, FAKE, odder, 0x100000, need1, None),
            "out", 8)
    refused(lib.moe_tile_weights(odd, FAKE, 1, 2, 256, 128, None), "src")
    refused(lib.moe_tile_weights(FAKE, odd, 1, 2, 256, 128, None), "dst")
    refused(lib.moe_router_topk(odd, FAKE, 8, 2048, 128, 8, FAKE, FAKE, 1, FAKE, None), "x")
    refused(lib.moe_router_topk(FAKE, odd, 8, 2048, 128, 8, FAKE, FAKE, 1, FAKE, None), "router weight")


def test_mxfp4_dtypes(lib):
    """MXFP4 (two E2M1 codes per byte, one E8M0 byte per 32 k): the shape rules
    (K in whole 128-deep chunks, N in 16-row tiles), non-NULL 4-byte aligned
    scales, half-byte tiled sizes, and the binding's detection by the scales'
    byte type with K read as twice the last dimension."""
    import torch

    import mixture_experts_routing_align_amd as moe

    t = _tables()
    u = _w()

    def gu(wdt=_ffi.MOE_W_MXFP4, H=256, I=128, g=None):
        return lib.moe_grouped_gate_up_silu(FAKE, wdt, ctypes.byref(g or _w()), ctypes.byref(u), ctypes.byref(t),
                                            FAKE, None, None, None, 4, H, I, 0, 8, 2, 16, None)

    for wdt in (_ffi.MOE_W_MXFP4, _ffi.MOE_W_MXFP4_TILED):
        assert gu(wdt, H=192) == _ffi.MOE_ERR_SHAPE      # K % 128
        assert "MXFP4" in _err(lib)
        assert gu(wdt, I=24) == _ffi.MOE_ERR_SHAPE       # N % 16
        assert gu(wdt, g=_ffi.MoeWeight(FAKE, None)) == _ffi.MOE_ERR_NULL
        assert gu(wdt, g=_ffi.MoeWeight(FAKE, FAKE + 2)) == _ffi.MOE_ERR_SHAPE
        assert "4-byte" in _err(lib)
        d = _ffi.MoeWeight(FAKE, FAKE)
        assert lib.moe_grouped_down(FAKE, wdt, ctypes.byref(d), ctypes.byref(t), FAKE, None, None, None,
                                    4, 256, 192, 0, 8, 2, 16, None) == _ffi.MOE_ERR_SHAPE  # I % 128
    for E, N, K in ((1, 16, 128), (8, 768, 2048), (3, 48, 384)):
        assert lib.moe_tiled_weight_bytes(_ffi.MOE_W_MXFP4, E, N, K) == E * N * K // 2
    assert lib.moe_tiled_weight_bytes(_ffi.MOE_W_MXFP4, 1, 16, 96) == 0
    assert lib.moe_tiled_weight_bytes(_ffi.MOE_W_MXFP4_TILED, 1, 16, 128) == 0  # not a source dtype
    codes = torch.zeros(4, 256, 64, dtype=torch.uint8)
    sc = torch.zeros(4, 256, 4, dtype=torch.uint8)
    assert moe.weight_dtype((codes, sc)) == _ffi.MOE_W_MXFP4
    assert moe.weight_shape((codes, sc)) == (4, 256, 128)
    assert moe.weight_shape((codes[0], sc[0])) == (1, 256, 128)
    assert moe.weight_dtype((codes, torch.ones(4, 2, 1))) == _ffi.MOE_W_FP8_E4M3
