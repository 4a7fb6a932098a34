"""Path control on the GPU: a forced path gives the bits of the path it
forces, and MOE_LOG=1 names each path the layer runs, once per process."""

import os
import subprocess
import sys

import pytest
import torch

import workloads
from moe_testlib import DeviceModel, device_inputs, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_routing_align_amd as m

    return m


def test_forced_paths_same_bits(moe):
    """The decode layer with tiled weights: AUTO (the steps at 8 tokens), forced
    onto the steps and forced onto the single pass give the same output bits,
    and so does 6 tokens under AUTO (the single pass) and forced onto the
    steps; a row-major layer cannot be forced onto the single pass."""
    cfg = workloads.CONFIGS["decode"]
    model = DeviceModel(cfg, threads=16)
    _, (xt, it, wt) = device_inputs(cfg)
    tiled = model.tiled_layer()
    assert tiled.path(cfg.M) == moe.MOE_LAYER_PATH_STEPS
    assert tiled.path(6) == moe.MOE_LAYER_PATH_SINGLE_PASS
    steps = tiled.with_path(moe.MOE_LAYER_PATH_STEPS)
    single = tiled.with_path(moe.MOE_LAYER_PATH_SINGLE_PASS)
    assert steps.path(cfg.M) == moe.MOE_LAYER_PATH_STEPS
    assert single.path(cfg.M) == moe.MOE_LAYER_PATH_SINGLE_PASS
    log("decode layer: AUTO, the forced steps path and the forced single pass")
    a = tiled.forward(xt, it, wt)
    b = steps.forward(xt, it, wt)
    c = single.forward(xt, it, wt)
    x6, i6, w6 = xt[:6].contiguous(), it[:6].contiguous(), wt[:6].contiguous()
    d = tiled.forward(x6, i6, w6)
    e = steps.forward(x6, i6, w6)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(d.view(torch.int16), e.view(torch.int16))
    assert torch.equal(d.view(torch.int16), a[:6].view(torch.int16))
    with pytest.raises(moe.MoeError):
        model.layer().with_path(moe.MOE_LAYER_PATH_SINGLE_PASS).forward(xt, it, wt)


LOG_SCRIPT = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import torch
import workloads
from moe_testlib import DeviceModel, device_inputs
cfg = workloads.CONFIGS["tiny"]
model = DeviceModel(cfg, threads=2)
_, (xt, it, wt) = device_inputs(cfg)
for _ in range(3):
    model.tiled_layer().forward(xt, it, wt)
    model.layer().forward(xt, it, wt)
torch.cuda.synchronize()
print("done", flush=True)
"""


@pytest.mark.parametrize("env", ["1", "0"])
def test_moe_log_once_per_path(env):
    """MOE_LOG=1: exactly one stderr line per path run (the tiny layer, tiled:
    single pass; row-major: steps), however many calls; MOE_LOG unset to 0:
    none.  Runs in a child process (the variable is read once per process)."""
    e = dict(os.environ, MOE_LOG=env)
    e.pop("MOE_FORCE_PATH", None)
    log(f"child process with MOE_LOG={env}")
    out = subprocess.run([sys.executable, "-c", LOG_SCRIPT.format(root=ROOT, tests=os.path.join(ROOT, "tests"))],
                         env=e, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert "done" in out.stdout
    lines = [l for l in out.stderr.splitlines() if l.startswith("moe_mi355x:")]
    if env == "1":
        assert len(lines) == 2, lines
        assert any("path single_pass" in l for l in lines) and any("path steps" in l for l in lines), lines
        assert all("M=4 H=256" in l for l in lines), lines
    else:
        assert lines == []
