"""The C-ABI boundary's launch contract on the GPU: a first launch inside
stream capture is refused cleanly (and captures nothing), ct_init makes
capture possible, a graph captured before its stream's workspace grew still
replays bit for bit, and repeated launches reuse one launch plan."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl

from _gpu_helpers import DEV, legal_configs, oracle_full, say, to_dev

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# A fresh process: its very first library call is a launch inside capture.
_CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
from tensor_compiler_tiling_amd import convtile as ct
from tensor_compiler_tiling_amd import workloads as wl
out = {}
w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
inp = wl.conv_inputs(w)
x = torch.from_numpy(inp["x"]).cuda()
k = torch.from_numpy(inp["w"]).cuda()
y = torch.empty((1, 512, 7, 7), device="cuda")
lib = ct.library()
s = torch.cuda.Stream()
args = w.shape_args() + (ct.CT_F32, 0)
def fwd():
    return lib.ct_conv2d_nchw_fwd(x.data_ptr(), k.data_ptr(), y.data_ptr(), *args, None, None, 1e-5,
                                  torch.cuda.current_stream().cuda_stream)
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):
    out["first_under_capture"] = fwd()
    out["first_msg"] = lib.ct_last_error().decode()
torch.cuda.synchronize()
out["init"] = ct.ct_init(0)
# the shipped tuning log: the layer's config uses split reduction
assert ct.ct_cache_load(sys.argv[2]) == 0
# the device is set up; the stream's split workspace does not exist yet
g2 = torch.cuda.CUDAGraph()
with torch.cuda.graph(g2, stream=s):
    out["grow_under_capture"] = fwd()
torch.cuda.synchronize()
# one eager launch on the stream grows its workspace; then capture works
with torch.cuda.stream(s):
    out["eager"] = fwd()
torch.cuda.synchronize()
ref = y.clone()
g3 = torch.cuda.CUDAGraph()
with torch.cuda.graph(g3, stream=s):
    out["captured"] = fwd()
same = []
for rep in range(3):
    y.fill_(float("nan"))
    torch.cuda.synchronize()
    g3.replay()
    torch.cuda.synchronize()
    same.append(bool(torch.equal(y.view(torch.int32), ref.view(torch.int32))))
out["replays_match"] = same
print("RESULT " + json.dumps(out), flush=True)
"""


def test_first_launch_under_capture_is_refused_cleanly():
    say("[boundary] fresh process, first launch inside capture")
    log = os.path.join(ROOT, "tensor_compiler_tiling_amd", "tuned", "gfx950.jsonl")
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, log], capture_output=True, text=True, timeout=240)
    line = [l for l in r.stdout.splitlines() if l.startswith("RESULT ")]
    assert r.returncode == 0 and line, r.stdout[-2000:] + r.stderr[-2000:]
    out = json.loads(line[0][7:])
    say(f"  {out}")
    assert out["first_under_capture"] == ct.CT_ERR_UNSUPPORTED
    assert "ct_init" in out["first_msg"]
    assert out["init"] == 0
    assert out["grow_under_capture"] == ct.CT_ERR_UNSUPPORTED
    assert out["eager"] == 0 and out["captured"] == 0
    assert out["replays_match"] == [True, True, True]


def test_graph_replays_after_the_stream_workspace_grew():
    """Capture the headline layer (split reduction) on a stream, then make a
    much larger split-reduction layer grow that stream's workspace, then
    replay the graph: the buffers it captured are still allocated, so every
    replay gives the eager bits."""
    w = wl.CONV_WORKLOADS["resnet_final_c512_7x7_k3"]
    inp = wl.conv_inputs(w)
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    s = torch.cuda.Stream()
    y = torch.empty((1, 512, 7, 7), device=DEV)
    with torch.cuda.stream(s):
        ct.conv2d(x, k, 1, 1, out=y, stream=s)
    torch.cuda.synchronize()
    ref = y.clone()
    yr, a = oracle_full(w, inp)
    assert float(np.abs(ref.cpu().numpy() - yr).max()) <= 1e-4 * float(a.max())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ct.conv2d(x, k, 1, 1, out=y, stream=s)
    # a 1x1 layer with 1024 output channels over 64x64 pixels, split in two:
    # its partials (2 x 1024 x 4096 floats, 32 MiB) exceed anything the
    # headline layer allocated
    big = wl.ConvWorkload("grow_ws", 120, 1, 256, 64, 64, 1024, 1, 1, 1, 0)
    cfg = min((c for c in legal_configs(big) if c.split_k > 1), key=lambda c: c.split_k)
    bx = torch.randn((1, 256, 64, 64), device=DEV)
    bk = torch.randn((1024, 256, 1, 1), device=DEV)
    with torch.cuda.stream(s):
        ct.conv2d(bx, bk, 1, 0, config=cfg, stream=s)
    torch.cuda.synchronize()
    say(f"[boundary] workspace grown by split {cfg.split_k}; replaying the earlier graph")
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), rep


def test_repeated_launches_reuse_the_plan():
    w = wl.CONV_WORKLOADS["resnet_c64_14x14_k3"]
    inp = wl.conv_inputs(w)
    x = to_dev(inp["x"], w.dtype)
    k = to_dev(inp["w"], w.dtype)
    y = ct.conv2d(x, k, 1, 1)
    m0 = ct.ct_plan_misses()
    for _ in range(20):
        ct.conv2d(x, k, 1, 1, out=y)
    torch.cuda.synchronize()
    assert ct.ct_plan_misses() == m0
    # a change of the config cache retires the plans: one more resolution
    ct.ct_cache_clear()
    ct.conv2d(x, k, 1, 1, out=y)
    ct.conv2d(x, k, 1, 1, out=y)
    torch.cuda.synchronize()
    assert ct.ct_plan_misses() == m0 + 1
    yr, a = oracle_full(w, inp)
    assert float(np.abs(y.cpu().numpy() - yr).max()) <= 1e-4 * float(a.max())


def test_init_rejects_a_missing_device():
    assert ct.ct_init(-1) == ct.CT_ERR_INVALID_ARG
    assert ct.ct_init(torch.cuda.device_count()) == ct.CT_ERR_INVALID_ARG
    assert ct.ct_init(0) == 0 and ct.ct_init(0) == 0
