"""The whole MoE layer captured in one HIP graph (through torch.cuda.CUDAGraph) and replayed.

Every kernel of the layer is deterministic, so each replay must give the eager result bit for
bit. The replays are interleaved with eager forwards of the same layer and synchronizations,
and every replay is checked, so a graph node that only works on its first replay (a memset
recorded inside the capture, a counter left dirty by the previous run) shows up. The layer
allocates its intermediates with torch inside the capture (the graph's private pool) and
launches on torch's current stream.
"""
import pytest
import torch

from nvfp4_block_scaled_moe_amd import inputs, layer, ops
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
_WEIGHTS = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    _WEIGHTS.clear()


def _weights(name, mx):
    key = (name, mx)
    if key not in _WEIGHTS:
        wl = inputs.WORKLOADS[name]
        _WEIGHTS[key] = layer.quantize_experts_mxfp4(wl, DEV) if mx else layer.quantize_experts(wl, DEV)
    return _WEIGHTS[key]


def _replays_match(fn, replays=3):
    want = fn().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # first use of the ops on the capture's kind of stream
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    for i in range(replays):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i} differs from the eager result"
        eager = fn()                 # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(eager, want), f"eager forward after replay {i} differs"
    del g


# (workload, tokens, format): the small-M streaming GEMMs with one and many tokens (one-launch
# and two-launch routing), the large-M f16 GEMMs with activation prep (W4A4, 64 rows per
# expert), the MX GEMMs with h quantized in the epilogue, and FP8-rounded activations.
CASES = [
    ("decode", 1, "w4a16"),
    ("decode", 512, "w4a16"),
    ("decode", 2048, "w4a4"),
    ("decode", 512, "mxfp4"),
    ("many_small", 16, "w4a16"),
]


@pytest.mark.parametrize("name,T,fmt", CASES)
def test_layer_graph_replays_match_eager(name, T, fmt):
    wl = inputs.WORKLOADS[name]
    say("graph replay", name, T, fmt)
    w = _weights(name, fmt == "mxfp4")
    x = inputs.activations_bf16(wl, T=T).to(DEV)
    lg = inputs.router_logits(wl, T=T).to(DEV)
    if fmt == "mxfp4":
        fn = lambda: layer.moe_forward_mxfp4(x, lg, wl.k, w)
    else:
        mode = ops.W4A16 if fmt == "w4a16" else ops.W4A4
        fn = lambda: layer.moe_forward(x, lg, wl.k, w, mode=mode, fp8_acts=wl.act == "fp8")
    _replays_match(fn)
