"""The layer's calls can be captured in a HIP graph: they allocate nothing,
never synchronise the host and issue no memset (every counter and cursor is
cleared by a kernel), so one captured step (fused forward and the one-launch
backward) replays to the bits of the same step run eagerly, replay after
replay, with eager work on the same buffers in between."""
import pytest
import torch

import synth
from combine_moe_route_histogram_amd import layer as L
from gpu_util import custom_config, device_inputs

pytestmark = pytest.mark.gpu

OUTS = ("topk_idx", "topk_w", "slot", "slot_src", "x_perm", "ab", "h", "y", "out", "dy",
        "dtopk_w", "dab", "dx_rows", "dx", "dlogits", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2")


def _step(b, p):
    L.forward(b, p, fused=True)
    L.backward(b, p, fused=True)


@pytest.mark.parametrize("shape", [(300, 256, 8, 2, 320, 0), (257, 128, 5, 3, 192, 2)],
                         ids=["routed", "shared"])
def test_captured_step_replays_eager_bits(shape):
    T, H, E, K, I, Ns = shape
    print(f"case graph shape={shape}", flush=True)
    cfg = custom_config(T, H, E, K, I, Ns, "bf16", number=400)
    p = device_inputs(synth.make_inputs(cfg, with_grad=True))
    d = L.make_dims(T, H, E, K, I, Ns, "bf16")
    b = L.Buffers(d)
    _step(b, p)
    torch.cuda.synchronize()
    ref = {n: getattr(b, n).clone() for n in OUTS if getattr(b, n) is not None}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on the capture stream
        _step(b, p)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(b, p)
    torch.cuda.synchronize()

    for rep in range(3):
        for n in ref:
            getattr(b, n).fill_(7)          # stale values must be overwritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in ref.items():
            assert torch.equal(t, getattr(b, n)), (rep, n)
        _step(b, p)                         # eager work between the replays
        torch.cuda.synchronize()
        for n, t in ref.items():
            assert torch.equal(t, getattr(b, n)), ("eager", rep, n)
