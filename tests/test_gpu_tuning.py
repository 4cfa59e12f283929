"""The auto-tuning knobs change the schedule, never the arithmetic: the fused
forward and the one-launch backward (and the plain calls) give the same bits
for every value of every knob (band heights of the gate/up projection and the
activation gradient, the small-group threshold, the weight-gradient band
heights, the fused combine and copy task sizes).  Shapes with groups of 9-10
row tiles (several bands) and shared experts; each knob is moved alone from
the shape's choice, through MOE_TUNE as moe_init reads it."""
import pytest
import torch

import synth
from combine_moe_route_histogram_amd import layer as L
from gpu_util import custom_config, debug_settings, device_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    (2400, 64, 1, 1, 64, 1),      # one expert of 2400 rows and a shared one: 10 row tiles each
    (2200, 128, 2, 2, 192, 0),    # two experts of 2200 rows (9 row tiles), partial N tiles
    (520, 192, 16, 4, 128, 0),    # skewed: empty and large experts
]
KNOBS = {
    "band_up": (1, 2, 3, 8, 16),
    "band_act": (1, 2, 8, 16),
    "small_group": (1, 2, 16),
    "band_wgrad_up": (1, 2, 8),
    "band_wgrad_down": (1, 2, 4, 16),
    "combine_tokens": (1, 7, 16, 64),
    "copy_tokens": (1, 5, 128),
    "copy_in_tiles": (0, 1),
}
OUTS = ("x_perm", "ab", "h", "y", "out", "dy", "dtopk_w", "dab", "dx_rows", "dx", "dlogits",
        "dw1", "dw3", "dw2", "dws1", "dws3", "dws2")


def _inputs(shape):
    T, H, E, K, I, Ns = shape
    cfg = custom_config(T, H, E, K, I, Ns, "bf16", number=600)
    inp = synth.make_inputs(cfg, with_grad=True)
    if E == 16:
        inp["logits"][:, [3, 7, 11]] = -30.0
        inp["logits"][: T // 2, 5] += 8.0
    return cfg, inp


def _step(cfg, p, fused, tune=None):
    with debug_settings(MOE_TUNE=tune):
        d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
        b = L.Buffers(d)
        for n in OUTS:
            t = getattr(b, n)
            if t is not None:
                t.fill_(7)                   # stale values must be overwritten
        L.forward(b, p, fused=fused)
        L.backward(b, p, fused=fused)
        L.check()
        return b


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_every_knob_value_gives_the_same_bits(shape):
    cfg, inp = _inputs(shape)
    p = device_inputs(inp)
    print(f"case tuning knobs shape={shape}", flush=True)
    ref = _step(cfg, p, fused=True)
    for knob, values in KNOBS.items():
        for v in values:
            for fused in (True, False):
                got = _step(cfg, p, fused, tune=f"{knob}={v}")
                for n in OUTS:
                    a, b = getattr(ref, n), getattr(got, n)
                    if a is not None:
                        assert torch.equal(a, b), (n, knob, v, fused)
