"""Determinism under a perturbed schedule.

MOE_DEBUG_PERTURB_SEED=n makes every persistent GEMM launch (the plain
grouped GEMMs, fused Dispatch+GroupGEMM, fused GroupGEMM+Combine and the
one-launch backward) claim each range's whole tiles in a seeded order and
sleep a seeded time before every claim; with, for the fused launches, fewer
persistent workers as well (MOE_FUSED_WORKERS), the tiles, split tails,
combine tasks and in-launch hand-offs then run in orders and at relative
times that the normal schedule never produces.  The UniEP article's claim
is that the fused, overlapped execution is bit-consistent with strictly
sequential execution: every output must be bit-identical to the unperturbed
run.
"""

import pytest
import torch

import synth
from combine_moe_route_histogram_amd import layer as L
from gpu_util import custom_config, debug_settings, device_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    (300, 256, 8, 2, 320, 0),     # ragged row tiles, partial N tiles
    (257, 128, 5, 3, 192, 2),     # shared experts
    (2400, 64, 1, 1, 64, 1),      # groups of 10 row tiles (several bands)
]
OUTS = ("x_perm", "ab", "h", "y", "out", "dy", "dtopk_w", "dab", "dx_rows", "dx", "dlogits",
        "dw1", "dw3", "dw2", "dws1", "dws3", "dws2")


def _run(cfg, inp, fused, seed=None, workers=None):
    with debug_settings(MOE_DEBUG_PERTURB_SEED=seed, MOE_FUSED_WORKERS=workers):
        d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
        b = L.Buffers(d)
        p = device_inputs(inp)
        L.forward(b, p, fused=fused)
        L.backward(b, p, fused=fused)
        torch.cuda.synchronize()
        return b


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "plain"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_perturbed_schedule_gives_the_same_bits(shape, fused):
    T, H, E, K, I, Ns = shape
    cfg = custom_config(T, H, E, K, I, Ns, "bf16", number=400)
    inp = synth.make_inputs(cfg, with_grad=True)
    print(f"case perturb shape={shape} fused={fused}", flush=True)
    ref = _run(cfg, inp, fused)
    for seed, workers in ((1, None), (2, 7), (3, 64)):
        got = _run(cfg, inp, fused, seed=seed, workers=workers)
        for n in OUTS:
            a, b = getattr(ref, n), getattr(got, n)
            if a is not None:
                assert torch.equal(a, b), (n, seed, workers)
