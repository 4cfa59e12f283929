"""The fused persistent kernels (Dispatch+GroupGEMM, GroupGEMM+Combine) give
the same bits as the unfused launch sequence, whatever the number of
persistent workers and on every rerun (the UniEP article's bit-consistency of
the fused, overlapped execution with strictly sequential execution), and match
the oracle like the unfused path."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from combine_moe_route_histogram_amd import layer as L
from gpu_util import custom_config, debug_settings, device_inputs, host, max_rel

pytestmark = pytest.mark.gpu

SHAPES = [
    (300, 256, 8, 2, 320, 0),
    (257, 128, 5, 3, 192, 2),
    (520, 192, 16, 4, 128, 0),
    (64, 128, 1, 1, 128, 1),
    (96, 64, 24, 12, 64, 1),      # 13 rows per token: the combine polls many tiles
    (200, 200, 6, 2, 136, 0),     # H, I not whole k slices
    (64, 64, 4, 4, 64, 0),        # K = E: every expert holds every token
    (40, 128, 256, 8, 64, 0),     # 256 experts, most of them empty
    (2400, 64, 1, 1, 64, 1),      # groups of 10 row tiles: split into several bands
    (33, 8, 4, 2, 8, 1),          # smallest H and I: one 16-byte vector per bf16 row
    (50, 64, 4, 2, 64, 8),        # the maximum of 8 shared experts
]
OUTS = ("x_perm", "ab", "h", "y", "out")


def _run(cfg, inp, fused, workers=None):
    with debug_settings(MOE_FUSED_WORKERS=workers):
        d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
        b = L.Buffers(d, backward=False)
        for t in (b.x_perm, b.ab, b.h, b.y, b.out):
            t.fill_(7)                       # stale values must be overwritten
        L.forward(b, device_inputs(inp), fused=fused)
        torch.cuda.synchronize()
        return b


def _inputs(shape, dtype, seed=0):
    T, H, E, K, I, Ns = shape
    cfg = custom_config(T, H, E, K, I, Ns, dtype, number=200 + seed)
    inp = synth.make_inputs(cfg, with_grad=False)
    if E == 16:
        inp["logits"][:, [2, 9]] = -30.0
        inp["logits"][: T // 2, 4] += 8.0
    return cfg, inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_fused_equals_unfused_bitwise(shape, dtype):
    cfg, inp = _inputs(shape, dtype)
    print(f"case fused shape={shape} dtype={dtype}", flush=True)
    ref = _run(cfg, inp, fused=False)
    got = _run(cfg, inp, fused=True)
    for n in OUTS:
        assert torch.equal(getattr(ref, n), getattr(got, n)), n
    fwd = O.forward(inp, cfg.K, dtype)
    if dtype == "bf16":
        assert max_rel(host(got.out), fwd["out"], dtype) <= 2e-2


@pytest.mark.parametrize("workers", [1, 7, 64])
def test_fused_result_independent_of_worker_count(workers):
    cfg, inp = _inputs(SHAPES[1], "bf16", seed=1)
    print(f"case fused workers={workers}", flush=True)
    ref = _run(cfg, inp, fused=True)
    got = _run(cfg, inp, fused=True, workers=workers)
    for n in OUTS:
        assert torch.equal(getattr(ref, n), getattr(got, n)), n


def test_fused_reruns_bit_identical():
    cfg, inp = _inputs(SHAPES[2], "bf16", seed=2)
    outs = [_run(cfg, inp, fused=True) for _ in range(3)]
    for b in outs[1:]:
        for n in OUTS:
            assert torch.equal(getattr(outs[0], n), getattr(b, n)), n


def test_dispatch_ffn_beyond_32_bit_row_offsets():
    """x of 2 GiB: the fused kernel's per-lane byte offsets into x would not
    fit 31 bits, so moe_dispatch_ffn runs the gather and the plain GEMM; the
    result is still the unfused one."""
    T, H, E, K, I = 131072, 8192, 2, 1, 64
    print(f"case dispatch_ffn large x T={T} H={H}", flush=True)
    assert T * H * 2 > 0x7FFF0000
    g = torch.Generator(device="cuda").manual_seed(5)
    p = {"logits": torch.randn(T, E, device="cuda", generator=g),
         "x": torch.randn(T, H, device="cuda", generator=g).bfloat16(),
         "w1": (0.02 * torch.randn(E, H, I, device="cuda", generator=g)).bfloat16(),
         "w3": (0.02 * torch.randn(E, H, I, device="cuda", generator=g)).bfloat16(),
         "w2": (0.02 * torch.randn(E, I, H, device="cuda", generator=g)).bfloat16()}
    d = L.make_dims(T, H, E, K, I, 0, "bf16")
    outs = {}
    for fused in (False, True):
        b = L.Buffers(d, backward=False)
        L.forward(b, p, fused=fused)
        torch.cuda.synchronize()
        outs[fused] = {n: getattr(b, n).clone() for n in ("x_perm", "ab", "h", "out")}
        del b
    for n in outs[True]:
        assert torch.equal(outs[False][n], outs[True][n]), n
