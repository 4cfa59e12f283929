"""The one-launch expert-FFN backward (moe_expert_ffn_bwd: input-gradient
"B" tiles with the weight-gradient "W" tiles scheduled into their gaps, as in
the GraphPP article's zero-bubble B/W split) gives the same bits as the two
plain calls, B then W, whatever the number of persistent workers and on every
rerun, and matches the oracle like them."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from combine_moe_route_histogram_amd import layer as L
from gpu_util import custom_config, debug_settings, device_inputs, f32_rel, host, max_rel

pytestmark = pytest.mark.gpu

SHAPES = [
    (300, 256, 8, 2, 320, 0),     # ragged row tiles, partial N tiles
    (257, 128, 5, 3, 192, 2),     # shared experts
    (520, 192, 16, 4, 128, 0),    # empty and huge experts
    (64, 128, 1, 1, 128, 1),      # one expert, one row tile
    (1, 64, 4, 2, 64, 0),         # a single token: most experts empty
    (150, 72, 4, 2, 88, 1),       # H, I not whole k slices, a shared expert
    (64, 64, 4, 4, 64, 0),        # K = E
    (40, 128, 256, 8, 64, 1),     # 256 experts, most empty, a shared expert
    (2400, 64, 1, 1, 64, 1),      # groups of 10 row tiles: split into several bands
    (33, 8, 4, 2, 8, 1),          # smallest H and I: one 16-byte vector per bf16 row
    (50, 64, 4, 2, 64, 8),        # the maximum of 8 shared experts
]
OUTS = ("dab", "dx_rows", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2", "dx", "dtopk_w", "dlogits")


def _inputs(shape, dtype, seed=0):
    T, H, E, K, I, Ns = shape
    cfg = custom_config(T, H, E, K, I, Ns, dtype, number=300 + seed)
    inp = synth.make_inputs(cfg, with_grad=True)
    if E == 16:
        inp["logits"][:, [3, 11]] = -30.0
        inp["logits"][: T // 2, 6] += 8.0
    return cfg, inp


def _run(cfg, inp, fused_bwd, workers=None):
    with debug_settings(MOE_FUSED_WORKERS=workers):
        d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
        p = device_inputs(inp)
        b = L.Buffers(d)
        for n in OUTS:
            t = getattr(b, n)
            if t is not None:
                t.fill_(7)                   # stale values must be overwritten
        L.forward(b, p)
        L.backward(b, p, fused=fused_bwd)
        torch.cuda.synchronize()
        return b


def _same(ref, got):
    for n in OUTS:
        a, b = getattr(ref, n), getattr(got, n)
        if a is None:
            continue
        assert torch.equal(a, b), n


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_fused_bwd_equals_b_then_w_bitwise(shape, dtype):
    cfg, inp = _inputs(shape, dtype)
    print(f"case fused bwd shape={shape} dtype={dtype}", flush=True)
    ref = _run(cfg, inp, fused_bwd=False)
    got = _run(cfg, inp, fused_bwd=True)
    _same(ref, got)


@pytest.mark.parametrize("workers", [1, 7, 64])
def test_fused_bwd_independent_of_worker_count(workers):
    cfg, inp = _inputs(SHAPES[1], "bf16", seed=1)
    print(f"case fused bwd workers={workers}", flush=True)
    _same(_run(cfg, inp, fused_bwd=True), _run(cfg, inp, fused_bwd=True, workers=workers))


def test_fused_bwd_reruns_bit_identical():
    cfg, inp = _inputs(SHAPES[2], "bf16", seed=2)
    outs = [_run(cfg, inp, fused_bwd=True) for _ in range(3)]
    for b in outs[1:]:
        _same(outs[0], b)


def test_fused_bwd_matches_oracle():
    cfg, inp = _inputs(SHAPES[1], "bf16", seed=3)
    b = _run(cfg, inp, fused_bwd=True)
    fwd = O.forward(inp, cfg.K, "bf16")
    bwd = O.backward(inp, fwd, "bf16")
    R = cfg.T * cfg.K
    assert max_rel(host(b.dab)[:R], bwd["dab"], "bf16") <= 2e-2
    assert max_rel(host(b.dx_rows)[:R], bwd["dx_perm"], "bf16") <= 2e-2
    assert max_rel(host(b.dx), bwd["dx"], "bf16") <= 2e-2
    for n in ("dw1", "dw3", "dw2", "dws1", "dws3", "dws2"):
        assert f32_rel(host(getattr(b, n)), bwd[n]) <= 2e-2, n
    for e in np.nonzero(fwd["counts"] == 0)[0]:
        assert np.all(host(b.dw1)[e] == 0) and np.all(host(b.dw2)[e] == 0)
