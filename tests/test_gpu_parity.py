"""GPU path vs the CPU oracle, element by element, on shapes the oracle runs
in seconds: several tiles, ragged row tiles, partial N tiles, empty experts, a
single expert, shared experts, both storage dtypes.

Bar: indices, counts, offsets, slots and the permuted rows bit-exact; every
float tensor, intermediates included, within max-abs-err 1e-5 (f32 storage)
or normwise max-rel-err 2e-2 (bf16 storage), the bars of the fp32 and bf16
workloads.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import custom_config, f32_rel, host, max_abs, max_rel, run_layer
import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5

SHAPES = [
    # T,   H,   E,  K,  I,  Ns
    (300, 256, 8, 2, 320, 0),     # ragged rows, partial N tiles (I = 5*64)
    (257, 128, 5, 3, 192, 2),     # shared experts, odd E
    (64, 64, 1, 1, 64, 0),        # one expert, one tile
    (1, 128, 4, 2, 128, 0),       # a single token
    (520, 192, 16, 4, 128, 0),    # skewed: empty and huge experts (see logits below)
    (96, 64, 32, 20, 64, 1),      # more rows per token than 16-byte vectors per row
    (200, 200, 6, 2, 136, 0),     # H, I multiples of 8, not of the 64-wide k slice
    (150, 72, 4, 2, 88, 1),       # the same with a shared expert
    (2400, 64, 1, 1, 64, 1),      # groups of 10 row tiles: split into several bands
    (2200, 64, 2, 2, 64, 0),      # two experts of 2200 rows (9 row tiles) each
    (33, 8, 4, 2, 8, 1),          # smallest H and I: one 16-byte vector per bf16 row
    (20, 16, 3, 3, 24, 0),        # K = E, H and I below the vector count of a wave
    (50, 64, 4, 2, 64, 8),        # the maximum of 8 shared experts (10 rows per token)
    (40, 64, 100, 70, 64, 1),     # K > 64: a token's pairs span two 64-lane chunks
]


def _inputs(shape, dtype, seed=0):
    T, H, E, K, I, Ns = shape
    cfg = custom_config(T, H, E, K, I, Ns, dtype, number=100 + seed)
    inp = synth.make_inputs(cfg, with_grad=True)
    if E == 16:
        l = inp["logits"]
        l[:, [3, 7, 11]] = -30.0            # three empty experts
        l[: T // 2, 5] += 8.0               # expert 5 takes half the tokens
    return cfg, inp


def _check(name, got, ref, dtype):
    if dtype == "f32":
        err = max_abs(got, ref)
        assert err <= F32_TOL, (name, err)
    else:
        err = max_rel(got, ref, dtype)
        assert err <= BF16_TOL, (name, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_layer_forward_backward_matches_oracle(shape, dtype):
    cfg, inp = _inputs(shape, dtype)
    print(f"case shape={shape} dtype={dtype}", flush=True)
    d, b = run_layer(cfg, inp)
    fwd = O.forward(inp, cfg.K, dtype)
    bwd = O.backward(inp, fwd, dtype)
    R = d.R
    # exact parts
    assert np.array_equal(host(b.topk_idx), fwd["topk_idx"])
    assert np.array_equal(host(b.counts), fwd["counts"])
    assert np.array_equal(host(b.offsets), fwd["offsets"])
    assert np.array_equal(host(b.slot), fwd["slot"])
    assert np.array_equal(host(b.slot_src), fwd["slot_src"])
    assert np.array_equal(host(b.x_perm), fwd["x_perm"])
    assert np.max(np.abs(host(b.topk_w) - fwd["topk_w"])) <= 1e-6
    # forward floats
    I = cfg.I
    ab, h, y = host(b.ab), host(b.h), host(b.y)
    _check("a", ab[:R, :I], fwd["ab"][:, :I], dtype)
    _check("b", ab[:R, I:], fwd["ab"][:, I:], dtype)
    _check("h", h[:R], fwd["h"], dtype)
    _check("y", y[:R], fwd["y"], dtype)
    if cfg.n_shared:
        T, Ns = cfg.T, cfg.n_shared
        _check("ab_sh", ab[R:].reshape(Ns, T, 2 * I), fwd["ab_sh"], dtype)
        _check("h_sh", h[R:].reshape(Ns, T, I), fwd["h_sh"], dtype)
        _check("y_sh", y[R:].reshape(Ns, T, -1), fwd["y_sh"], dtype)
    _check("out", host(b.out), fwd["out"], dtype)
    # backward
    _check("dy", host(b.dy), bwd["dy"], dtype)
    dab, dx_rows = host(b.dab), host(b.dx_rows)
    _check("dab", dab[:R], bwd["dab"], dtype)
    _check("dx_perm", dx_rows[:R], bwd["dx_perm"], dtype)
    if cfg.n_shared:
        T, Ns = cfg.T, cfg.n_shared
        _check("dab_sh", dab[R:].reshape(Ns, T, 2 * I), bwd["dab_sh"], dtype)
        _check("dx_sh", dx_rows[R:].reshape(Ns, T, -1), bwd["dx_sh"], dtype)
    _check("dx", host(b.dx), bwd["dx"], dtype)
    # float32 outputs of both storage dtypes: gate-weight, weight and logit
    # gradients (max-abs for the f32 layer, normwise for the bf16 one)
    f32_out = ["dtopk_w", "dw1", "dw3", "dw2", "dlogits"]
    if cfg.n_shared:
        f32_out += ["dws1", "dws3", "dws2"]
    for n in f32_out:
        got, ref = host(getattr(b, n)), bwd[n]
        err = max_abs(got, ref) if dtype == "f32" else f32_rel(got, ref)
        assert err <= (F32_TOL if dtype == "f32" else BF16_TOL), (n, err)
    # empty experts get exact zero weight gradients
    for e in np.nonzero(fwd["counts"] == 0)[0]:
        assert np.all(host(b.dw1)[e] == 0) and np.all(host(b.dw2)[e] == 0)


def test_reruns_are_bit_identical():
    cfg, inp = _inputs(SHAPES[1], "bf16", seed=3)
    _, b1 = run_layer(cfg, inp)
    _, b2 = run_layer(cfg, inp)
    for name in ("topk_idx", "topk_w", "slot", "slot_src", "x_perm", "ab", "h", "y", "out", "dy",
                 "dtopk_w", "dab", "dx_rows", "dx", "dlogits", "dw1", "dw3", "dw2", "dws1", "dws3",
                 "dws2"):
        assert torch.equal(getattr(b1, name), getattr(b2, name)), name


ROUTE_CASES = [
    # T, E, K, logits kind
    (1, 1, 1, "gauss"), (255, 8, 2, "ties"), (256, 8, 2, "gauss"), (257, 8, 2, "ties"),
    (1000, 64, 6, "ties"), (700, 64, 6, "gauss"), (333, 3, 3, "ties"), (512, 256, 8, "gauss"),
    (600, 100, 7, "ties"), (64, 32, 32, "ties"), (300, 17, 5, "equal"), (2000, 128, 64, "ties"),
    (300, 128, 65, "gauss"), (200, 256, 256, "ties"), (150, 200, 130, "equal"), (90, 70, 70, "gauss"),
]


LANE_CASES = [(131072, 32, 4, "gauss"), (5000, 8, 2, "ties"), (3001, 16, 8, "ties"),
              (777, 32, 8, "equal"), (129, 20, 3, "gauss"), (64, 5, 5, "ties")]


@pytest.mark.parametrize("case", LANE_CASES, ids=[str(c) for c in LANE_CASES])
def test_route_lane_and_group_topk_agree(case):
    """E <= 32 and K <= 8 take the top-k with one lane per token; the same
    logits padded to 33 experts with -inf columns (never picked) take the
    group kernel.  The picks must match the oracle and the two kernels must
    give the same bits, weights included."""
    from combine_moe_route_histogram_amd import layer as L
    T, E, K, kind = case
    g = np.random.default_rng(T + 31 * E + K)
    if kind == "gauss":
        logits = g.standard_normal((T, E)).astype(np.float32)
    elif kind == "ties":
        logits = g.integers(-1, 2, size=(T, E)).astype(np.float32)
        logits[g.random((T, E)) < 0.25] = -0.0
    else:
        logits = np.full((T, E), 0.5, np.float32)
    padded = np.full((T, 33), -np.inf, np.float32)
    padded[:, :E] = logits
    out = []
    for lg in (logits, padded):
        d = L.make_dims(T, 64, lg.shape[1], K, 64, 0, "bf16")
        b = L.Buffers(d, backward=False)
        print(f"case lane/group top-k T={T} E={lg.shape[1]} K={K} {kind}", flush=True)
        L.route(b, {"logits": torch.from_numpy(lg).cuda()})
        torch.cuda.synchronize()
        out.append((host(b.topk_idx), host(b.topk_w)))
    idx, w = O.route(logits, K)
    assert np.array_equal(out[0][0], idx)
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][1].view(np.uint32), out[1][1].view(np.uint32))
    assert np.max(np.abs(out[0][1] - w)) <= 1e-6


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[str(c) for c in ROUTE_CASES])
def test_route_bit_exact(case):
    from combine_moe_route_histogram_amd import layer as L
    T, E, K, kind = case
    g = np.random.default_rng(T * 7 + E)
    if kind == "gauss":
        logits = g.standard_normal((T, E)).astype(np.float32)
    elif kind == "ties":
        logits = g.integers(-1, 2, size=(T, E)).astype(np.float32)
        logits[g.random((T, E)) < 0.25] = -0.0
    else:
        logits = np.full((T, E), 0.5, np.float32)
    d = L.make_dims(T, 64, E, K, 64, 0, "bf16")
    b = L.Buffers(d, backward=False)
    L.route(b, {"logits": torch.from_numpy(logits).cuda()})
    torch.cuda.synchronize()
    idx, w = O.route(logits, K)
    counts, offsets, slot, slot_src = O.slot_map(idx, E)
    assert np.array_equal(host(b.topk_idx), idx)
    assert np.max(np.abs(host(b.topk_w) - w)) <= 1e-6
    assert np.array_equal(host(b.counts), counts)
    assert np.array_equal(host(b.offsets), offsets)
    assert np.array_equal(host(b.slot), slot)
    assert np.array_equal(host(b.slot_src), slot_src)
