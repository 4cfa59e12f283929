"""Every workload at its full size, run through the C ABI in the launch
configuration the benchmark times (fused forward, then the backward calls),
checked against the oracle.

At these sizes the oracle cannot run the whole layer, so the check is:
routing, counts, offsets, slot map and its inverse in full (bit-exact); a
seeded sample of permuted rows (bit-exact); a seeded sample of tokens whose
outputs, input gradients and gate gradients the oracle evaluates one by one
from the definition (normwise max-rel-err <= 2e-2 for bf16, max-abs-err <=
1e-5 for the fp32 workload); a seeded sample of intermediate units whose
columns of dW1/dW3 and rows of dW2 the oracle forms for sampled experts, and
the weight gradients of whole experts (two at the long-sequence size, where
the token sample is 4096, one elsewhere).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from combine_moe_route_histogram_amd import layer as L
from gpu_util import f32_rel, host, max_rel

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _run(cfg, inp, fused=True, backward=True):
    d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
    p = {k: synth.to_torch(v, "cuda") for k, v in inp.items()}
    b = L.Buffers(d, backward=backward)
    L.forward(b, p, fused=fused)
    if backward:
        L.backward(b, p, fused=fused)
    torch.cuda.synchronize()
    return d, b


def _rows(t, idx):
    return host(t[torch.as_tensor(idx, device=t.device, dtype=torch.long)])


@pytest.mark.parametrize("name", ["mixtral", "dsv3", "skewed", "longseq"])
def test_full_size_workload(name):
    cfg = synth.config(name)
    backward = "bwd" in cfg.passes
    print(f"case workload={name} T={cfg.T} H={cfg.H} E={cfg.E} K={cfg.K} I={cfg.I}", flush=True)
    inp = synth.make_inputs(cfg, with_grad=backward)
    d, b = _run(cfg, inp, fused=True, backward=backward)
    dt, K, E, T = cfg.dtype, cfg.K, cfg.E, cfg.T
    rng = np.random.default_rng(cfg.seed)

    # routing and the slot map, in full
    idx, w = O.route(inp["logits"], K)
    counts, offsets, slot, slot_src = O.slot_map(idx, E)
    assert np.array_equal(host(b.topk_idx), idx)
    assert np.max(np.abs(host(b.topk_w) - w)) <= 1e-6
    assert np.array_equal(host(b.counts), counts)
    assert np.array_equal(host(b.offsets), offsets)
    assert np.array_equal(host(b.slot), slot)
    assert np.array_equal(host(b.slot_src), slot_src)
    if name == "skewed":
        assert (counts == 0).sum() == 8            # empty groups exercised

    # permuted rows (bit copies)
    ss = np.sort(rng.choice(d.R, size=min(d.R, 2048), replace=False))
    assert np.array_equal(_rows(b.x_perm, ss), inp["x"][slot_src[ss]])

    # token outputs from the definition
    # 4096 sampled tokens at the long-sequence size, 256 elsewhere
    toks = np.sort(rng.choice(T, size=4096 if name == "longseq" else 256, replace=False))
    out_ref, _ = O.tokens_forward(inp["x"][toks], idx[toks], w[toks], inp, dt)
    assert max_rel(_rows(b.out, toks), out_ref, dt) <= BF16_TOL

    if not backward:
        return
    dx_ref, dw_ref = O.tokens_backward(inp["x"][toks], inp["dout"][toks], idx[toks], w[toks], inp, dt)
    assert max_rel(_rows(b.dx, toks), dx_ref, dt) <= BF16_TOL
    assert f32_rel(_rows(b.dtopk_w, toks), dw_ref) <= BF16_TOL
    dl_ref = O.route_bwd(dw_ref, w[toks], idx[toks], E)
    assert f32_rel(_rows(b.dlogits, toks), dl_ref) <= BF16_TOL

    # weight-gradient columns of sampled experts and intermediate units
    cols = np.sort(rng.choice(cfg.I, size=8, replace=False))
    experts = np.sort(rng.choice(np.nonzero(counts)[0], size=min(3, int((counts > 0).sum())), replace=False))
    g64 = O.widen(inp["dout"], dt)
    for e in experts:
        rows = np.arange(offsets[e], offsets[e + 1])
        toks_e = slot_src[rows]
        k_e = np.argmax(idx[toks_e] == e, axis=1)
        X = inp["x"][toks_e]
        DY = O.store(w[toks_e, k_e].astype(np.float64)[:, None] * g64[toks_e], dt)
        d1, d3, d2 = O.expert_wgrad_columns(X, DY, inp["w1"][e], inp["w3"][e], inp["w2"][e], cols, dt)
        e_t = torch.tensor(int(e))
        assert f32_rel(host(b.dw1[e_t][:, torch.as_tensor(cols)]), d1) <= BF16_TOL
        assert f32_rel(host(b.dw3[e_t][:, torch.as_tensor(cols)]), d3) <= BF16_TOL
        assert f32_rel(host(b.dw2[e_t][torch.as_tensor(cols)]), d2) <= BF16_TOL
    # whole routed experts' weight gradients: two at the long-sequence size, one elsewhere
    for e in experts[: 2 if name == "longseq" else 1]:
        e = int(e)
        rows = np.arange(offsets[e], offsets[e + 1])
        toks_e = slot_src[rows]
        k_e = np.argmax(idx[toks_e] == e, axis=1)
        DY = O.store(w[toks_e, k_e].astype(np.float64)[:, None] * g64[toks_e], dt)
        d1, d3, d2 = O.expert_wgrad_columns(inp["x"][toks_e], DY, inp["w1"][e], inp["w3"][e],
                                            inp["w2"][e], np.arange(cfg.I), dt)
        e_t = torch.tensor(e)
        assert f32_rel(host(b.dw1[e_t]), d1) <= BF16_TOL
        assert f32_rel(host(b.dw3[e_t]), d3) <= BF16_TOL
        assert f32_rel(host(b.dw2[e_t]), d2) <= BF16_TOL
    for s in range(cfg.n_shared):
        sub = {"w1": inp["ws1"], "w3": inp["ws3"], "w2": inp["ws2"]}
        d1, d3, d2 = O.expert_wgrad_columns(inp["x"], inp["dout"], sub["w1"][s], sub["w3"][s],
                                            sub["w2"][s], cols, dt)
        s_t = torch.tensor(s)
        assert f32_rel(host(b.dws1[s_t][:, torch.as_tensor(cols)]), d1) <= BF16_TOL
        assert f32_rel(host(b.dws3[s_t][:, torch.as_tensor(cols)]), d3) <= BF16_TOL
        assert f32_rel(host(b.dws2[s_t][torch.as_tensor(cols)]), d2) <= BF16_TOL


def test_tiny_fp32_workload_in_full():
    """The fp32 workload is small enough for the whole oracle: max-abs-err <= 1e-5."""
    cfg = synth.config("tiny")
    inp = synth.make_inputs(cfg, with_grad=True)
    for fused in (False, True):
        d, b = _run(cfg, inp, fused=fused, backward=True)
        fwd = O.forward(inp, cfg.K, "f32")
        bwd = O.backward(inp, fwd, "f32")
        assert np.array_equal(host(b.slot), fwd["slot"])
        assert np.array_equal(host(b.x_perm), fwd["x_perm"])
        assert np.max(np.abs(host(b.out) - fwd["out"])) <= 1e-5
        assert np.max(np.abs(host(b.y)[: d.R] - fwd["y"])) <= 1e-5
        assert np.max(np.abs(host(b.dx) - bwd["dx"])) <= 1e-5
        for n in ("dw1", "dw3", "dw2"):
            assert np.max(np.abs(host(getattr(b, n)) - bwd[n])) <= 1e-5, n
        assert np.max(np.abs(host(b.dlogits) - bwd["dlogits"])) <= 1e-5


def test_full_size_reruns_bit_identical():
    """Two full Mixtral-like steps give the same bits in every output."""
    cfg = synth.config("mixtral")
    inp = synth.make_inputs(cfg, with_grad=True)
    _, b1 = _run(cfg, inp)
    names = ("slot", "x_perm", "ab", "h", "y", "out", "dy", "dtopk_w", "dab", "dx_rows", "dx",
             "dlogits", "dw1", "dw3", "dw2")
    first = {n: getattr(b1, n).clone() for n in names}
    del b1
    _, b2 = _run(cfg, inp)
    for n in names:
        assert torch.equal(first[n], getattr(b2, n)), n


@pytest.mark.parametrize("name", ["mixtral", "dsv3"])
def test_full_size_one_launch_backward_bitwise(name):
    """At the benchmarked sizes the one-launch backward gives the bits of the
    plain B then W calls."""
    cfg = synth.config(name)
    print(f"case one-launch backward workload={name}", flush=True)
    inp = synth.make_inputs(cfg, with_grad=True)
    d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
    p = {k: synth.to_torch(v, "cuda") for k, v in inp.items()}
    b = L.Buffers(d)
    L.forward(b, p, fused=True)
    outs = ("dab", "dx_rows", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2", "dx")
    L.backward(b, p, fused=False)
    torch.cuda.synchronize()
    ref = {n: getattr(b, n).clone() for n in outs if getattr(b, n) is not None}
    for n in ref:
        getattr(b, n).fill_(7)
    L.backward(b, p, fused=True)
    torch.cuda.synchronize()
    for n, t in ref.items():
        assert torch.equal(t, getattr(b, n)), n
