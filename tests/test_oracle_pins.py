"""Pins of the CPU oracle against things other than itself.

Each test ties one part of the oracle to brute force, a closed form, an
invariant, a library routine (torch fp64 autograd / matmul / bf16 cast) or a
hand-worked fixture, chosen so that a plausible slip (dropped term, wrong
sign, transposed operand, wrong index, wrong tie-break) fails at least one.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def close(got, ref, rel):
    """Normwise check: max |got - ref| <= rel * max |ref|."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return np.max(np.abs(got - ref)) <= rel * max(np.max(np.abs(ref)), 1e-300)


def _small(T=24, H=16, E=5, K=2, I=12, Ns=0, dtype="f64", seed=0, logits=None):
    """Tiny random layer; f64 draws, stored in `dtype`."""
    g = np.random.default_rng(seed)
    inp = {
        "logits": (g.standard_normal((T, E)) if logits is None else logits).astype(np.float32),
        "x": O.store(g.standard_normal((T, H)), dtype),
        "w1": O.store(0.3 * g.standard_normal((E, H, I)), dtype),
        "w3": O.store(0.3 * g.standard_normal((E, H, I)), dtype),
        "w2": O.store(0.3 * g.standard_normal((E, I, H)), dtype),
        "dout": O.store(g.standard_normal((T, H)), dtype),
    }
    if Ns:
        inp["ws1"] = O.store(0.3 * g.standard_normal((Ns, H, I)), dtype)
        inp["ws3"] = O.store(0.3 * g.standard_normal((Ns, H, I)), dtype)
        inp["ws2"] = O.store(0.3 * g.standard_normal((Ns, I, H)), dtype)
    return inp


# ---------------------------------------------------------------- storage ---

def test_bf16_store_matches_torch_cast():
    g = np.random.default_rng(1)
    v = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                         3.3895313892515355e38]])
    mine = O.store(v, "bf16")
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # ties to even: 1 + 2^-8 is halfway between 1.0 and 1 + 2^-7 -> 1.0
    assert O.widen(O.store(np.array([1.0 + 2.0 ** -8]), "bf16"), "bf16")[0] == 1.0
    assert O.widen(O.store(np.array([1.0 + 3 * 2.0 ** -8]), "bf16"), "bf16")[0] == 1.0 + 2.0 ** -6


# ---------------------------------------------------------------- routing ---

def _brute_select(logits, K):
    T, E = logits.shape
    out = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        # python float compare: -0.0 == 0.0; sort key (-logit, id) is the tie rule
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        out[t] = order[:K]
    return out


@pytest.mark.parametrize("E,K", [(8, 2), (64, 6), (5, 5), (32, 4), (3, 1)])
def test_route_select_brute_force_with_ties(E, K):
    g = np.random.default_rng(E * 100 + K)
    T = 300
    # quantised logits force many ties; include signed zeros explicitly
    lq = g.integers(-1, 2, size=(T, E)).astype(np.float32)
    lq[g.random((T, E)) < 0.2] = -0.0
    lg = g.standard_normal((T, E)).astype(np.float32)
    for logits in (lq, lg):
        assert np.array_equal(O.route_select(logits, K), _brute_select(logits, K))


def test_route_all_equal_row_and_weight_closed_forms():
    T, E = 7, 9
    for K in (1, 2, 4, 9):
        idx, w = O.route(np.full((T, E), 0.25, np.float32), K)
        assert np.array_equal(idx, np.tile(np.arange(K), (T, 1)))
        assert np.allclose(w, 1.0 / K, rtol=0, atol=1e-7)
    g = np.random.default_rng(3)
    l = g.standard_normal((50, 6)).astype(np.float32)
    idx, w = O.route(l, 1)
    assert np.all(w == 1.0)                                # K = 1 -> weight exactly one
    idx, w = O.route(l, 2)
    l0 = np.take_along_axis(l, idx[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(l, idx[:, 1:].astype(np.int64), 1)[:, 0].astype(np.float64)
    assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-7, atol=0)
    idx, w = O.route(l, 4)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 4 * 2.0 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)                 # picks by descending logit


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = [[float(z) for z in part.split()] for part in v.split("|")]
    return vals


def test_golden_hand_worked_route_and_slots():
    g = _read_golden("route_slot_T4_E3_K2.txt")
    logits = np.array(g["logits"], dtype=np.float32)
    assert np.signbit(logits[2, 0]) and not np.signbit(logits[2, 1])
    idx, w = O.route(logits, 2)
    assert np.array_equal(idx, np.array(g["topk_idx"], dtype=np.int32))
    assert np.allclose(w, np.array(g["topk_w"]), rtol=1e-7, atol=0)
    counts, offsets, slot, slot_src = O.slot_map(idx, 3)
    assert counts.tolist() == [int(v) for v in g["counts"][0]]
    assert offsets.tolist() == [int(v) for v in g["offsets"][0]]
    assert np.array_equal(slot, np.array(g["slot"], dtype=np.int32))
    assert slot_src.tolist() == [int(v) for v in g["slot_src"][0]]


def test_golden_hand_worked_bf16_rounding_points():
    """One token through the whole bf16 layer, worked by hand: pins where the
    layer rounds (h from the unrounded a, b; y from the stored h; out rounded
    once; dy stored; da, db from the saved a, b; dx_perm one rounding of the
    two paths; dx from the stored dx_perm rows).  Moving any of these rounding
    points changes at least one value (each alternative is worked out in the
    fixture's comments)."""
    g = _read_golden("bf16_rounding_T1_H2_E2_K2_I1.txt")
    bf = lambda key, shape: O.store(np.array(g[key], dtype=np.float64).reshape(shape), "bf16")
    inp = {"logits": np.array(g["logits"], dtype=np.float32).reshape(1, 2),
           "x": bf("x", (1, 2)), "w1": bf("w1", (2, 2, 1)), "w3": bf("w3", (2, 2, 1)),
           "w2": bf("w2", (2, 1, 2)), "dout": bf("dout", (1, 2))}
    # every input is exactly representable in bf16
    for k in ("x", "w1", "w3", "w2", "dout"):
        assert np.array_equal(O.widen(inp[k], "bf16").ravel(), np.array(g[k]).ravel()), k
    f = O.forward(inp, 2, "bf16")
    b = O.backward(inp, f, "bf16")
    wid = lambda a: O.widen(a, "bf16")
    assert f["topk_idx"].tolist() == [[0, 1]]
    assert np.allclose(f["topk_w"].ravel(), np.array(g["topk_w"]).ravel(), rtol=1e-7, atol=0)
    assert f["slot"].tolist() == [[0, 1]]
    # bf16 storage points: exact bit equality with the hand-worked values
    assert np.array_equal(wid(f["ab"][:, 0]), np.array(g["a"]).ravel())
    assert np.array_equal(wid(f["ab"][:, 1]), np.array(g["b"]).ravel())
    assert np.array_equal(wid(f["h"][:, 0]), np.array(g["h"]).ravel())
    assert np.array_equal(wid(f["y"]), np.array(g["y"]).reshape(2, 2))
    assert np.array_equal(wid(f["out"]).ravel(), np.array(g["out"]).ravel())
    assert np.array_equal(wid(b["dy"]), np.array(g["dy"]).reshape(2, 2))
    assert np.array_equal(wid(b["dab"][:, 0]), np.array(g["da"]).ravel())
    assert np.array_equal(wid(b["dab"][:, 1]), np.array(g["db"]).ravel())
    assert np.array_equal(wid(b["dx_perm"]), np.array(g["dx_perm"]).reshape(2, 2))
    assert np.array_equal(wid(b["dx"]).ravel(), np.array(g["dx"]).ravel())
    # float32 gradients: fp64 sums of stored operands, one float32 rounding
    assert np.array_equal(b["dtopk_w"].ravel(), np.array(g["dtopk_w"], np.float32).ravel())
    assert np.array_equal(b["dw1"].reshape(2, 2), np.array(g["dw1"], np.float32).reshape(2, 2))
    assert np.array_equal(b["dw3"].reshape(2, 2), np.array(g["dw3"], np.float32).reshape(2, 2))
    assert np.array_equal(b["dw2"].reshape(2, 2), np.array(g["dw2"], np.float32).reshape(2, 2))
    assert np.allclose(b["dlogits"].ravel(), np.array(g["dlogits"]).ravel(), rtol=2e-7, atol=0)


# ---------------------------------------------------------------- slot map ---

def _cursor_map(idx, E):
    """Single pass, t ascending then k ascending, one cursor per expert."""
    T, K = idx.shape
    counts = [0] * E
    for t in range(T):
        for k in range(K):
            counts[idx[t, k]] += 1
    cur = [sum(counts[:e]) for e in range(E)]
    slot = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            slot[t, k] = cur[e]
            cur[e] += 1
    return slot


@pytest.mark.parametrize("T,E,K", [(1, 4, 2), (97, 8, 2), (200, 64, 6), (50, 5, 5)])
def test_slot_map_invariants_and_cursor_pass(T, E, K):
    g = np.random.default_rng(T + E)
    logits = g.standard_normal((T, E)).astype(np.float32)
    if E == 64:
        logits[:, :10] -= 100.0            # experts 0..9 never picked -> empty groups
    idx = O.route_select(logits, K)
    counts, offsets, slot, slot_src = O.slot_map(idx, E)
    R = T * K
    assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(slot.ravel()), np.arange(R))          # bijection
    assert np.array_equal(slot_src[slot], np.repeat(np.arange(T)[:, None], K, 1))
    for e in range(E):                                                   # expert-contiguous,
        toks = slot_src[offsets[e]:offsets[e + 1]]                       # ascending tokens
        assert np.all((idx[toks] == e).any(1))
        assert np.all(np.diff(toks) > 0)
    assert np.array_equal(slot, _cursor_map(idx, E))
    x = g.integers(0, 2 ** 16, size=(T, 3), dtype=np.uint16)
    xp = O.dispatch(x, slot)
    for k in range(K):
        assert np.array_equal(xp[slot[:, k]], x)                         # bit-exact copy


def test_slot_map_K_equals_E_every_expert_holds_all_tokens():
    T, E = 33, 4
    idx = O.route_select(np.random.default_rng(0).standard_normal((T, E)).astype(np.float32), E)
    counts, offsets, slot, slot_src = O.slot_map(idx, E)
    assert np.all(counts == T)
    for e in range(E):
        assert np.array_equal(slot_src[offsets[e]:offsets[e + 1]], np.arange(T))


@pytest.mark.parametrize("G", [1, 2, 3, 7, 16])
def test_algorithm1_multirank_equals_single_rank(G):
    g = np.random.default_rng(G)
    T, E, K = 129, 16, 4
    idx = O.route_select(g.standard_normal((T, E)).astype(np.float32), K)
    _, _, slot, _ = O.slot_map(idx, E)
    counts_rank, slot_g = O.slot_map_ranks(idx, E, G)
    assert counts_rank.shape == (G, E) and counts_rank.sum() == T * K
    assert np.array_equal(slot_g, slot)
    # base table, brute force: rank r's first slot in expert e is the slot of
    # its first pair routed to e (when it has one), and consecutive ranks'
    # bases differ by the lower rank's count; rank 0 starts at the offsets
    base = O.rank_base_offsets(counts_rank)
    counts, offsets, _, _ = O.slot_map(idx, E)
    assert np.array_equal(base[0], offsets[:-1])
    assert np.array_equal(np.diff(base, axis=0), counts_rank[:-1])
    bounds = [(T * r) // G for r in range(G + 1)]
    for r in range(G):
        for e in range(E):
            hit = [slot[t, k] for t in range(bounds[r], bounds[r + 1]) for k in range(K) if idx[t, k] == e]
            if hit:
                assert min(hit) == base[r, e]


# ---------------------------------------------------------------- forward ---

def _torch_layer(inp, K, Ns):
    """Independent fp64 torch composition of the layer (per token, no permutation)."""
    f = lambda a: torch.tensor(O.widen(a, "f64"), dtype=torch.float64, requires_grad=True)
    P = {k: f(v) for k, v in inp.items() if k != "dout"}
    P["logits"] = torch.tensor(inp["logits"].astype(np.float64), requires_grad=True)
    idx = torch.tensor(O.route_select(inp["logits"], K).astype(np.int64))
    w = torch.softmax(P["logits"].gather(1, idx), dim=1)
    w.retain_grad()
    x = P["x"]
    out = torch.zeros_like(x)
    for k in range(K):
        e = idx[:, k]
        a = torch.bmm(x[:, None, :], P["w1"][e])[:, 0]
        b = torch.bmm(x[:, None, :], P["w3"][e])[:, 0]
        h = torch.nn.functional.silu(a) * b
        out = out + w[:, k:k + 1] * torch.bmm(h[:, None, :], P["w2"][e])[:, 0]
    for s in range(Ns):
        h = torch.nn.functional.silu(x @ P["ws1"][s]) * (x @ P["ws3"][s])
        out = out + h @ P["ws2"][s]
    return out, P, w


@pytest.mark.parametrize("Ns", [0, 2])
def test_forward_and_backward_match_torch_autograd_f64(Ns):
    K = 3
    inp = _small(T=20, H=8, E=5, K=K, I=6, Ns=Ns, dtype="f64", seed=Ns)
    fwd = O.forward(inp, K, "f64")
    bwd = O.backward(inp, fwd, "f64")
    out, P, w = _torch_layer(inp, K, Ns)
    # the oracle keeps gate weights and weight/gate gradients in float32
    assert close(fwd["out"], out.detach().numpy(), 1e-6)
    (out * torch.tensor(inp["dout"])).sum().backward()
    assert close(bwd["dx"], P["x"].grad.numpy(), 1e-6)
    for n in ("w1", "w3", "w2", "logits"):
        assert close(bwd["d" + n], P[n].grad.numpy(), 1e-6), n
    assert close(bwd["dtopk_w"], w.grad.numpy(), 1e-6)
    if Ns:
        for n in ("ws1", "ws3", "ws2"):
            assert close(bwd["d" + n], P[n].grad.numpy(), 1e-6), n


def test_forward_f32_storage_matches_torch_within_rounding():
    K = 2
    inp = _small(T=40, H=16, E=6, K=K, I=24, dtype="f32", seed=5)
    fwd = O.forward(inp, K, "f32")
    out, _, _ = _torch_layer(inp, K, 0)
    ref = out.detach().numpy()
    assert np.max(np.abs(fwd["out"] - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_dense_closed_form_shared_weights():
    """All experts share W1, W3, W2 -> out = FFN(x) because the gate weights sum to one."""
    T, H, E, K, I = 30, 12, 6, 3, 10
    g = np.random.default_rng(9)
    W1, W3, W2 = (0.3 * g.standard_normal(s) for s in ((H, I), (H, I), (I, H)))
    inp = {"logits": g.standard_normal((T, E)).astype(np.float32),
           "x": g.standard_normal((T, H)),
           "w1": np.repeat(W1[None], E, 0), "w3": np.repeat(W3[None], E, 0),
           "w2": np.repeat(W2[None], E, 0), "dout": g.standard_normal((T, H))}
    fwd = O.forward(inp, K, "f64")
    xt = torch.tensor(inp["x"])
    dense = (torch.nn.functional.silu(xt @ torch.tensor(W1)) * (xt @ torch.tensor(W3))) @ torch.tensor(W2)
    assert np.allclose(fwd["out"], dense.numpy(), rtol=1e-6, atol=1e-9)
    bwd = O.backward(inp, fwd, "f64")
    # sum over experts of the weight gradients = the dense layer's weight gradients
    Wt = [torch.tensor(W, requires_grad=True) for W in (W1, W3, W2)]
    d = (torch.nn.functional.silu(xt @ Wt[0]) * (xt @ Wt[1])) @ Wt[2]
    (d * torch.tensor(inp["dout"])).sum().backward()
    for name, Wg in zip(("dw1", "dw3", "dw2"), Wt):
        assert np.allclose(bwd[name].sum(0), Wg.grad.numpy(), rtol=1e-5, atol=1e-7)
    # every expert returns the same row, so the gate gradient is zero
    assert np.max(np.abs(bwd["dlogits"])) < 1e-6


def test_combine_special_cases():
    g = np.random.default_rng(4)
    T, H = 10, 5
    y = g.standard_normal((T, H))
    slot = g.permutation(T).astype(np.int32)[:, None]
    out = O.combine(y, slot, np.ones((T, 1), np.float32), "f64")
    assert np.array_equal(out, y[slot[:, 0]])                  # K = 1 -> unpermute
    K = 3
    row = g.standard_normal(H)
    yy = np.tile(row, (T * K, 1))
    slot = g.permutation(T * K).astype(np.int32).reshape(T, K)
    idx, w = O.route(g.standard_normal((T, 7)).astype(np.float32), K)
    out = O.combine(yy, slot, w, "f64")
    assert np.allclose(out, np.tile(row, (T, 1)), rtol=1e-7)  # identical rows -> y


def test_empty_expert_has_exact_zero_weight_grads():
    T, E, K = 16, 6, 2
    logits = np.random.default_rng(2).standard_normal((T, E)).astype(np.float32)
    logits[:, 3] = -50.0
    inp = _small(T=T, E=E, K=K, dtype="bf16", logits=logits)
    fwd = O.forward(inp, K, "bf16")
    assert fwd["counts"][3] == 0
    bwd = O.backward(inp, fwd, "bf16")
    for n in ("dw1", "dw3", "dw2"):
        assert np.all(bwd[n][3] == 0)


def test_finite_differences_f64():
    """Central differences of L = <out, dout> against the oracle backward."""
    T, H, E, K, I = 8, 8, 4, 2, 8
    inp = _small(T=T, H=H, E=E, K=K, I=I, Ns=1, dtype="f64", seed=11)
    # keep every selection margin >> step so the routing does not flip
    l = inp["logits"].astype(np.float64)
    srt = np.sort(l, axis=1)
    assert np.min(np.diff(srt, axis=1)) > 1e-4
    fwd = O.forward(inp, K, "f64")
    bwd = O.backward(inp, fwd, "f64")

    def loss(mod):
        f = O.forward(mod, K, "f64")
        return float((f["out"] * inp["dout"]).sum())

    eps = 1e-6
    g = np.random.default_rng(0)
    checks = [("x", "dx"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2"), ("ws1", "dws1"),
              ("ws2", "dws2"), ("logits", "dlogits")]
    for name, gname in checks:
        for _ in range(6):
            arr = inp[name]
            pos = tuple(int(g.integers(0, n)) for n in arr.shape)
            step = 1e-3 if name == "logits" else eps      # logit margins are > 1e-4
            plus = {k: v.copy() for k, v in inp.items()}
            minus = {k: v.copy() for k, v in inp.items()}
            if name == "logits":
                plus[name] = plus[name].astype(np.float64)
                minus[name] = minus[name].astype(np.float64)
            plus[name][pos] += step
            minus[name][pos] -= step
            fd = (loss(plus) - loss(minus)) / (2 * step)
            an = float(bwd[gname][pos])
            tol = 1e-5 * max(1.0, abs(fd)) if name != "logits" else 1e-4 * max(1.0, abs(fd))
            assert abs(fd - an) <= tol, (name, pos, fd, an)


# ------------------------------------------------------- subset evaluation ---

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_token_and_column_subsets_agree_with_full_pipeline(dtype):
    K, Ns = 3, 1
    inp = _small(T=30, H=16, E=5, K=K, I=12, Ns=Ns, dtype=dtype, seed=21)
    fwd = O.forward(inp, K, dtype)
    bwd = O.backward(inp, fwd, dtype)
    wid = lambda a: O.widen(a, dtype)
    sel = np.array([0, 7, 29])
    out_t, _ = O.tokens_forward(inp["x"][sel], fwd["topk_idx"][sel], fwd["topk_w"][sel], inp, dtype)
    ref = wid(fwd["out"][sel])
    assert np.max(np.abs(wid(out_t) - ref)) <= 1e-2 * np.max(np.abs(ref))
    dx_t, dw_t = O.tokens_backward(inp["x"][sel], inp["dout"][sel], fwd["topk_idx"][sel],
                                   fwd["topk_w"][sel], inp, dtype)
    ref = wid(bwd["dx"][sel])
    assert np.max(np.abs(wid(dx_t) - ref)) <= 1e-2 * np.max(np.abs(ref))
    assert close(dw_t, bwd["dtopk_w"][sel], 1e-2)
    cols = np.array([0, 5, 11])
    for e in range(5):
        lo, hi = fwd["offsets"][e], fwd["offsets"][e + 1]
        if hi == lo:
            continue
        d1, d3, d2 = O.expert_wgrad_columns(fwd["x_perm"][lo:hi], bwd["dy"][lo:hi], inp["w1"][e],
                                            inp["w3"][e], inp["w2"][e], cols, dtype)
        for got, ref in ((d1, bwd["dw1"][e][:, cols]), (d3, bwd["dw3"][e][:, cols]),
                         (d2, bwd["dw2"][e][cols, :])):
            assert np.max(np.abs(got - ref)) <= 1e-2 * np.max(np.abs(ref)) + 1e-6


def test_synth_is_seeded_and_shaped():
    cfg = synth.Config("small", 77, 64, 256, 8, 3, 128, 2, 128, "bf16", "fwd+bwd", "gauss")
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["x"].dtype == np.uint16 and a["x"].shape == (64, 256)
    assert a["ws1"].shape == (2, 256, 128) and a["dout"].shape == (64, 256)
    assert a["w2"].shape == (8, 128, 256) and a["logits"].dtype == np.float32
    # Zipf(1.2) recipe of the skewed workload: 8 experts never picked, a heavy head
    z = synth._zipf_logits(np.random.SeedSequence(5), 4096, 64)
    idx = O.route_select(z, 6)
    counts = np.bincount(idx.ravel(), minlength=64)
    assert (counts == 0).sum() == 8 and counts.max() > 4 * counts[counts > 0].mean()
