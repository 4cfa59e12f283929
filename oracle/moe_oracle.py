"""CPU oracle of the MoE expert layer (route -> permute -> per-expert SwiGLU FFN
-> combine, forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never imports or calls it, and this module imports nothing
from the product path: the two share no code.

It is the plain sequential definition of the layer, written from the pages:

* UniEP article ("UniEP: Unified Expert-Parallel MoE MegaKernel for LLM
  Training"), section 1.1 and Figure 1: a gating network scores every expert
  for every token, top-k picks the experts, tokens are reordered and sent to
  their experts (dispatch), a grouped GEMM, SwiGLU and a second grouped GEMM
  back to the model dim run per expert, and the results are weighted by the
  gate scores and summed (combine).  The backward mirrors the forward; weight
  gradients are a transposed grouped GEMM summed over each expert's tokens.
* Same article, section 2.2, "deterministic token mapping" (Algorithm 1):
  a local stable sort by expert, the per-expert counts, and prefix-sum base
  offsets give every (token, k) pair a unique, order-fixed slot.
* GraphPP article, section 5.1/5.2: the SwiGLU MLP -- gate projection w1,
  up projection w3, SiLU, gate product, down projection w2; grad_w2 is
  h^T @ grad_out, grad_w1/grad_w3 come from x^T and the intermediate
  gradients, and grad_x is the sum of two paths.  The h^T @ grad_out form
  fixes the weight orientation y = x @ W, i.e. W1, W3 are [H, I] and W2 is
  [I, H].

Readings where the pages are silent are listed in the repository's design
notes; in short: logits are the given f32 router outputs; selection is by
logit, descending, ties to the lower expert id, -0.0 equal to +0.0; gate
weights are the softmax over the K selected logits; slots within an expert
are in ascending (token, k) order; shared experts have weight 1 and are added
after the routed sum.

Numerics: every sum is accumulated in float64 (numpy matmul of float64
operands, a library primitive, or explicit float64 sums).  Results are
rounded to the storage dtype only at the layer's storage points (x_perm, the
saved a/b, h, y, out, dy, da/db, dx_perm, dx); weight and gate gradients are
float32.  Storage dtypes: "f64" (no rounding; used by the derivative pins),
"f32", and "bf16" (numpy uint16 holding bf16 bits; float64 -> float32 ->
bfloat16, each step round-to-nearest-even).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# storage dtypes
# ---------------------------------------------------------------------------


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (exact)."""
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def store(v: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage dtype, round to nearest even at each narrowing."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f64":
        return v.copy()
    f = v.astype(np.float32)
    if dtype == "f32":
        return f
    if dtype == "bf16":
        u = f.view(np.uint32).astype(np.uint64)
        # round to nearest, ties to even, on the 16 bits that are dropped
        u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        return u.astype(np.uint16)
    raise ValueError(dtype)


def storage_zeros(shape, dtype: str) -> np.ndarray:
    return np.zeros(shape, dtype={"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[dtype])


def _silu(a):
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def _sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


# ---------------------------------------------------------------------------
# routing: gate top-k and gate weights (UniEP section 1.1)
# ---------------------------------------------------------------------------


def route_select(logits: np.ndarray, K: int) -> np.ndarray:
    """K experts per token by repeated arg-max over the f32 logits.

    A logit beats another if it is larger, or equal and its expert id is
    lower (-0.0 and +0.0 are equal).  Picks are recorded in selection order,
    so topk_idx[t] is by descending logit.  Inputs must be finite.
    """
    work = np.array(logits, dtype=np.float64)          # exact copy of f32 values
    T, E = work.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    idx = np.empty((T, K), dtype=np.int32)
    rows = np.arange(T)
    for k in range(K):
        j = np.argmax(work, axis=1)                     # first maximum = lowest id
        idx[:, k] = j
        work[rows, j] = -np.inf                         # an expert is picked once
    return idx


def route_weights(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """Softmax over the K selected logits (float64, stored as float32).

    w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), with l_0 the largest selected
    logit, so the weights of a token sum to one.
    """
    l = np.take_along_axis(np.asarray(logits, dtype=np.float64), topk_idx.astype(np.int64), axis=1)
    z = np.exp(l - l[:, :1])
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def route(logits: np.ndarray, K: int):
    idx = route_select(logits, K)
    return idx, route_weights(logits, idx)


# ---------------------------------------------------------------------------
# deterministic slot map: UniEP section 2.2, Algorithm 1 (one rank)
# ---------------------------------------------------------------------------


def slot_map(topk_idx: np.ndarray, E: int):
    """counts, offsets, slot[T,K] and its inverse slot_src[R] for one rank.

    counts[e] is the histogram of the selected experts; offsets is its
    exclusive prefix sum (offsets[E] = R).  The (token, k) pairs are taken in
    t-major, k-minor order and stably sorted by expert; the position of a pair
    in the sorted list is its slot, i.e. offsets[e] plus its stable-sort index
    inside expert e.  slot_src[s] is the token whose row lands in slot s.
    """
    T, K = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")             # local stable sort by expert
    slot_flat = np.empty(T * K, dtype=np.int32)
    slot_flat[order] = np.arange(T * K, dtype=np.int32)
    slot = slot_flat.reshape(T, K)
    slot_src = (order // K).astype(np.int32)
    return counts, offsets, slot, slot_src


def rank_base_offsets(counts_rank: np.ndarray) -> np.ndarray:
    """Algorithm 1's base offsets from the gathered [G, E] count table: rank r's
    first slot in expert e = the expert's start in the shared buffer (the
    exclusive prefix of the expert totals) + the counts of lower ranks for e."""
    c = counts_rank.astype(np.int64)
    G, E = c.shape
    total = c.sum(axis=0)
    expert_start = np.concatenate([[0], np.cumsum(total)[:-1]])
    lower = np.concatenate([np.zeros((1, E), np.int64), np.cumsum(c, axis=0)[:-1]])
    return (expert_start[None, :] + lower).astype(np.int32)


def slot_map_ranks(topk_idx: np.ndarray, E: int, G: int):
    """Algorithm 1 with G ranks, each holding a contiguous block of tokens.

    Every rank stably sorts its own (token, k) pairs by expert; the per-rank
    counts are gathered into a [G, E] table; the base offset of rank r in
    expert e is the sum of the counts of lower ranks for e (plus the expert's
    start offset, since all experts share one buffer here).  slot = base +
    local stable-sort index.  Returns (counts_by_rank[G,E], slot[T,K]).
    """
    T, K = topk_idx.shape
    bounds = [(T * r) // G for r in range(G + 1)]
    local = []
    counts_rank = np.zeros((G, E), dtype=np.int64)
    for r in range(G):
        sel = topk_idx[bounds[r]:bounds[r + 1]].reshape(-1).astype(np.int64)
        counts_rank[r] = np.bincount(sel, minlength=E)
        order = np.argsort(sel, kind="stable")
        rank_in_expert = np.empty_like(order)
        # stable-sort index inside each expert = position in sorted list - start of that expert
        start = np.concatenate([[0], np.cumsum(counts_rank[r])[:-1]])
        rank_in_expert[order] = np.arange(order.size) - start[sel[order]]
        local.append((sel, rank_in_expert))
    base = rank_base_offsets(counts_rank).astype(np.int64)
    slot = np.empty(T * K, dtype=np.int64)
    for r in range(G):
        sel, rie = local[r]
        slot[bounds[r] * K:bounds[r + 1] * K] = base[r, sel] + rie
    return counts_rank.astype(np.int32), slot.reshape(T, K).astype(np.int32)


# ---------------------------------------------------------------------------
# forward: dispatch, per-expert SwiGLU FFN, combine (UniEP 1.1; GraphPP 5.x)
# ---------------------------------------------------------------------------


def dispatch(x: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """x_perm[slot[t,k]] = x[t]: expert-contiguous rows, no padding."""
    T, K = slot.shape
    x_perm = np.empty((T * K,) + x.shape[1:], dtype=x.dtype)
    for k in range(K):
        x_perm[slot[:, k]] = x
    return x_perm


def swiglu_up(X: np.ndarray, W1e: np.ndarray, W3e: np.ndarray, dtype: str):
    """a = X W1e, b = X W3e, h = silu(a) * b for one expert's rows.

    a and b are float64 sums of storage-dtype operands; h is formed from the
    unrounded a and b.  Returns stored (a, b, h).
    """
    Xf = widen(X, dtype)
    a = Xf @ widen(W1e, dtype)
    b = Xf @ widen(W3e, dtype)
    h = _silu(a) * b
    return store(a, dtype), store(b, dtype), store(h, dtype)


def down_proj(Hs: np.ndarray, W2e: np.ndarray, dtype: str) -> np.ndarray:
    """y = h W2e from the stored h."""
    return store(widen(Hs, dtype) @ widen(W2e, dtype), dtype)


def expert_ffn(x_perm, x, offsets, w1, w3, w2, dtype, ws1=None, ws3=None, ws2=None):
    """Per-expert SwiGLU FFN over expert-contiguous rows (+ shared experts).

    Returns a dict: ab [R, 2I] (a then b, stored), h [R, I], y [R, H], and for
    shared experts ab_sh [Ns, T, 2I], h_sh [Ns, T, I], y_sh [Ns, T, H].
    An expert with no rows contributes nothing.
    """
    E = w1.shape[0]
    R, H = x_perm.shape
    I = w1.shape[2]
    ab = storage_zeros((R, 2 * I), dtype)
    h = storage_zeros((R, I), dtype)
    y = storage_zeros((R, H), dtype)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a_e, b_e, h_e = swiglu_up(x_perm[lo:hi], w1[e], w3[e], dtype)
        ab[lo:hi, :I], ab[lo:hi, I:], h[lo:hi] = a_e, b_e, h_e
        y[lo:hi] = down_proj(h_e, w2[e], dtype)
    res = {"ab": ab, "h": h, "y": y}
    if ws1 is not None and ws1.shape[0] > 0:
        Ns, T = ws1.shape[0], x.shape[0]
        Is = ws1.shape[2]
        res["ab_sh"] = storage_zeros((Ns, T, 2 * Is), dtype)
        res["h_sh"] = storage_zeros((Ns, T, Is), dtype)
        res["y_sh"] = storage_zeros((Ns, T, H), dtype)
        for s in range(Ns):
            a_s, b_s, h_s = swiglu_up(x, ws1[s], ws3[s], dtype)
            res["ab_sh"][s, :, :Is], res["ab_sh"][s, :, Is:], res["h_sh"][s] = a_s, b_s, h_s
            res["y_sh"][s] = down_proj(h_s, ws2[s], dtype)
    return res


def combine(y, slot, topk_w, dtype, y_sh=None):
    """out[t] = sum_k w[t,k] y[slot[t,k]] (k = 0..K-1), then + sum_s y_sh[s,t].

    Float64 accumulation in that fixed order, one rounding at the end.
    """
    T, K = slot.shape
    acc = np.zeros((T, y.shape[1]), dtype=np.float64)
    for k in range(K):
        acc += topk_w[:, k].astype(np.float64)[:, None] * widen(y[slot[:, k]], dtype)
    if y_sh is not None:
        for s in range(y_sh.shape[0]):
            acc += widen(y_sh[s], dtype)
    return store(acc, dtype)


def forward(inp: dict, K: int, dtype: str) -> dict:
    """Whole forward pass; returns every intermediate the backward needs."""
    idx, w = route(inp["logits"], K)
    E = inp["w1"].shape[0]
    counts, offsets, slot, slot_src = slot_map(idx, E)
    x_perm = dispatch(inp["x"], slot)
    ffn = expert_ffn(x_perm, inp["x"], offsets, inp["w1"], inp["w3"], inp["w2"], dtype,
                     inp.get("ws1"), inp.get("ws3"), inp.get("ws2"))
    out = combine(ffn["y"], slot, w, dtype, ffn.get("y_sh"))
    res = dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets, slot=slot,
               slot_src=slot_src, x_perm=x_perm, out=out)
    res.update(ffn)
    return res


# ---------------------------------------------------------------------------
# backward (UniEP 1.1: mirror of the forward, transposed grouped GEMM for the
# weight gradients; GraphPP 5.1/5.2: SwiGLU backward, B/W split)
# ---------------------------------------------------------------------------


def combine_bwd(dout, y, slot, topk_w, dtype):
    """dy[slot[t,k]] = w[t,k] dout[t];  dw[t,k] = <dout[t], y[slot[t,k]]>."""
    T, K = slot.shape
    g = widen(dout, dtype)
    dy = storage_zeros((T * K, dout.shape[1]), dtype)
    dw = np.empty((T, K), dtype=np.float32)
    for k in range(K):
        dy[slot[:, k]] = store(topk_w[:, k].astype(np.float64)[:, None] * g, dtype)
        dw[:, k] = np.einsum("th,th->t", g, widen(y[slot[:, k]], dtype)).astype(np.float32)
    return dy, dw


def swiglu_bwd(DY, W2e, A, B, dtype):
    """dh = dy W2e^T; da = dh b sig(a) (1 + a (1 - sig(a))); db = dh silu(a).

    a and b are the saved (stored) forward values.  Returns stored (da, db).
    """
    dh = widen(DY, dtype) @ widen(W2e, dtype).T
    a, b = widen(A, dtype), widen(B, dtype)
    s = _sigmoid(a)
    da = dh * b * s * (1.0 + a * (1.0 - s))
    db = dh * a * s
    return store(da, dtype), store(db, dtype)


def input_grad(DA, DB, W1e, W3e, dtype):
    """dx = da W1e^T + db W3e^T: the two paths summed, then rounded once."""
    return store(widen(DA, dtype) @ widen(W1e, dtype).T + widen(DB, dtype) @ widen(W3e, dtype).T,
                 dtype)


def expert_ffn_bwd_data(dy, dout, offsets, w1, w3, w2, ab, dtype,
                        ws1=None, ws3=None, ws2=None, ab_sh=None):
    """Input-gradient part ("B") of the expert FFN backward.

    Returns dab [R, 2I] (da then db), dx_perm [R, H] and, for shared experts,
    dab_sh [Ns, T, 2I] and dx_sh [Ns, T, H] (a shared expert's output
    gradient is dout itself, its gate weight being 1).
    """
    E, H, I = w1.shape
    R = dy.shape[0]
    dab = storage_zeros((R, 2 * I), dtype)
    dxp = storage_zeros((R, H), dtype)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        da, db = swiglu_bwd(dy[lo:hi], w2[e], ab[lo:hi, :I], ab[lo:hi, I:], dtype)
        dab[lo:hi, :I], dab[lo:hi, I:] = da, db
        dxp[lo:hi] = input_grad(da, db, w1[e], w3[e], dtype)
    res = {"dab": dab, "dx_perm": dxp}
    if ws1 is not None and ws1.shape[0] > 0:
        Ns, T, Is = ws1.shape[0], dout.shape[0], ws1.shape[2]
        res["dab_sh"] = storage_zeros((Ns, T, 2 * Is), dtype)
        res["dx_sh"] = storage_zeros((Ns, T, H), dtype)
        for s in range(Ns):
            da, db = swiglu_bwd(dout, ws2[s], ab_sh[s, :, :Is], ab_sh[s, :, Is:], dtype)
            res["dab_sh"][s, :, :Is], res["dab_sh"][s, :, Is:] = da, db
            res["dx_sh"][s] = input_grad(da, db, ws1[s], ws3[s], dtype)
    return res


def expert_ffn_bwd_weight(x_perm, h, dy, dab, offsets, E, I, dtype,
                          x=None, h_sh=None, dout=None, dab_sh=None):
    """Weight-gradient part ("W"): a transposed grouped GEMM per expert.

    dW1[e] = X_e^T dA_e, dW3[e] = X_e^T dB_e, dW2[e] = H_e^T dY_e, summed in
    float64 over the expert's rows in slot order, written as float32.  An
    expert with no rows gets exact zeros.  Shared experts use all tokens:
    X = x, dY = dout.
    """
    H = x_perm.shape[1]
    dw1 = np.zeros((E, H, I), dtype=np.float32)
    dw3 = np.zeros((E, H, I), dtype=np.float32)
    dw2 = np.zeros((E, I, H), dtype=np.float32)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = widen(x_perm[lo:hi], dtype)
        D = widen(dab[lo:hi], dtype)
        dw1[e] = (X.T @ D[:, :I]).astype(np.float32)
        dw3[e] = (X.T @ D[:, I:]).astype(np.float32)
        dw2[e] = (widen(h[lo:hi], dtype).T @ widen(dy[lo:hi], dtype)).astype(np.float32)
    res = {"dw1": dw1, "dw3": dw3, "dw2": dw2}
    if h_sh is not None and h_sh.shape[0] > 0:
        Ns, Is = h_sh.shape[0], h_sh.shape[2]
        X = widen(x, dtype)
        G = widen(dout, dtype)
        res["dws1"] = np.stack([(X.T @ widen(dab_sh[s, :, :Is], dtype)).astype(np.float32) for s in range(Ns)])
        res["dws3"] = np.stack([(X.T @ widen(dab_sh[s, :, Is:], dtype)).astype(np.float32) for s in range(Ns)])
        res["dws2"] = np.stack([(widen(h_sh[s], dtype).T @ G).astype(np.float32) for s in range(Ns)])
    return res


def dispatch_bwd(dx_perm, slot, dtype, dx_sh=None):
    """dx[t] = sum_k dx_perm[slot[t,k]] (k ascending) + sum_s dx_sh[s,t]; one rounding."""
    T, K = slot.shape
    acc = np.zeros((T, dx_perm.shape[1]), dtype=np.float64)
    for k in range(K):
        acc += widen(dx_perm[slot[:, k]], dtype)
    if dx_sh is not None:
        for s in range(dx_sh.shape[0]):
            acc += widen(dx_sh[s], dtype)
    return store(acc, dtype)


def route_bwd(dtopk_w, topk_w, topk_idx, E):
    """Softmax-over-selected Jacobian: dl[t,e_k] = w_k (dw_k - sum_j w_j dw_j).

    Unselected experts get 0 (the selection is piecewise constant in the
    logits).  Float64, stored as float32.
    """
    w = topk_w.astype(np.float64)
    g = dtopk_w.astype(np.float64)
    inner = (w * g).sum(axis=1, keepdims=True)
    T, K = topk_idx.shape
    dl = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dl, topk_idx.astype(np.int64), w * (g - inner), axis=1)
    return dl.astype(np.float32)


def backward(inp: dict, fwd: dict, dtype: str) -> dict:
    E, H, I = inp["w1"].shape
    dy, dtw = combine_bwd(inp["dout"], fwd["y"], fwd["slot"], fwd["topk_w"], dtype)
    bd = expert_ffn_bwd_data(dy, inp["dout"], fwd["offsets"], inp["w1"], inp["w3"], inp["w2"],
                             fwd["ab"], dtype, inp.get("ws1"), inp.get("ws3"), inp.get("ws2"),
                             fwd.get("ab_sh"))
    bw = expert_ffn_bwd_weight(fwd["x_perm"], fwd["h"], dy, bd["dab"], fwd["offsets"], E, I, dtype,
                               inp["x"], fwd.get("h_sh"), inp["dout"], bd.get("dab_sh"))
    dx = dispatch_bwd(bd["dx_perm"], fwd["slot"], dtype, bd.get("dx_sh"))
    dl = route_bwd(dtw, fwd["topk_w"], fwd["topk_idx"], E)
    res = dict(dy=dy, dtopk_w=dtw, dx=dx, dlogits=dl)
    res.update(bd)
    res.update(bw)
    return res


# ---------------------------------------------------------------------------
# evaluation on a subset (for checks at full size, where the whole layer is
# too large for the CPU): the same definitions restricted to some tokens or
# some weight-gradient columns.
# ---------------------------------------------------------------------------


def _expert_weights(inp, e, dtype):
    """float64 copies of expert e's weights (e >= E: shared expert e - E)."""
    E = inp["w1"].shape[0]
    if e < E:
        return widen(inp["w1"][e], dtype), widen(inp["w3"][e], dtype), widen(inp["w2"][e], dtype)
    s = e - E
    return widen(inp["ws1"][s], dtype), widen(inp["ws3"][s], dtype), widen(inp["ws2"][s], dtype)


def tokens_forward(X, experts, weights, inp, dtype):
    """out for a few tokens straight from the definition, no permutation.

    X [n, H] storage rows, experts/weights [n, K] (the route of those tokens).
    Each (token, k) branch is h = silu(x W1_e) * (x W3_e), y = h W2_e with the
    layer's storage roundings; out = sum_k w_k y_k (k ascending) + shared
    experts, rounded once.  Returns (out [n, H] stored, y [n, K, H] stored).
    """
    n, K = experts.shape
    H = X.shape[1]
    E = inp["w1"].shape[0]
    Ns = inp["ws1"].shape[0] if "ws1" in inp else 0
    ys = storage_zeros((n, K, H), dtype)
    ysh = storage_zeros((Ns, n, H), dtype)
    for e in sorted(set(experts.ravel().tolist())) + [E + s for s in range(Ns)]:
        W1, W3, W2 = _expert_weights(inp, e, dtype)
        if e < E:
            rows, ks = np.nonzero(experts == e)
        else:
            rows = np.arange(n)
        Xf = widen(X[rows], dtype)
        a, b = Xf @ W1, Xf @ W3
        y = store(widen(store(_silu(a) * b, dtype), dtype) @ W2, dtype)
        if e < E:
            ys[rows, ks] = y
        else:
            ysh[e - E] = y
    acc = np.zeros((n, H), dtype=np.float64)
    for k in range(K):
        acc += weights[:, k].astype(np.float64)[:, None] * widen(ys[:, k], dtype)
    for s in range(Ns):
        acc += widen(ysh[s], dtype)
    return store(acc, dtype), ys


def tokens_backward(X, G, experts, weights, inp, dtype):
    """dx and dtopk_w for a few tokens straight from the definition.

    X, G [n, H] storage rows of x and dout.  Per branch: dy = w_k dout
    (stored), dh = dy W2_e^T, da/db from the branch's saved a, b, dx_k =
    da W1_e^T + db W3_e^T (stored); dx = sum_k dx_k (k ascending) + shared
    branches (dy = dout), rounded once; dw_k = <dout, y_k>.
    Returns (dx [n, H] stored, dw [n, K] float32).
    """
    n, K = experts.shape
    H = X.shape[1]
    E = inp["w1"].shape[0]
    Ns = inp["ws1"].shape[0] if "ws1" in inp else 0
    Gf = widen(G, dtype)
    dxk = np.zeros((n, K, H), dtype=np.float64)
    dxs = np.zeros((Ns, n, H), dtype=np.float64)
    dw = np.zeros((n, K), dtype=np.float32)
    for e in sorted(set(experts.ravel().tolist())) + [E + s for s in range(Ns)]:
        W1, W3, W2 = _expert_weights(inp, e, dtype)
        if e < E:
            rows, ks = np.nonzero(experts == e)
            dy = store(weights[rows, ks].astype(np.float64)[:, None] * Gf[rows], dtype)
        else:
            rows = np.arange(n)
            dy = G
        Xf = widen(X[rows], dtype)
        af, bf = Xf @ W1, Xf @ W3
        a, b = store(af, dtype), store(bf, dtype)
        y = store(widen(store(_silu(af) * bf, dtype), dtype) @ W2, dtype)
        dh = widen(dy, dtype) @ W2.T
        A, B = widen(a, dtype), widen(b, dtype)
        sg = _sigmoid(A)
        da = store(dh * B * sg * (1.0 + A * (1.0 - sg)), dtype)
        db = store(dh * A * sg, dtype)
        dx = widen(store(widen(da, dtype) @ W1.T + widen(db, dtype) @ W3.T, dtype), dtype)
        if e < E:
            dxk[rows, ks] = dx
            dw[rows, ks] = np.einsum("nh,nh->n", Gf[rows], widen(y, dtype)).astype(np.float32)
        else:
            dxs[e - E] = dx
    acc = np.zeros((n, H), dtype=np.float64)
    for k in range(K):
        acc += dxk[:, k]
    for s in range(Ns):
        acc += dxs[s]
    return store(acc, dtype), dw


def expert_wgrad_columns(X, DY, W1e, W3e, W2e, cols_I, dtype):
    """Columns cols_I of dW1/dW3 and rows cols_I of dW2 for one expert.

    X are the expert's input rows in slot order, DY its output-gradient rows
    (already gate-weighted and stored).  Only the intermediate units in cols_I
    are formed: a, b, h, da, db for those units, then
    dW1[:, j] = X^T da[:, j], dW3[:, j] = X^T db[:, j], dW2[j, :] = h[:, j]^T DY.
    Returns (dw1_cols [H, J], dw3_cols [H, J], dw2_rows [J, H]) float32.
    """
    cols_I = np.asarray(cols_I)
    Xf = widen(X, dtype)
    af64 = Xf @ widen(W1e[:, cols_I], dtype)
    bf64 = Xf @ widen(W3e[:, cols_I], dtype)
    a, b = store(af64, dtype), store(bf64, dtype)
    h = store(_silu(af64) * bf64, dtype)
    da, db = swiglu_bwd(DY, W2e[cols_I, :], a, b, dtype)
    DA, DB = widen(da, dtype), widen(db, dtype)
    dw1 = (Xf.T @ DA).astype(np.float32)
    dw3 = (Xf.T @ DB).astype(np.float32)
    dw2 = (widen(h, dtype).T @ widen(DY, dtype)).astype(np.float32)
    return dw1, dw3, dw2
