"""Algorithm 1 with G explicit ranks on the GPU (moe_route_ranks) against the
oracle: the [G, E] count table, the rank base offsets and the slot map, all
bit-exact, for rank counts from 1 to one rank per token, uniform and skewed
routings, and the full-size token counts of the workloads.  The slots must
also equal the one-rank map (moe_route's), which is the point of the
algorithm."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import combine_moe_route_histogram_amd as M
from gpu_util import host

pytestmark = pytest.mark.gpu


def _gpu_ranks(idx, E, G):
    T, K = idx.shape
    d = M.Dims(T=T, H=64, E=E, K=K, I=64, n_shared=0, dtype=M.BF16)
    i32 = lambda *s: torch.empty(*s, dtype=torch.int32, device="cuda")
    out = dict(rank_counts=i32(G * E), rank_base=i32(G * E), counts=i32(E), offsets=i32(E + 1),
               slot=i32(T * K), slot_src=i32(T * K))
    ws = torch.empty(M.moe_route_ranks_workspace_bytes(d, G), dtype=torch.uint8, device="cuda")
    M.moe_route_ranks(d, torch.as_tensor(idx, device="cuda"), G, out["rank_counts"], out["rank_base"],
                      out["counts"], out["offsets"], out["slot"], out["slot_src"], ws)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _check(idx, E, G):
    T, K = idx.shape
    print(f"case T={T} E={E} K={K} G={G}", flush=True)
    counts_rank, slot_g = O.slot_map_ranks(idx, E, G)
    counts, offsets, slot, slot_src = O.slot_map(idx, E)
    assert np.array_equal(slot_g, slot)   # the oracle's own multi-rank map equals one rank
    got = _gpu_ranks(idx, E, G)
    assert np.array_equal(got["rank_counts"].reshape(G, E), counts_rank)
    assert np.array_equal(got["rank_base"].reshape(G, E), O.rank_base_offsets(counts_rank))
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["slot"].reshape(T, K), slot)
    assert np.array_equal(got["slot_src"], slot_src)


def _uniform_idx(T, E, K, seed):
    g = np.random.default_rng(seed)
    return O.route_select(g.standard_normal((T, E)).astype(np.float32), K)


@pytest.mark.parametrize("T,E,K", [(1000, 8, 2), (777, 64, 6), (300, 256, 8), (1, 4, 2)])
@pytest.mark.parametrize("G", [1, 2, 3, 7, 64, "T"])
def test_ranks_small(T, E, K, G):
    G = T if G == "T" else min(G, T)
    _check(_uniform_idx(T, E, K, seed=T + E + G), E, G)


def test_ranks_skewed_with_empty_experts():
    T, E, K = 3000, 64, 6
    logits = synth._zipf_logits(np.random.SeedSequence(7), T, E)
    idx = O.route_select(logits, K)
    assert (np.bincount(idx.ravel(), minlength=E) == 0).sum() == 8
    for G in (5, 17, 300):
        _check(idx, E, G)


@pytest.mark.parametrize("name,G", [("mixtral", 8), ("dsv3", 16), ("longseq", 8), ("longseq", 4096)])
def test_ranks_full_size_token_counts(name, G):
    cfg = synth.config(name)
    g = np.random.default_rng(cfg.seed)
    idx = O.route_select(g.standard_normal((cfg.T, cfg.E)).astype(np.float32), cfg.K)
    _check(idx, cfg.E, G)


def test_ranks_equal_route_slot_map():
    """moe_route's one-rank map and moe_route_ranks agree for any G on the GPU."""
    T, E, K = 2048, 32, 4
    g = np.random.default_rng(3)
    logits = torch.as_tensor(g.standard_normal((T, E)).astype(np.float32), device="cuda")
    d = M.Dims(T=T, H=64, E=E, K=K, I=64, n_shared=0, dtype=M.BF16)
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")
    idx, w = i32(T * K), torch.empty(T * K, dtype=torch.float32, device="cuda")
    counts, offsets, slot, slot_src = i32(E), i32(E + 1), i32(T * K), i32(T * K)
    ws = torch.empty(M.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    M.moe_route(d, logits, idx, w, counts, offsets, slot, slot_src, ws)
    torch.cuda.synchronize()
    for G in (1, 6, 100, T):
        got = _gpu_ranks(host(idx).reshape(T, K), E, G)
        assert np.array_equal(got["slot"], host(slot))
        assert np.array_equal(got["slot_src"], host(slot_src))
