"""moe_route_noalloc: the routing call for callers that cannot allocate,
whose scratch is a fixed device array of the library.  Checked through the C
ABI against moe_route (caller workspace) on the same logits, bit for bit, on
two calls in a row, the second with fewer tokens (the array keeps the first
call's contents); and the size limit is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import combine_moe_route_histogram_amd as M
from combine_moe_route_histogram_amd import layer as L
from gpu_util import host

pytestmark = pytest.mark.gpu


def _route_both(T, E, K, seed):
    g = np.random.default_rng(seed)
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits[g.random((T, E)) < 0.1] = 0.0                   # some ties
    lg = torch.from_numpy(logits).cuda()
    d = L.make_dims(T, 64, E, K, 64, 0, "bf16")
    ref = L.Buffers(d, backward=False)
    L.route(ref, {"logits": lg})                             # moe_route with a workspace
    i32 = lambda n: torch.full((n,), -7, dtype=torch.int32, device="cuda")
    got = {"topk_idx": i32(T * K), "topk_w": torch.full((T * K,), -7.0, device="cuda"),
           "counts": i32(E), "offsets": i32(E + 1), "slot": i32(T * K), "slot_src": i32(T * K)}
    M.moe_route_noalloc(d, lg, got["topk_idx"], got["topk_w"], got["counts"], got["offsets"],
                        got["slot"], got["slot_src"])
    M.moe_sync_status()
    for n, t in got.items():
        assert np.array_equal(host(t).ravel(), host(getattr(ref, n)).ravel()), (T, E, K, n)


def test_noalloc_route_equals_workspace_route_twice():
    print("case moe_route_noalloc T=131072 E=32 K=4 then T=1000 E=64 K=6", flush=True)
    _route_both(131072, 32, 4, seed=1)     # ceil(T/64) * E = 65536 of the 131072 limit
    _route_both(1000, 64, 6, seed=2)       # a second, smaller call on the same array


def test_noalloc_route_at_the_limit_and_refused_beyond():
    print("case moe_route_noalloc at the limit (T=8192, E=256, K=8)", flush=True)
    _route_both(8192, 256, 8, seed=3)      # ceil(T/64) * E = 128 * 256 = 32768
    _route_both(32768, 256, 2, seed=4)     # exactly the limit: 512 chunks * 256 = 131072
    d = L.make_dims(32769, 64, 256, 2, 64, 0, "bf16")
    p = torch.empty(16, dtype=torch.int32, device="cuda")
    lib = M.load()
    st = lib.moe_route_noalloc(ctypes.byref(d), *([ctypes.c_void_p(p.data_ptr())] * 7), None)
    assert st == 2                                           # MOE_EUNSUPPORTED
    assert "fixed scratch" in M.moe_last_error()
