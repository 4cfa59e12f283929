"""Helpers of the GPU parity tests: device upload/download and the error
measures of the parity bar (normwise relative error for bf16, max absolute
error for f32)."""
import contextlib
import dataclasses
import os

import numpy as np
import torch

import combine_moe_route_histogram_amd as M

import oracle as O
import synth
from combine_moe_route_histogram_amd import layer as L


def dev(a):
    return None if a is None else synth.to_torch(a, "cuda")


def host(t):
    """Device tensor -> numpy storage array (bf16 -> uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def max_rel(got, ref, dtype):
    """max |got - ref| / max |ref| over a tensor (both storage arrays)."""
    g, r = O.widen(got, dtype), O.widen(ref, dtype)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / den) if den > 0 else float(np.max(np.abs(g)))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def f32_rel(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got.astype(np.float64) - ref.astype(np.float64))) / max(den, 1e-30))


def custom_config(T, H, E, K, I, Ns=0, dtype="bf16", logits="gauss", number=90):
    return synth.Config("custom", number, T, H, E, K, I, Ns, I if Ns else 0, dtype, "fwd+bwd", logits)


def device_inputs(inp):
    return {k: dev(v) for k, v in inp.items()}


def run_layer(cfg, inp, fused=False, backward=True):
    d = L.make_dims(cfg.T if "x" not in inp else inp["x"].shape[0], cfg.H, cfg.E, cfg.K, cfg.I,
                    cfg.n_shared, cfg.dtype)
    p = device_inputs(inp)
    b = L.Buffers(d, backward=backward)
    L.forward(b, p, fused=fused)
    if backward:
        L.backward(b, p)
    torch.cuda.synchronize()
    return d, b


@contextlib.contextmanager
def debug_settings(**env):
    """Run a block with the library's debug settings (environment variables
    that moe_init reads; no other call reads the environment) set to `env`
    (None: unset); they are unset and re-read afterwards."""
    try:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = str(v)
        M.moe_init(0)
        yield
    finally:
        for k in env:
            os.environ.pop(k, None)
        M.moe_init(0)
