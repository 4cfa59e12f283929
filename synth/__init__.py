"""Seeded synthetic inputs for the MoE expert-layer workloads.

This module only *draws* the tensors the layer consumes -- activations,
router logits, expert weights, output gradients.  It holds none of the
layer's own arithmetic (no routing, no permutation, no FFN, no rounding
rule of the layer), so both the CPU oracle and the GPU path can take their
inputs from here without sharing any code of the method.

Workload shapes follow the UniEP article ("UniEP: Unified Expert-Parallel
MoE MegaKernel for LLM Training", section 1.1: a gate picks top-k experts per
token, tokens are dispatched to a SwiGLU expert FFN and combined with the gate
scores); the five shapes are the layer sizes this library is measured on:
tiny fp32, Mixtral-like, DeepSeek-V3-16B-like with two shared experts, a
Zipf-skewed load, and a 128k-token long-sequence share.

Storage convention (numpy side): float32 tensors are ``np.float32`` arrays;
bfloat16 tensors are ``np.uint16`` arrays holding the bf16 bit patterns.
The float32 -> bfloat16 cast of the draws is done by torch's CPU cast
(round to nearest even), a library routine, not by code of the layer.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

__all__ = ["Config", "CONFIGS", "config", "make_inputs", "to_torch"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    number: int          # 1-based position in the workload list; seed = 1000 + number
    T: int               # tokens
    H: int               # hidden (model) dim
    E: int               # routed experts
    K: int               # experts per token (top-k)
    I: int               # SwiGLU intermediate dim of a routed expert
    n_shared: int        # shared experts applied to every token (weight 1)
    I_shared: int        # intermediate dim of a shared expert
    dtype: str           # storage dtype of activations/weights: "f32" or "bf16"
    passes: str          # "fwd" or "fwd+bwd"
    logits: str          # recipe: "router" | "gauss" | "zipf"

    @property
    def R(self) -> int:
        return self.T * self.K

    @property
    def seed(self) -> int:
        return 1000 + self.number

    def scaled(self, T: int) -> "Config":
        """Same layer, fewer tokens (used for bounded CPU samples)."""
        return dataclasses.replace(self, T=T)


CONFIGS = {
    "tiny": Config("tiny", 1, 256, 128, 8, 2, 256, 0, 0, "f32", "fwd", "router"),
    "mixtral": Config("mixtral", 2, 4096, 4096, 8, 2, 14336, 0, 0, "bf16", "fwd+bwd", "gauss"),
    "dsv3": Config("dsv3", 3, 8192, 2048, 64, 6, 1408, 2, 1408, "bf16", "fwd+bwd", "gauss"),
    "skewed": Config("skewed", 4, 16384, 2048, 64, 6, 1408, 0, 0, "bf16", "fwd", "zipf"),
    "longseq": Config("longseq", 5, 131072, 2048, 32, 4, 1408, 0, 0, "bf16", "fwd+bwd", "gauss"),
}


def config(name: str) -> Config:
    return CONFIGS[name]


# ---------------------------------------------------------------------------
# drawing
# ---------------------------------------------------------------------------
_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _normal_f32(seq: np.random.SeedSequence, shape, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) float32 draw, filled chunk by chunk from child seeds.

    The chunking (fixed chunk size, one child SeedSequence per chunk) makes the
    result independent of the number of threads used to fill it.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nchunk = max(1, (n + _CHUNK - 1) // _CHUNK)
    children = seq.spawn(nchunk)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunk == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunk)))
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


def _cast(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def _zipf_logits(seq: np.random.SeedSequence, T: int, E: int, s: float = 1.2,
                 n_empty: int = 8) -> np.ndarray:
    """Gumbel-perturbed log-probabilities of a Zipf(s) expert popularity.

    A seeded permutation assigns popularity ranks 1..E-n_empty to experts with
    p proportional to rank^-s; the last n_empty experts get p = 0 (log p taken
    as -1e4, finite).  Top-k of log p + Gumbel(0,1) samples k distinct experts
    without replacement in proportion to p, so the load is Zipf-skewed with a
    large head and n_empty experts that receive no token.
    """
    g = np.random.Generator(np.random.PCG64(seq))
    perm = g.permutation(E)
    logp = np.full(E, -1.0e4, dtype=np.float64)
    ranks = np.arange(1, E - n_empty + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    logp[perm[: E - n_empty]] = np.log(p)
    gumbel = g.gumbel(size=(T, E))
    return (logp[None, :] + gumbel).astype(np.float32)


def make_inputs(cfg: Config, T: int | None = None, seed: int | None = None,
                with_grad: bool | None = None) -> dict:
    """All inputs of one workload as numpy storage arrays.

    Keys: logits [T,E] f32; x [T,H]; w1, w3 [E,H,I]; w2 [E,I,H];
    ws1, ws3 [Ns,H,Is]; ws2 [Ns,Is,H] (absent when Ns == 0);
    dout [T,H] (when the workload has a backward pass or with_grad=True).

    Recipe: x ~ N(0,1); every weight ~ N(0, 0.02^2); dout ~ N(0,1);
    logits: "router" = x . Wg with Wg ~ N(0, 0.02^2) (float64 product of the
    float32 draws, rounded once to float32 -- the router GEMM sits upstream of
    the layer), "gauss" = iid N(0,1), "zipf" = see _zipf_logits.
    Each tensor has its own child seed of SeedSequence(seed) in a fixed order,
    so a smaller T gives a different (but equally seeded) draw of x.
    """
    T = cfg.T if T is None else T
    seed = cfg.seed if seed is None else seed
    if with_grad is None:
        with_grad = "bwd" in cfg.passes
    root = np.random.SeedSequence([seed, T])
    s_x, s_logit, s_w1, s_w3, s_w2, s_ws1, s_ws3, s_ws2, s_dout = root.spawn(9)
    H, E, I = cfg.H, cfg.E, cfg.I
    out = {}
    x32 = _normal_f32(s_x, (T, H))
    if cfg.logits == "router":
        wg = _normal_f32(s_logit, (H, E), 0.02)
        out["logits"] = (x32.astype(np.float64) @ wg.astype(np.float64)).astype(np.float32)
    elif cfg.logits == "gauss":
        out["logits"] = _normal_f32(s_logit, (T, E))
    elif cfg.logits == "zipf":
        out["logits"] = _zipf_logits(s_logit, T, E)
    else:
        raise ValueError(cfg.logits)
    out["x"] = _cast(x32, cfg.dtype)
    del x32
    out["w1"] = _cast(_normal_f32(s_w1, (E, H, I), 0.02), cfg.dtype)
    out["w3"] = _cast(_normal_f32(s_w3, (E, H, I), 0.02), cfg.dtype)
    out["w2"] = _cast(_normal_f32(s_w2, (E, I, H), 0.02), cfg.dtype)
    if cfg.n_shared:
        Ns, Is = cfg.n_shared, cfg.I_shared
        out["ws1"] = _cast(_normal_f32(s_ws1, (Ns, H, Is), 0.02), cfg.dtype)
        out["ws3"] = _cast(_normal_f32(s_ws3, (Ns, H, Is), 0.02), cfg.dtype)
        out["ws2"] = _cast(_normal_f32(s_ws2, (Ns, Is, H), 0.02), cfg.dtype)
    if with_grad:
        out["dout"] = _cast(_normal_f32(s_dout, (T, H)), cfg.dtype)
    return out


def to_torch(a: np.ndarray, device="cpu"):
    """numpy storage array -> torch tensor (uint16 bit patterns become bfloat16)."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device) if device != "cpu" else t
