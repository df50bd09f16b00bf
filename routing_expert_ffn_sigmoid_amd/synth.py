"""Seeded synthetic inputs for the DeepSeekMoE layer workloads.

Inputs only: nothing here routes, scores, multiplies experts or reduces
statistics.  Every tensor is drawn from its own torch Philox stream, seeded
by a hash of (workload seed, tensor name), on the device it is created on,
so the same call on the same kind of device gives the same bytes.  Gaussians
are drawn in fp32, scaled by the tensor's standard deviation and rounded
once (round-to-nearest-even) to the tensor's dtype.

Recipe per tensor (shapes [rows, cols], weights stored out x in):
  x      [T, H]             N(0, x_std^2)                 act dtype
  w_router [N, H]           N(0, wg_std^2)                router dtype
  bias   [N] fp32           U(-p, p) ("uniform"), zeros ("none"), or Zipf
                            rank bias ("zipf", below)
  w13    [N, 2I, H]         N(0, w_std^2); rows [0,I) gate, [I,2I) up
  w2     [N, H, I]          N(0, w_std^2)
  ws13   [2 n_sh I_sh, H]   packed shared experts (gate rows of every shared
                            expert, then their up rows)
  ws2    [H, n_sh I_sh]

Zipf bias: a seeded permutation pi of the experts ranks them; expert pi[r-1]
gets bias -beta * s * ln(r) for rank r = 1..N (s = exponent, beta = 0.05),
so the selection odds fall off with rank like a power law.
"""
from __future__ import annotations

import hashlib
import math

import torch

from .workloads import BF16, Workload

ZIPF_BETA = 0.05


def _dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def _gen(seed: int, name: str, device) -> torch.Generator:
    h = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def normal(shape, std: float, dtype: torch.dtype, device, seed: int, name: str,
           chunk_dim0: bool = False) -> torch.Tensor:
    """N(0, std^2) in fp32, rounded once to dtype.  chunk_dim0 draws one
    slice of dim 0 at a time (bounded fp32 temporaries for big tensors)."""
    g = _gen(seed, name, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    if chunk_dim0 and len(shape) > 1:
        for i in range(shape[0]):
            tmp = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            out[i].copy_(tmp.mul_(std))
    else:
        tmp = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.copy_(tmp.mul_(std))
    return out


def uniform(shape, lo: float, hi: float, device, seed: int, name: str) -> torch.Tensor:
    g = _gen(seed, name, device)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return u.mul_(hi - lo).add_(lo)


def zipf_bias(N: int, s: float, device, seed: int, beta: float = ZIPF_BETA) -> torch.Tensor:
    g = _gen(seed, "zipf_perm", "cpu")
    perm = torch.randperm(N, generator=g)
    b = torch.empty(N, dtype=torch.float32)
    for r in range(1, N + 1):
        b[perm[r - 1]] = -beta * s * math.log(r)
    return b.to(device)


def make_inputs(wl: Workload, device="cpu", with_experts: bool = True) -> dict:
    """All inputs of one layer call for workload wl, on device."""
    seed = wl.seed
    act = _dtype(wl.act_dtype)
    wdt = _dtype(wl.w_dtype)
    rdt = _dtype(wl.router_dtype)
    big = wl.N * 2 * wl.I * wl.H > (1 << 26)
    inp = {
        "x": normal((wl.T, wl.H), wl.x_std, act, device, seed, f"x_T{wl.T}"),
        "w_router": normal((wl.N, wl.H), wl.wg_std, rdt, device, seed, "w_router"),
    }
    if wl.bias_kind == "uniform":
        inp["bias"] = uniform((wl.N,), -wl.bias_param, wl.bias_param, device, seed, "bias")
    elif wl.bias_kind == "zipf":
        inp["bias"] = zipf_bias(wl.N, wl.bias_param, device, seed)
    else:
        inp["bias"] = None
    if with_experts:
        inp["w13"] = normal((wl.N, 2 * wl.I, wl.H), wl.w_std, wdt, device, seed, "w13",
                            chunk_dim0=big)
        inp["w2"] = normal((wl.N, wl.H, wl.I), wl.w_std, wdt, device, seed, "w2",
                           chunk_dim0=big)
        ish = wl.n_shared * wl.I_shared
        if ish > 0:
            inp["ws13"] = normal((2 * ish, wl.H), wl.w_std, wdt, device, seed, "ws13")
            inp["ws2"] = normal((wl.H, ish), wl.w_std, wdt, device, seed, "ws2")
        else:
            inp["ws13"] = None
            inp["ws2"] = None
    return inp
