"""Router GEMM through moe_route, against the fp64 oracle.

Sizes span several 256-token tiles, K splits, ragged token tails and expert
counts that are not a multiple of the 256-expert tile, for both kernels:
bf16 MFMA over the exact bf16 pieces of the router weight (bf16 x with an
fp32 or bf16 weight), and fp32 MFMA (fp32 x).
A one-hot case pins the piece split and its tiled layout: with x[t] = a
power of two at one column h, logit (t, e) is that power times w[e, h]
exactly, so it must equal the product computed on the host bit for bit,
for weights of every magnitude the split covers."""
import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import workloads
from routing_expert_ffn_sigmoid_amd.workloads import BF16, F32

from gpu_common import F32_MAXREL, gpu, normwise, require_gpu, say, typed

pytestmark = gpu


def _wl(T, H, N, act, rdt):
    return workloads.TINY.with_(T=T, H=H, N=N, k=4, n_groups=1, topk_groups=1,
                                act_dtype=act, w_dtype=act, router_dtype=rdt,
                                bias_kind="none")


def _logits(wl, x, wr):
    cfg = moe.make_cfg(wl)
    ws = moe.alloc_workspace(cfg)
    T, N, k = wl.T, wl.N, wl.k
    dev = "cuda"
    lg = torch.full((T, N), float("nan"), device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), device=dev)
    score = torch.empty((T, k), device=dev)
    moe.moe_route(cfg, x, wr, lg, None, idx, gate, score, None, ws)
    torch.cuda.synchronize()
    return lg


CASES = [
    # T, H, N, x dtype, router dtype
    (300, 2048, 256, BF16, F32),    # 2 token tiles (ragged), 16 K splits
    (1037, 7168, 160, BF16, F32),   # 5 token tiles, partial expert tile, V3 width
    (600, 1024, 64, BF16, BF16),    # one bf16 piece
    (300, 256, 20, BF16, F32),      # N % 16 != 0: a part-padded 16-expert block
    (300, 192, 64, BF16, F32),      # 6 k-steps: one split, logits written directly
    (1, 256, 16, BF16, F32),        # a single token
    (300, 256, 64, F32, F32),       # fp32 activations: fp32 MFMA kernel
]


@pytest.mark.parametrize("T,H,N,act,rdt", CASES)
def test_router_logits_match_oracle(T, H, N, act, rdt):
    require_gpu()
    say(f"router T={T} H={H} N={N} act={act} router={rdt}")
    g = torch.Generator(device="cpu").manual_seed(T * 131 + H * 7 + N)
    xdt = torch.bfloat16 if act == BF16 else torch.float32
    wdt = torch.bfloat16 if rdt == BF16 else torch.float32
    x = torch.randn((T, H), generator=g).to(xdt).cuda()
    wr = (torch.randn((N, H), generator=g) * 0.02).to(wdt).cuda()
    lg = _logits(_wl(T, H, N, act, rdt), x, wr)
    ref = oracle.router_logits(typed(x), typed(wr))
    got = lg.cpu().numpy()
    assert np.isfinite(got).all()
    mr, l2 = normwise(got, ref)
    say(f"  max-rel {mr:.2e} rel-L2 {l2:.2e}")
    assert mr <= F32_MAXREL


@pytest.mark.parametrize("rdt", [F32, BF16])
def test_router_one_hot_logits_are_exact_weights(rdt):
    require_gpu()
    T, H, N = 356, 2048, 256
    say(f"router one-hot T={T} H={H} N={N} router={rdt}")
    rng = np.random.default_rng(7)
    # weights over many binades (2^-80 <= |w| < 2^81), both signs, full
    # 24-bit significands, and exact zeros
    mant = rng.integers(1 << 23, 1 << 24, (N, H)).astype(np.float64) / (1 << 23)
    w = np.where(rng.random((N, H)) < 0.5, -1.0, 1.0) * np.ldexp(mant, rng.integers(-80, 81, (N, H)))
    w[rng.random((N, H)) < 0.05] = 0.0
    w32 = w.astype(np.float32)
    if rdt == BF16:
        wt = torch.from_numpy(w32).to(torch.bfloat16)
        w32 = wt.float().numpy()
    else:
        wt = torch.from_numpy(w32)
    cols = (np.arange(T) * 37) % H
    scale = np.where(np.arange(T) % 3 == 0, -2.0, 0.5).astype(np.float32)
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), cols] = scale
    lg = _logits(_wl(T, H, N, BF16, rdt), torch.from_numpy(x).to(torch.bfloat16).cuda(),
                 wt.cuda())
    # the fp32 sum starts from +0, so a zero product gives +0 (not -0)
    want = (np.float32(0.0) + w32[:, cols].T * scale[:, None]).astype(np.float32)
    np.testing.assert_array_equal(lg.cpu().numpy().view(np.uint32), want.view(np.uint32))
