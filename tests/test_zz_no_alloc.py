"""moe_layer_forward_noalloc (the layer forward on the library's fixed
per-GPU scratch, for callers that cannot allocate) against moe_layer_forward
with a caller workspace, through the C ABI: two calls in a row, the second
with fewer tokens, each bit-identical to the workspace call on the same
inputs (same kernels; the scratch keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import synth, workloads

from gpu_common import gpu, require_gpu, say

pytestmark = gpu

AUX_CHECK = ("logits", "topk_idx", "topk_gate", "topk_score", "counts", "offsets", "inv_row",
             "n_dropped", "f", "P", "scalars")


def _pair(wl, inp, weights):
    cfg = moe.make_cfg(wl)
    dt = torch.bfloat16 if wl.act_dtype == workloads.BF16 else torch.float32
    out_ref = torch.empty((wl.T, wl.H), dtype=dt, device="cuda")
    out_na = torch.full((wl.T, wl.H), float("nan"), dtype=dt, device="cuda")
    aux_ref = moe.alloc_aux(cfg)
    aux_na = moe.alloc_aux(cfg)
    ws = moe.alloc_workspace(cfg)
    ws.fill_(0x5A)
    moe.moe_layer_forward(cfg, weights, inp["x"], inp["bias"], out_ref, aux_ref, ws)
    moe.moe_layer_forward_noalloc(cfg, weights, inp["x"], inp["bias"], out_na, aux_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na.view(torch.int16) if dt == torch.bfloat16 else out_na,
                       out_ref.view(torch.int16) if dt == torch.bfloat16 else out_ref)
    M = int(aux_ref["offsets"][-1].item())
    for name in AUX_CHECK:
        assert torch.equal(aux_na[name], aux_ref[name]), name
    assert torch.equal(aux_na["row_token"][:M], aux_ref["row_token"][:M])
    return out_na


@pytest.mark.parametrize("base,T0,T1", [
    (workloads.V1.with_(name="v1_shape_small"), 512, 200),
    (workloads.V3_DECODE.with_(name="v3_routing_narrow", H=1024, I=256, I_shared=256), 128, 40),
    (workloads.V3_SKEW.with_(name="v3_routing_capacity_narrow", H=512, I=128, I_shared=128,
                             capacity=20), 300, 77),
    (workloads.TINY, 64, 13),
])
def test_noalloc_forward_matches_workspace_forward_twice(base, T0, T1):
    require_gpu()
    big = base.with_(T=T0)
    small = base.with_(T=T1)
    inp = synth.make_inputs(big, device="cuda")
    weights = moe.prepare_weights(moe.make_cfg(big),
                                  {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2")})
    say(f"no-alloc forward {base.name}: T={T0} then T={T1}")
    _pair(big, inp, weights)
    inp_small = dict(inp)
    inp_small["x"] = inp["x"][:T1].contiguous()
    out = _pair(small, inp_small, weights)
    assert torch.isfinite(out.float()).all()


def test_noalloc_forward_rejects_a_layer_beyond_the_scratch():
    require_gpu()
    wl = workloads.V1  # T = 4096: about 200 MiB of workspace
    cfg = moe.make_cfg(wl)
    assert moe.moe_workspace_size(cfg) > moe.NOALLOC_SCRATCH_BYTES
    inp = synth.make_inputs(wl.with_(T=1), device="cuda")
    x = torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    weights = moe.prepare_weights(cfg, {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2")})
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(cfg, weights, x, None, out, None)
    assert e.value.code == moe.MOE_ERR_TOO_LARGE
