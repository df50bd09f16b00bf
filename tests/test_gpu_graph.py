"""moe_layer_forward captured in a HIP graph (torch.cuda.CUDAGraph on ROCm)
and replayed.  The library only launches kernels on the caller's stream:
buffers are cleared by fill kernels (no memset nodes) and nothing waits on
the host, so a serving loop can capture a layer once and replay it.  Every
replay, with eager work and synchronizations between replays, must
reproduce the eager call bit for bit: the output and every auxiliary result
(logits, routing, dispatch, statistics)."""
import torch

import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import workloads

from gpu_common import gpu, make_inputs, require_gpu, say

pytestmark = gpu


def _poison(out, aux):
    out.fill_(float("nan"))
    for t in aux.values():
        if t.dtype == torch.int32:
            t.fill_(-7)
        else:
            t.fill_(float("nan"))


def test_layer_forward_replays_from_a_hip_graph():
    require_gpu()
    # >= 128 rows per expert and K = 1024 / 2048: both FFN phases run on the
    # ping-pong kernel (down with its staged epilogue)
    wl = workloads.V3_PREFILL.with_(T=2048, H=1024, N=64, k=8, n_groups=8, topk_groups=4,
                                    I=2048, I_shared=2048)
    say(f"graph replay: {wl.name} T={wl.T} H={wl.H} N={wl.N} I={wl.I}")
    inp = make_inputs(wl)
    cfg = moe.make_cfg(wl)
    w = moe.prepare_weights(cfg, {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2")})
    ws = moe.alloc_workspace(cfg)
    aux = moe.alloc_aux(cfg)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    def call():
        moe.moe_layer_forward(cfg, w, inp["x"], inp["bias"], out, aux, ws)

    _poison(out, aux)
    call()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_aux = {n: t.clone() for n, t in aux.items()}
    assert not torch.isnan(ref_out.float()).any()

    side = torch.cuda.Stream()  # warm-up on a side stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    a = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        _poison(out, aux)
        a = torch.tanh(a @ a.t())  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: out"
        for n, t in ref_aux.items():
            assert torch.equal(aux[n].view(torch.int32), t.view(torch.int32)), f"replay {rep}: {n}"
    say("  4 replays bit-identical to the eager call")
