"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (moe_layer_forward with the default tiles): routing,
dispatch and statistics over every token; layer outputs on every token of
the v1, v2, V3 prefill and V3 decode layers and, at skew (16384 tokens), on a
stratified sample of at least 2048 (the first and last row of every row tile
of every expert segment, every shared-expert tile, tokens with dropped
slots, random tokens), which the oracle computes one token at a time, the
calls spread over the host cores."""
import time

import numpy as np
import pytest
import torch

import oracle
from routing_expert_ffn_sigmoid_amd import workloads

from gpu_common import (F32_MAXREL, check_dispatch, check_outputs, check_routing, check_seq_stats,
                        check_stats, f64, gpu, layer_forward, make_inputs, normwise, oracle_rows,
                        oracle_workers, require_gpu, row_rel_l2, say, stratified_tokens, typed)

pytestmark = gpu


@pytest.fixture(scope="module")
def v3_weights():
    require_gpu()
    say("generating V3-shaped weights (256 experts, H=7168, I=2048) on the GPU")
    inp = make_inputs(workloads.V3_PREFILL)
    w = {n: inp[n] for n in ("w_router", "w13", "w2", "ws13", "ws2", "bias")}
    yield w
    del w
    torch.cuda.empty_cache()


def _logit_sample_check(inp, aux, tokens):
    ref = oracle.router_logits(typed(inp["x"][tokens]), typed(inp["w_router"]))
    mr, _ = normwise(aux["logits"][tokens].cpu().numpy(), ref)
    assert mr <= F32_MAXREL, f"router logits max-rel {mr}"


def _run(wl, inp, min_tokens, all_tokens=False):
    """The layer at full size: routing, dispatch and statistics over every
    token; outputs on every token (all_tokens) or on a stratified sample
    that reaches the first and last row of every row tile of every expert
    segment, every shared-expert tile and tokens with dropped slots."""
    say(f"layer {wl.name}")
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    st = check_stats(wl, aux)
    toks = list(range(wl.T)) if all_tokens else stratified_tokens(wl, d, min_count=min_tokens)
    _logit_sample_check(inp, aux, toks[:: max(1, len(toks) // 64)])
    t0 = time.perf_counter()
    ref = oracle_rows(wl, inp, r, d, toks)
    dt = time.perf_counter() - t0
    mr, l2 = check_outputs(wl, out, ref, toks)
    worst_row = float(row_rel_l2(f64(out[toks]), ref).max())
    n_drop_tok = int(((d["inv_row"][toks] < 0).any(axis=1)).sum())
    say(f"  {len(toks)} tokens ({n_drop_tok} with a dropped slot) against the oracle in "
        f"{dt:.1f} s on {oracle_workers()} host threads: max-rel {mr:.2e} rel-L2 {l2:.2e} "
        f"(worst row {worst_row:.2e}); "
        f"L_B {st['L_B']:.4f} dropped {d['n_dropped']}")
    return out, aux, d, toks


def test_v1_shaped_layer():
    require_gpu()
    wl = workloads.V1
    inp = make_inputs(wl)
    _run(wl, inp, 0, all_tokens=True)


def test_v2_shaped_layer_device_limited_with_device_drop():
    """160 experts on 8 devices (3 kept, top-1 group score), softmax gate,
    dropping at the average device load; sampled rows include dropped ones."""
    require_gpu()
    wl = workloads.V2
    inp = make_inputs(wl)
    _, _, d, toks = _run(wl, inp, 0, all_tokens=True)
    assert d["n_dropped"] > 0
    assert (d["inv_row"][toks] < 0).any()


def test_v3_prefill_layer(v3_weights):
    wl = workloads.V3_PREFILL
    from routing_expert_ffn_sigmoid_amd import synth
    inp = dict(v3_weights)
    inp["x"] = synth.normal((wl.T, wl.H), wl.x_std, torch.bfloat16, "cuda", wl.seed, f"x_T{wl.T}")
    _, aux, _, toks = _run(wl, inp, 0, all_tokens=True)
    assert len(toks) == wl.T
    # the batch as four sequences of 2048 tokens (sequence-wise statistics)
    ref = check_seq_stats(wl, [0, 2048, 4096, 6144, 8192], aux["topk_idx"], aux["token_lse"],
                          aux["logits"])
    say(f"  sequence-wise L_B {np.round(ref['L'], 4).tolist()} mean {ref['L_mean']:.4f}")


def test_v3_decode_layer(v3_weights):
    wl = workloads.V3_DECODE
    from routing_expert_ffn_sigmoid_amd import synth
    inp = dict(v3_weights)
    inp["x"] = synth.normal((wl.T, wl.H), wl.x_std, torch.bfloat16, "cuda", wl.seed, f"x_T{wl.T}")
    _run(wl, inp, 0, all_tokens=True)


def test_v3_skew_layer_with_capacity(v3_weights):
    wl = workloads.V3_SKEW
    from routing_expert_ffn_sigmoid_amd import synth
    inp = dict(v3_weights)
    inp["x"] = synth.normal((wl.T, wl.H), wl.x_std, torch.bfloat16, "cuda", wl.seed, f"x_T{wl.T}")
    inp["bias"] = synth.zipf_bias(wl.N, wl.bias_param, "cuda", wl.seed)
    out, aux, d, toks = _run(wl, inp, 2048)
    assert wl.capacity == 640
    assert d["n_dropped"] > 0 and len(toks) >= 2048
    with_drop = int((d["inv_row"] < 0).any(axis=1).sum())
    assert int(((d["inv_row"][toks] < 0).any(axis=1)).sum()) >= min(64, with_drop)
    assert int(np.max(np.diff(d["offsets"]))) <= wl.capacity
