"""GPU parity of every entry point at sizes the oracle finishes in seconds,
with ragged tails, empty segments, ties, drops and degenerate shapes."""
import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import synth, workloads

from gpu_common import (BF16_MAXREL, BF16_RELL2, F32_MAXREL, check_dispatch, check_outputs,
                        check_routing, check_stats, f64, gpu, layer_forward, make_inputs,
                        normwise, oracle_route, oracle_rows, require_gpu, say, typed)

pytestmark = gpu


def _route_only(wl, logits, bias):
    cfg = moe.make_cfg(wl)
    T, k = wl.T, wl.k
    dev = "cuda"
    lg = logits.clone()
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    score = torch.empty((T, k), dtype=torch.float32, device=dev)
    lse = torch.empty((T,), dtype=torch.float32, device=dev)
    moe.moe_route(cfg, None, None, lg, bias, idx, gate, score, lse)
    torch.cuda.synchronize()
    return dict(logits=lg, topk_idx=idx, topk_gate=gate, topk_score=score, token_lse=lse)


def test_sigmoid_scores_bit_identical_to_oracle_on_a_sweep():
    """All 64 scores of each token are returned (k = N = 64, no groups), so the
    GPU's fp32 sigmoid is compared bit for bit with the oracle's."""
    require_gpu()
    vals = np.concatenate([
        np.linspace(-90, 90, 1 << 20, dtype=np.float32),
        np.arange(0, 0x42B40000, 4099, dtype=np.uint32).view(np.float32),
    ])
    vals = np.concatenate([vals, -vals])
    n = (vals.size // 64) * 64
    logits = torch.from_numpy(vals[:n].reshape(-1, 64).copy()).cuda()
    wl = workloads.TINY.with_(T=logits.shape[0], N=64, k=64, n_groups=1, topk_groups=1,
                              norm_topk=0)
    say(f"sigmoid sweep: {n} values")
    g = _route_only(wl, logits, None)
    r = oracle_route(wl, logits.cpu().numpy(), None)
    np.testing.assert_array_equal(g["topk_idx"].cpu().numpy(), r["topk_idx"])
    np.testing.assert_array_equal(g["topk_score"].cpu().numpy(), r["topk_score"])


@pytest.mark.parametrize("N,k", [(64, 64), (160, 64), (256, 64), (16, 16), (4, 4)])
def test_softmax_scores_bit_identical_to_oracle(N, k):
    """The fp32 softmax (exact exponential, terms 64 below the maximum set
    to 0, pairwise sum over 256 slots, correctly rounded divide) on the GPU
    and in the oracle, bit for bit: the k largest scores of each token at
    logit scales from 0.05 to 40 (the largest cross the cut-off), with ties
    and a token of equal logits."""
    require_gpu()
    rng = np.random.default_rng(N + k)
    T = 4096
    scale = rng.choice([0.05, 0.5, 2.0, 8.0, 40.0], size=(T, 1)).astype(np.float32)
    logits = (rng.standard_normal((T, N)).astype(np.float32) * scale).astype(np.float32)
    logits[:64] = np.round(logits[:64])  # ties
    logits[64] = 1.25                    # all equal
    wl = workloads.TINY.with_(T=T, N=N, k=k, n_groups=1, topk_groups=1,
                              score_fn=workloads.SOFTMAX, norm_topk=0)
    say(f"softmax scores N={N} k={k}")
    g = _route_only(wl, torch.from_numpy(logits).cuda(), None)
    r = oracle_route(wl, logits, None)
    np.testing.assert_array_equal(g["topk_idx"].cpu().numpy(), r["topk_idx"])
    np.testing.assert_array_equal(g["topk_score"].cpu().numpy(), r["topk_score"])
    mr, _ = normwise(g["token_lse"].cpu().numpy(), r["lse"])
    assert mr <= F32_MAXREL, f"lse max-rel {mr}"


@pytest.mark.parametrize("G,keep,k,topn", [(4, 2, 4, 2), (4, 1, 3, 1), (2, 1, 5, 2), (1, 1, 6, 2)])
@pytest.mark.parametrize("fn", [workloads.SIGMOID, workloads.SOFTMAX])
def test_route_ties_match_oracle(G, keep, k, topn, fn):
    """Integer-valued keys with many ties: ties must resolve to the lower
    group / expert index exactly as in the oracle."""
    require_gpu()
    rng = np.random.default_rng(G * 100 + k * 10 + topn + fn)
    T, N = 333, 16
    if fn == workloads.SIGMOID:
        logits = np.zeros((T, N), np.float32)  # every score exactly 0.5
        bias = rng.integers(-2, 3, size=N).astype(np.float32)
        # vary keys per token through the logit: l = 0 or a large value
        logits = (rng.integers(0, 2, size=(T, N)) * 30.0).astype(np.float32)
    else:
        logits = rng.integers(-3, 4, size=(T, N)).astype(np.float32)
        bias = None
    wl = workloads.TINY.with_(T=T, N=N, k=k, n_groups=G, topk_groups=keep, group_topn=topn,
                              score_fn=fn, norm_topk=1 if fn == workloads.SIGMOID else 0)
    say(f"ties: G={G} keep={keep} k={k} topn={topn} fn={fn}")
    bt = torch.from_numpy(bias).cuda() if bias is not None else None
    g = _route_only(wl, torch.from_numpy(logits).cuda(), bt)
    r = oracle_route(wl, logits, bias)
    np.testing.assert_array_equal(g["topk_idx"].cpu().numpy(), r["topk_idx"])
    mr, _ = normwise(g["topk_gate"].cpu().numpy(), r["topk_gate"])
    assert mr <= F32_MAXREL


def test_uniform_routing_balance_loss_is_one_on_gpu():
    """Construction with exactly uniform routing: L_B = 1 within fp32."""
    require_gpu()
    T, N, k = 64, 16, 4
    logits = np.full((T, N), -1000.0, np.float32)
    for t in range(T):
        for j in range(k):
            logits[t, (4 * t + j) % N] = 0.0
    wl = workloads.TINY.with_(T=T, N=N, k=k, n_groups=1, topk_groups=1, score_fn=workloads.SOFTMAX,
                              norm_topk=0)
    cfg = moe.make_cfg(wl)
    g = _route_only(wl, torch.from_numpy(logits).cuda(), None)
    ws = moe.alloc_workspace(cfg)
    counts = torch.empty(N, dtype=torch.int32, device="cuda")
    offsets = torch.empty(N + 1, dtype=torch.int32, device="cuda")
    rt = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty((T, k), dtype=torch.int32, device="cuda")
    moe.moe_permute(cfg, g["topk_idx"], g["topk_score"], None, counts, offsets, rt, inv, ws=ws)
    f = torch.empty(N, device="cuda")
    P = torch.empty(N, device="cuda")
    sc = torch.empty(3, device="cuda")
    moe.moe_load_stats(cfg, counts, g["token_lse"], g["logits"], f, P, sc, ws)
    torch.cuda.synchronize()
    assert np.all(counts.cpu().numpy() == T * k // N)
    assert abs(float(sc[0]) - 1.0) <= 1e-6
    assert abs(float(sc[1]) - np.log(4)) <= 1e-6


@pytest.mark.parametrize("T", [64, 77, 1, 300])
def test_tiny_layer_full_parity(T):
    """fp32 tiny layer: every output row against the oracle at 1e-5."""
    require_gpu()
    wl = workloads.TINY.with_(T=T)
    say(f"tiny layer T={T}")
    inp = make_inputs(wl)
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    check_stats(wl, aux)
    toks = list(range(T))
    ref = oracle_rows(wl, inp, r, d, toks)
    mr, _ = check_outputs(wl, out, ref, toks)
    say(f"  max-rel {mr:.2e}")


@pytest.mark.parametrize("C", [1, 3, 17])
def test_tiny_layer_with_capacity_drops(C):
    require_gpu()
    wl = workloads.TINY.with_(T=200, capacity=C)
    say(f"tiny capacity C={C}")
    inp = make_inputs(wl)
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    assert d["n_dropped"] > 0
    toks = list(range(wl.T))
    ref = oracle_rows(wl, inp, r, d, toks)
    check_outputs(wl, out, ref, toks)


def test_shared_only_and_empty_batch():
    require_gpu()
    wl = workloads.TINY.with_(k=0)
    inp = make_inputs(wl)
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    ref = oracle_rows(wl, inp, r, d, list(range(wl.T)))
    check_outputs(wl, out, ref, list(range(wl.T)))
    wl0 = workloads.TINY.with_(T=0)
    inp0 = make_inputs(wl0)
    out0, aux0 = layer_forward(wl0, inp0)
    assert out0.numel() == 0 and int(aux0["offsets"][-1]) == 0


def test_bf16_small_layer_parity_and_determinism():
    """A small bf16 V3-like layer (groups, sigmoid, scale 2.5) exercising the
    MFMA path with ragged segments."""
    require_gpu()
    wl = workloads.V3_PREFILL.with_(T=333, H=256, N=32, k=4, n_groups=4, topk_groups=2, I=128,
                                    I_shared=192)
    say("bf16 small layer")
    inp = make_inputs(wl)
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    check_stats(wl, aux)
    toks = list(range(0, wl.T, 7))
    ref = oracle_rows(wl, inp, r, d, toks)
    mr, l2 = check_outputs(wl, out, ref, toks)
    say(f"  max-rel {mr:.2e} rel-L2 {l2:.2e}")
    out2, aux2 = layer_forward(wl, inp)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    for n in ("topk_idx", "topk_gate", "row_token", "inv_row", "f", "P", "scalars"):
        assert torch.equal(aux[n], aux2[n]), n


@pytest.mark.parametrize("rows_per_seg,inter,H", [(5, 192, 256), (40, 192, 256), (150, 192, 256),
                                                   (400, 192, 256), (150, 2048, 256),
                                                   (400, 2048, 256), (150, 2048, 448),
                                                   (150, 128, 128), (150, 256, 4096),
                                                   (300, 128, 4096), (150, 1408, 256),
                                                   (600, 1024, 384), (700, 2048, 256)])
def test_grouped_ffn_ragged_segments(rows_per_seg, inter, H):
    """moe_grouped_ffn alone: ragged and empty segments, every tile height.
    Large segments run the gate/up projection on the ping-pong kernel when
    K = H is a multiple of 128 from 256 (eight k-steps: only its first and
    last blocks of four) up to 4096 here, on the 2-stage kernel for H = 128
    and 448; expert widths of 1024, 1408 and 2048 send the down projection to
    the ping-pong kernel too (K >= 1024; with H = 384 its second column tile
    is partial), 128-256 through the 2-stage kernel.  The last case has more
    gate/up tiles than workgroups at eight k-steps per tile, so tiles of
    different heights follow each other in one workgroup's stream."""
    require_gpu()
    rng = np.random.default_rng(rows_per_seg)
    nseg = 9
    sizes = rng.integers(0, 2 * rows_per_seg, size=nseg)
    sizes[2] = 0
    sizes[5] = 3 * rows_per_seg + 7
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offs[-1])
    wl = workloads.V3_PREFILL.with_(H=H, N=16, n_groups=1, topk_groups=1, k=2, I=64)
    cfg = moe.make_cfg(wl)
    say(f"grouped ffn: inter={inter} sizes={sizes.tolist()}")
    a = synth.normal((M, H), 1.0, torch.bfloat16, "cuda", 1, "a")
    w13 = synth.normal((nseg, 2 * inter, H), 0.02, torch.bfloat16, "cuda", 1, "w13")
    w2 = synth.normal((nseg, H, inter), 0.02, torch.bfloat16, "cuda", 1, "w2")
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_grouped_ffn_workspace_size(cfg, M, inter), dtype=torch.uint8,
                     device="cuda")
    moe.moe_grouped_ffn(cfg, nseg, torch.from_numpy(offs).cuda(), M, inter, a, None,
                        moe.pack_weights(w13), moe.pack_weights(w2),
                        y, ws)
    torch.cuda.synchronize()
    an = typed(a)
    w13n, w2n = typed(w13), typed(w2)
    ref = np.empty((M, H))
    for s in range(nseg):
        for r_ in range(offs[s], offs[s + 1]):
            ref[r_] = oracle.swiglu_row(an[r_], w13n[s], w2n[s])
    mr, l2 = normwise(f64(y), ref)
    say(f"  max-rel {mr:.2e} rel-L2 {l2:.2e}")
    assert mr <= BF16_MAXREL and l2 <= BF16_RELL2


def test_grouped_ffn_activation_buffer_within_256mib_of_4gib():
    """An activation buffer of 4.1e9 bytes: the large-tile kernels address
    it with 32-bit offsets, so rows past a partial tile's end repeat its last
    valid row there instead of reading from past the buffer's end (the zero
    padding used below that size could wrap).  Rows of every segment's
    partial last tile and of its first tile are compared with the oracle."""
    require_gpu()
    H, inter = 2048, 128
    sizes = np.array([400000, 300007, 300013])
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offs[-1])
    assert 0xF0000000 < M * H * 2 < 0xFFFFFFFF
    wl = workloads.V3_PREFILL.with_(H=H, N=16, n_groups=1, topk_groups=1, k=2, I=64)
    cfg = moe.make_cfg(wl)
    say(f"grouped ffn near 4 GiB: M={M} H={H} inter={inter}")
    a = synth.normal((M, H), 1.0, torch.bfloat16, "cuda", 2, "a", chunk_dim0=False)
    w13 = synth.normal((3, 2 * inter, H), 0.02, torch.bfloat16, "cuda", 2, "w13")
    w2 = synth.normal((3, H, inter), 0.02, torch.bfloat16, "cuda", 2, "w2")
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_grouped_ffn_workspace_size(cfg, M, inter), dtype=torch.uint8,
                     device="cuda")
    moe.moe_grouped_ffn(cfg, 3, torch.from_numpy(offs).cuda(), M, inter, a, None,
                        moe.pack_weights(w13), moe.pack_weights(w2), y, ws)
    torch.cuda.synchronize()
    rows = []
    for sg in range(3):
        rows += list(range(offs[sg], offs[sg] + 3)) + list(range(offs[sg + 1] - 40, offs[sg + 1]))
    idx = torch.tensor(rows, device="cuda")
    an = typed(a[idx].cpu())
    w13n, w2n = typed(w13), typed(w2)
    ref = np.empty((len(rows), H))
    for i, r_ in enumerate(rows):
        sg = int(np.searchsorted(offs, r_, side="right") - 1)
        ref[i] = oracle.swiglu_row(an[i], w13n[sg], w2n[sg])
    got = y[idx].float().cpu().numpy().astype(np.float64)
    mr, l2 = normwise(got, ref)
    say(f"  max-rel {mr:.2e} rel-L2 {l2:.2e}")
    assert mr <= BF16_MAXREL and l2 <= BF16_RELL2


@pytest.mark.parametrize("T,I", [(1024, 192), (1500, 128)])
def test_bf16_layer_with_large_segments(T, I):
    """Segments of ~hundreds of rows (the large-segment kernel), an odd
    number of k-steps (I = 192) and a ragged token count."""
    require_gpu()
    wl = workloads.V3_PREFILL.with_(T=T, H=256, N=8, k=2, n_groups=2, topk_groups=1, I=I,
                                    I_shared=128)
    say(f"bf16 large segments T={T} I={I}")
    inp = make_inputs(wl)
    out, aux = layer_forward(wl, inp)
    r = check_routing(wl, aux, inp["bias"])
    d = check_dispatch(wl, aux, r)
    toks = list(range(0, wl.T, 37))
    ref = oracle_rows(wl, inp, r, d, toks)
    mr, l2 = check_outputs(wl, out, ref, toks)
    say(f"  max-rel {mr:.2e} rel-L2 {l2:.2e}")


def test_combine_and_bias_update_match_oracle():
    require_gpu()
    rng = np.random.default_rng(21)
    T, H, k, M = 50, 256, 4, 230
    wl = workloads.V3_PREFILL.with_(T=T, H=H, N=16, n_groups=1, topk_groups=1, k=k, I=64)
    cfg = moe.make_cfg(wl)
    y = synth.normal((M, H), 1.0, torch.bfloat16, "cuda", 2, "y")
    ysh = synth.normal((T, H), 1.0, torch.bfloat16, "cuda", 2, "ysh")
    inv = rng.permutation(M)[:T * k].reshape(T, k).astype(np.int32)
    inv[rng.random((T, k)) < 0.2] = -1
    gate = rng.random((T, k)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(cfg, y, torch.from_numpy(inv).cuda(), torch.from_numpy(gate).cuda(), ysh, out)
    torch.cuda.synchronize()
    ref = oracle.combine(typed(y), typed(ysh), inv, gate.astype(np.float64))
    mr, l2 = normwise(f64(out), ref)
    assert mr <= BF16_MAXREL and l2 <= BF16_RELL2
    # bias update: exact
    counts = rng.integers(0, 40, size=16).astype(np.int32)
    counts[3] = int(round(counts.mean()))
    bias = rng.uniform(-0.1, 0.1, 16).astype(np.float32)
    bt = torch.from_numpy(bias.copy()).cuda()
    moe.moe_bias_update(cfg, torch.from_numpy(counts).cuda(), bt, 0.001)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bt.cpu().numpy(), oracle.bias_update(counts, bias, 0.001))


def test_combine_rounds_once_to_nearest_even():
    """The combine accumulates in fp32 and rounds once to bf16, to nearest
    with ties to even.  Inputs are chosen so that every product and sum is
    exact in fp32 (small integer gates, values on a 2^-8 grid below 2^12),
    so the expected output is the round-to-nearest-even of the exact sum,
    computed here from the definition; about half the outputs are ties."""
    require_gpu()
    rng = np.random.default_rng(33)
    T, H, k, M = 64, 256, 3, 200
    wl = workloads.V3_PREFILL.with_(T=T, H=H, N=16, n_groups=1, topk_groups=1, k=k, I=64)
    cfg = moe.make_cfg(wl)
    # bf16 values: odd multiples of 2^-8 (|m| < 256), shared values with an
    # exponent that puts the sum's rounding bit at 2^-8 or 2^-7
    y_np = (rng.integers(-127, 128, size=(M, H)) * 2 + 1).astype(np.float32) / 256.0
    ysh_np = rng.choice(np.array([1.0, -1.0, 2.0, -2.0, 1.5, 3.0], np.float32), size=(T, H))
    inv = rng.permutation(M)[:T * k].reshape(T, k).astype(np.int32)
    inv[rng.random((T, k)) < 0.2] = -1
    gate = rng.integers(1, 4, size=(T, k)).astype(np.float32)
    y = torch.from_numpy(y_np).to(torch.bfloat16).cuda()
    ysh = torch.from_numpy(ysh_np).to(torch.bfloat16).cuda()
    assert torch.equal(y.float().cpu(), torch.from_numpy(y_np))  # inputs exact in bf16
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(cfg, y, torch.from_numpy(inv).cuda(), torch.from_numpy(gate).cuda(), ysh, out)
    torch.cuda.synchronize()
    exact = ysh_np.astype(np.float64).copy()
    for j in range(k):
        kept = inv[:, j] >= 0
        exact[kept] += gate[kept, j, None].astype(np.float64) * y_np[inv[kept, j]].astype(np.float64)
    f32 = exact.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), exact)  # the sum is exact in fp32
    u = f32.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    ties = int(((u & 0xFFFF) == 0x8000).sum())
    say(f"combine rounding: {ties} ties of {u.size}")
    assert ties > u.size // 8
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("T", [96, 600])
def test_granular_calls_compose_to_layer_forward(T):
    """route -> permute -> grouped_ffn -> combine gives the layer's output, and
    the layer's fused route -> dispatch counting (per-block expert counts
    added up by the route kernel) gives exactly the dispatch of the granular
    calls, whose moe_permute counts on its own; T = 600 spans three dispatch
    blocks of 256 tokens."""
    require_gpu()
    wl = workloads.TINY.with_(T=T, n_shared=0)
    cfg = moe.make_cfg(wl)
    inp = make_inputs(wl)
    out_ref, aux = layer_forward(wl, inp)
    T, N, k, H = wl.T, wl.N, wl.k, wl.H
    dev = "cuda"
    ws = moe.alloc_workspace(cfg)
    lg = torch.empty((T, N), device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), device=dev)
    score = torch.empty((T, k), device=dev)
    moe.moe_route(cfg, inp["x"], inp["w_router"], lg, inp["bias"], idx, gate, score, None, ws)
    counts = torch.empty(N, dtype=torch.int32, device=dev)
    offs = torch.empty(N + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    xp = torch.empty((T * k, H), device=dev)
    moe.moe_permute(cfg, idx, score, inp["x"], counts, offs, rt, inv, xp, ws=ws)
    torch.cuda.synchronize()
    M = int(offs[-1])
    assert torch.equal(xp[:M], inp["x"][rt[:M].long()])
    for name, got in (("counts", counts), ("offsets", offs), ("inv_row", inv)):
        assert torch.equal(got, aux[name]), name
    assert torch.equal(rt[:M], aux["row_token"][:M])
    y = torch.empty((T * k, H), device=dev)
    ws2 = torch.empty(moe.moe_grouped_ffn_workspace_size(cfg, T * k, wl.I), dtype=torch.uint8,
                      device=dev)
    moe.moe_grouped_ffn(cfg, N, offs, T * k, wl.I, xp, None, inp["w13"], inp["w2"], y, ws2)
    out = torch.empty((T, H), device=dev)
    moe.moe_combine(cfg, y, inv, gate, None, out)
    torch.cuda.synchronize()
    mr, _ = normwise(f64(out), f64(out_ref))
    assert mr <= F32_MAXREL


@pytest.mark.parametrize("shape", [(3, 48, 96), (1, 16, 32), (2, 4096, 7168)])
def test_pack_weights_layout(shape):
    """moe_pack_weights against the tiled layout written out element by
    element: block (i, j) of 16 rows x 32 columns at (i*(K/32) + j)*512,
    chunk l of the block = row 16i + l%16, columns 32j + 8(l/16) .. +7."""
    require_gpu()
    n, R, K = shape
    say(f"pack {shape}")
    w = torch.arange(n * R * K, device="cuda", dtype=torch.int32).reshape(n, R, K)
    w = (w % 65521).to(torch.int16).view(torch.bfloat16)  # distinct-ish bit patterns
    p = moe.pack_weights(w)
    torch.cuda.synchronize()
    src = w.view(torch.int16).cpu().numpy()
    got = p.view(torch.int16).cpu().numpy().reshape(n, R * K)
    # reference built with numpy index arithmetic
    blk = src.reshape(n, R // 16, 16, K // 32, 4, 8)        # mat, i, row-in-block, j, chunk, e
    ref = blk.transpose(0, 1, 3, 4, 2, 5).reshape(n, R * K)  # mat, i, j, chunk, row, e
    np.testing.assert_array_equal(got, ref)
