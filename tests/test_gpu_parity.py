"""GPU parity: the HIP layer (through the C ABI) against the oracle.

Small cases are compared on every token; the full Step-3.5-Flash shapes on
every token where the oracle is quick (decode batches) and on a spread sample
of tokens otherwise.  See tests/moe_check.py for the comparison rules.
"""
import numpy as np
import pytest
import torch

import moe_synth
from moe_check import compare, make_layer, run_gpu, tile_edge_tokens

pytestmark = pytest.mark.gpu

W = moe_synth.WORKLOADS


def _say(*a):
    print("[case]", *a, flush=True)


def _run(shape, seed=0, tokens=None, max_tokens=None, layer_kw=None, cmp_kw=None, sample=None,
         edges=None):
    """Runs one case; shapes other than the benchmarked workloads may use the
    rounding-aware output check (see moe_check).  edges: also compare the
    tokens at the first and last row of every m-tile of every group (a dict of
    tile_edge_tokens arguments), read off the GPU's own dispatch."""
    cmp_kw = dict(cmp_kw or {})
    cmp_kw.setdefault("strict", shape.name in W)
    _say(shape.name, f"seed={seed}", f"tokens={tokens or shape.tokens}", layer_kw or "")
    inp = moe_synth.make_layer(shape, seed=seed, device="cuda",
                               tokens=max(tokens or 0, shape.tokens))
    layer = make_layer(shape, max_tokens=max_tokens or shape.tokens, **(layer_kw or {}))
    layer.pack_inputs(inp)
    out, route = run_gpu(layer, inp, tokens)
    if edges is not None:
        T = out.shape[0]
        sh = T if shape.shared_inter else None
        sample = sorted(set(sample or []) | set(tile_edge_tokens(route, shape.top_k, T=sh,
                                                                 **edges)))
        _say("tile-edge sample", len(sample), "tokens")
    res = compare(inp, out, route, sample=sample, **cmp_kw)
    _say("ok", res)
    return inp, layer, out, route, res


# ----------------------------------------------------------------- tiny (fp32 activations)

@pytest.mark.parametrize("tokens", [64, 1, 7, 33])
def test_tiny_ragged(tokens):
    _run(W["tiny"], tokens=tokens, max_tokens=64)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_seeds(seed):
    _run(W["tiny"], seed=seed)


def test_tiny_bf16_activations():
    _run(W["tiny"].replace(name="tiny_bf16", act_dtype="bf16"))


def test_tiny_no_shared_expert():
    _run(W["tiny"].replace(name="tiny_noshared", shared_inter=0))


@pytest.mark.parametrize("k", [1, 16])
def test_tiny_k_extremes(k):
    _run(W["tiny"].replace(name=f"tiny_k{k}", top_k=k))


def test_tiny_no_renorm():
    s = W["tiny"].replace(name="tiny_norenorm", renormalize=False)
    _run(s, cmp_kw=dict(renormalize=False))


@pytest.mark.parametrize("bias_mode", ["logit", "select"])
def test_tiny_sigmoid_router_with_bias(bias_mode):
    """The page's router configuration: sigmoid scores, a router bias,
    renormalised weights scaled by 3."""
    s = W["tiny"].replace(name=f"tiny_sigmoid_{bias_mode}")
    inp = moe_synth.make_layer(s, seed=0, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    inp.router_bias = torch.randn(s.experts, generator=g, device="cuda", dtype=torch.float32)
    _say(s.name)
    layer = make_layer(s, score="sigmoid", routed_scale=3.0, bias_mode=bias_mode)
    layer.pack_inputs(inp)
    out, route = run_gpu(layer, inp)
    res = compare(inp, out, route, score="sigmoid", routed_scale=3.0, bias_mode=bias_mode)
    _say("ok", res)


def test_tiny_sigmoid_without_renorm():
    """Sigmoid scores without renormalisation: each weight is the selected
    expert's sigmoid score times routed_scale."""
    s = W["tiny"].replace(name="tiny_sigmoid_norenorm", renormalize=False, score="sigmoid",
                          routed_scale=2.5)
    _run(s)


def test_int4_large_batch_sampled():
    """INT4-g32 weights past 1024 tokens: the multi-workgroup dispatch and the
    INT4 streaming kernels with 32-row tiles, full layer shape, sampled tokens."""
    s = W["int4_decode"].replace(name="int4_1537", tokens=1537)
    _run(s, sample=_spread(1537, 10))


def test_tiny_int4():
    s = W["tiny"].replace(name="tiny_int4", act_dtype="bf16", weight_dtype="int4_g32", inter=128,
                          shared_inter=128)
    _run(s)


def test_tiny_int4_f32_activations():
    s = W["tiny"].replace(name="tiny_int4_f32", weight_dtype="int4_g32", inter=128,
                          shared_inter=128)
    _run(s)


def test_exact_ties_go_to_lower_index():
    """Duplicated router rows give bitwise-equal logits; the lower index must win."""
    s = W["tiny"].replace(name="tiny_ties", act_dtype="bf16")
    inp = moe_synth.make_layer(s, seed=5, device="cuda")
    for a, b in [(1, 9), (3, 4), (0, 15), (7, 12)]:
        inp.router_w[b] = inp.router_w[a]
    _say(s.name)
    layer = make_layer(s)
    layer.pack_inputs(inp)
    out, route = run_gpu(layer, inp)
    idx = route.topk_idx.cpu().numpy()
    both_seen = 0
    for a, b in [(1, 9), (3, 4), (0, 15), (7, 12)]:
        has_a = (idx == a).any(axis=1)
        has_b = (idx == b).any(axis=1)
        assert not (has_b & ~has_a).any(), f"expert {b} chosen over its twin {a}"
        both = has_a & has_b   # both twins selected: the lower one ranks first
        ja = np.argmax(idx == a, axis=1)
        jb = np.argmax(idx == b, axis=1)
        assert (ja[both] < jb[both]).all(), f"twin {b} ranked before {a}"
        both_seen += int(both.sum())
    assert both_seen > 0
    compare(inp, out, route)


def test_zero_tokens_is_noop():
    s = W["tiny"]
    inp = moe_synth.make_layer(s, seed=0, device="cuda")
    layer = make_layer(s)
    layer.pack_inputs(inp)
    out = layer.forward(inp.x[:0], inp.router_w)
    torch.cuda.synchronize()
    assert out.shape == (0, s.hidden)


def test_deterministic():
    s = W["tiny"].replace(name="tiny_bf16", act_dtype="bf16")
    inp = moe_synth.make_layer(s, seed=0, device="cuda")
    layer = make_layer(s)
    layer.pack_inputs(inp)
    o1, r1 = run_gpu(layer, inp)
    o2, r2 = run_gpu(layer, inp)
    assert torch.equal(o1, o2)
    assert torch.equal(r1.perm, r2.perm) and torch.equal(r1.topk_idx, r2.topk_idx)


def test_concurrent_streams_one_handle():
    """Forwards on one handle, on two streams at once, each with its own
    workspace and output, give bit for bit what each gives alone: a 32-token
    batch (fused top-k + dispatch, streaming GEMMs) beside a 700-token one
    (LDS-staged router, tiled GEMMs)."""
    s = W["tiny"].replace(name="tiny_bf16_732", act_dtype="bf16", tokens=732)
    inp = moe_synth.make_layer(s, seed=3, device="cuda")
    layer = make_layer(s)
    layer.pack_inputs(inp)
    xa, xb = inp.x[:32].contiguous(), inp.x[32:].contiguous()
    ref_a = layer.forward(xa, inp.router_w)
    ref_b = layer.forward(xb, inp.router_w)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        ws_a = torch.empty(layer.workspace_bytes(32), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(layer.workspace_bytes(xb.shape[0]), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            oa = layer.forward(xa, inp.router_w, workspace=ws_a)
        with torch.cuda.stream(s2):
            ob = layer.forward(xb, inp.router_w, workspace=ws_b)
        torch.cuda.synchronize()
        _say("concurrent", rep)
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


def test_concurrent_streams_share_the_second_stream():
    """Two hot-expert batches (a router bias makes three of 64 experts hot)
    on one handle, on two streams at once, each with its own workspace and
    output: both put their LDS-tiled GEMMs on the handle's one second stream,
    and each output equals, bit for bit, that batch's forward alone."""
    s = W["tiny"].replace(name="tiny_bf16_hot_pair", act_dtype="bf16", experts=64, top_k=2,
                          tokens=640)   # 256 + 384 tokens: 8 and 12 rows per expert, streaming
    inp = moe_synth.make_layer(s, seed=5, device="cuda")
    bias = torch.zeros(s.experts, device="cuda", dtype=torch.float32)
    bias[:3] = 3.0
    layer = make_layer(s)
    layer.pack_inputs(inp)
    xa, xb = inp.x[:256].contiguous(), inp.x[256:].contiguous()
    ref_a, ra = layer.forward(xa, inp.router_w, bias, return_route=True)
    ref_b, rb = layer.forward(xb, inp.router_w, bias, return_route=True)
    torch.cuda.synchronize()
    for r in (ra, rb):   # hot experts (LDS tiles on the second stream) and streaming ones
        c = r.expert_counts.cpu().numpy()
        assert (c[:3] >= 32).all() and (c[3:] < 32).all(), c
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        ws_a = torch.empty(layer.workspace_bytes(xa.shape[0]), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(layer.workspace_bytes(xb.shape[0]), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            oa = layer.forward(xa, inp.router_w, bias, workspace=ws_a)
        with torch.cuda.stream(s2):
            ob = layer.forward(xb, inp.router_w, bias, workspace=ws_b)
        torch.cuda.synchronize()
        _say("concurrent hot batches", rep)
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


@pytest.mark.parametrize("tokens,experts", [(32, 16), (600, 16), (256, 64)])
def test_graph_capture_replays(tokens, experts):
    """A forward captured in a HIP graph (no host synchronisation, no memset
    nodes: the fused dispatch's counter is cleared by a kernel) replays to the
    eager result bit for bit, with other eager forwards in between: streaming
    GEMMs, LDS-tiled GEMMs, and streaming with hot experts on a second tile
    list (a router bias makes three of 64 experts hot)."""
    s = W["tiny"].replace(name=f"tiny_bf16_graph_{tokens}", act_dtype="bf16", tokens=tokens,
                          experts=experts)
    inp = moe_synth.make_layer(s, seed=4, device="cuda")
    bias = None
    if experts == 64:
        bias = torch.zeros(experts, device="cuda", dtype=torch.float32)
        bias[:3] = 3.0
    layer = make_layer(s)
    layer.pack_inputs(inp)
    x = inp.x.clone()
    ref = layer.forward(x, inp.router_w, bias)
    out = torch.empty_like(ref)
    ws = torch.empty(layer.workspace_bytes(tokens), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the capture
        layer.forward(x, inp.router_w, bias, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x, inp.router_w, bias, out=out, workspace=ws)
    other = torch.flip(inp.x, dims=[0]).contiguous()
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _say("graph replay", rep)
        assert torch.equal(out, ref)
        layer.forward(other, inp.router_w, bias)   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fill", ["zeros", "ones", "ramp", "random"])
def test_small_batch_workspace_of_any_contents(fill):
    """No state carries over through the workspace: one holding zeros, all
    ones, a ramp of 64-bit words or random bytes, and one last used by
    batches of other sizes (other offsets for every buffer, the fused top-k +
    dispatch's completion counter among them), give the output and routing of
    a fresh workspace, bit for bit -- batches of 1 to 64 tokens, whose
    dispatch runs on one wave."""
    s = W["tiny"].replace(name="tiny_bf16_ws", act_dtype="bf16", tokens=64)
    inp = moe_synth.make_layer(s, seed=8, device="cuda")
    layer = make_layer(s)
    layer.pack_inputs(inp)
    sizes = (48, 17, 64, 1, 48, 48)
    refs = {t: layer.forward(inp.x[:t].contiguous(), inp.router_w, return_route=True)
            for t in set(sizes)}
    torch.cuda.synchronize()
    nbytes = max(layer.workspace_bytes(t) for t in sizes)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(255)
    elif fill == "ramp":
        ws.view(torch.int64).copy_(torch.arange(nbytes // 8, dtype=torch.int64, device="cuda"))
    else:
        g = torch.Generator(device="cuda").manual_seed(11)
        ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g))
    for t in sizes:
        out, route = layer.forward(inp.x[:t].contiguous(), inp.router_w, workspace=ws,
                                   return_route=True)
        torch.cuda.synchronize()
        _say("workspace", fill, "tokens", t)
        ref, rref = refs[t]
        assert torch.equal(out, ref)
        for name in ("topk_idx", "topk_w", "expert_counts", "expert_offsets", "perm", "inv"):
            assert torch.equal(getattr(route, name), getattr(rref, name)), name


@pytest.mark.parametrize("tokens", [32, 200, 1500])
def test_timed_forward_matches(tokens):
    """The timed entry point runs the same kernels as the plain one (same
    output bit for bit) and leaves five finite, positive stage durations, on
    batches whose fused top-k + dispatch ends in the one-wave dispatch (32
    tokens) or the one-workgroup dispatch (200), and on one with the
    multi-workgroup dispatch."""
    from sparse_mixture_experts_layer_amd import _binding as B
    s = W["tiny"].replace(name=f"tiny_bf16_timed_{tokens}", act_dtype="bf16", tokens=tokens)
    inp = moe_synth.make_layer(s, seed=6, device="cuda")
    layer = make_layer(s)
    layer.pack_inputs(inp)
    ref = layer.forward(inp.x, inp.router_w)
    ev = B.StageEvents(sets=2)
    outs = [layer.forward(inp.x, inp.router_w, stage_events=ev, event_set=i) for i in range(2)]
    torch.cuda.synchronize()
    _say("timed forward", tokens)
    for i, out in enumerate(outs):
        assert torch.equal(out, ref)
        ms = ev.stage_ms(i)
        assert len(ms) == len(B.STAGES) == 5
        assert all(np.isfinite(v) and v > 0 for v in ms), ms
    # only the gate/up stage's two boundaries recorded (NULL entries elsewhere)
    gu = B.STAGES.index("gate_up")
    part = B.StageEvents(sets=1, only=(gu, gu + 1))
    out = layer.forward(inp.x, inp.router_w, stage_events=part)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    ms = part.stage_ms(0)
    assert ms[gu] is not None and ms[gu] > 0 and all(v is None for j, v in enumerate(ms) if j != gu)


def test_argument_errors():
    from sparse_mixture_experts_layer_amd import _binding as B
    s = W["tiny"]
    inp = moe_synth.make_layer(s, seed=0, device="cuda")
    layer = make_layer(s, max_tokens=32)
    layer.pack_inputs(inp)
    with pytest.raises(B.MoeError) as e:   # T > max_tokens
        layer.forward(inp.x, inp.router_w)
    assert e.value.status == B.MOE_ERR_SHAPE
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as e:
        layer.forward(inp.x[:8], inp.router_w, workspace=ws)
    assert e.value.status == B.MOE_ERR_WORKSPACE


# ----------------------------------------------------------------- large-batch (tiled) path

TILED_SMALL = W["tiny"].replace(name="tiled_small", act_dtype="bf16", tokens=512)


@pytest.mark.parametrize("tokens", [512, 300, 1000])
def test_tiled_small_ragged(tokens):
    """16+ rows per expert selects the LDS-tiled GEMMs: partial 128-row tiles,
    intermediate width 64 (half a 256-row weight tile)."""
    _run(TILED_SMALL, tokens=tokens, max_tokens=1000)


def test_tiled_shared_width_differs():
    s = TILED_SMALL.replace(name="tiled_mid", hidden=512, experts=8, inter=256, shared_inter=128,
                            tokens=1024)
    _run(s)


def test_tiled_no_shared():
    _run(TILED_SMALL.replace(name="tiled_noshared", shared_inter=0))


@pytest.mark.parametrize("tokens,inter,shared_inter", [(4000, 96, 160), (3001, 64, 0)])
def test_tiled_many_rows_per_expert(tokens, inter, shared_inter):
    """Several hundred rows per expert (as in prefill): many m-tiles per
    expert, ragged row tails, a weight-block count that leaves a partial
    column tile (96 -> 3 gate/up blocks of 64), a shared expert wider than
    the routed ones."""
    s = TILED_SMALL.replace(name="tiled_deep", inter=inter, shared_inter=shared_inter, tokens=tokens)
    _run(s)


@pytest.mark.parametrize("tokens,hidden,inter,shared_inter,experts,top_k",
                         [(8192, 256, 1024, 1024, 8, 2), (16000, 512, 96, 160, 8, 2),
                          (16000, 256, 384, 0, 64, 2)])
def test_tiled_256_many_tiles(tokens, hidden, inter, shared_inter, experts, top_k):
    """256-row gate/up and down tiles with more tiles than CUs (several per
    CU): the shortest K of these shapes (hidden 256: 8 k-steps) and a longer
    one, ragged row tails, a partial column tile, a shared expert of another
    width, no shared expert.  Compared on every token."""
    s = TILED_SMALL.replace(name=f"tiled_256_{tokens}_{hidden}", experts=experts, top_k=top_k,
                            hidden=hidden, inter=inter, shared_inter=shared_inter, tokens=tokens)
    _run(s)


@pytest.mark.parametrize("shared_inter", [64, 0])
def test_hot_experts_take_tiles(shared_inter):
    """A load-imbalanced streaming batch: a router bias sends most tokens to
    three of 64 experts, which (with 32+ rows) go to the LDS-tiled GEMMs in
    128-row tiles while the other experts (and the shared one) stream.
    Compared on every token."""
    s = W["tiny"].replace(name=f"hot_experts_{shared_inter}", act_dtype="bf16", experts=64,
                          top_k=2, tokens=256, shared_inter=shared_inter)
    inp = moe_synth.make_layer(s, seed=6, device="cuda")
    bias = torch.zeros(s.experts, device="cuda", dtype=torch.float32)
    bias[:3] = 3.0
    inp.router_bias = bias
    _say(s.name)
    layer = make_layer(s)
    layer.pack_inputs(inp)
    out, route = run_gpu(layer, inp)
    counts = route.expert_counts.cpu().numpy()
    assert (counts[:3] >= 32).all() and (counts[3:] < 32).all(), counts
    res = compare(inp, out, route, strict=False)
    _say("ok", res)


@pytest.mark.parametrize("tokens,act", [(3001, "bf16"), (1537, "f32")])
def test_large_batch_dispatch(tokens, act):
    """Past 1024 tokens the dispatch runs over many workgroups (per-block
    counts, a scan, a per-block scatter); ragged block tails, 64 experts,
    top-8, compared on every token."""
    s = W["tiny"].replace(name=f"many_tokens_{act}", experts=64, top_k=8, act_dtype=act,
                          tokens=tokens)
    _run(s)


@pytest.mark.parametrize("act,experts,tokens", [("bf16", 2, 3), ("f32", 2, 3), ("bf16", 1, 100),
                                                ("bf16", 1, 200), ("bf16", 2, 700)])
def test_minimal_widths(act, experts, tokens):
    """The smallest widths the boundary accepts (hidden 64, expert widths 32):
    one K step of the router and of the down GEMM, one double step of the
    256-row gate/up tiles (200 rows on one expert), 128-row tiles (100 rows),
    the LDS-staged router with a single K step (700 tokens)."""
    s = W["tiny"].replace(name=f"minimal_{act}_{experts}_{tokens}", act_dtype=act, hidden=64,
                          experts=experts, top_k=1, inter=32, shared_inter=32, tokens=tokens)
    _run(s)


@pytest.mark.parametrize("tokens", [64, 700])
def test_max_experts_and_top_k(tokens):
    """The largest expert count and top-k the boundary accepts (512, 16): every
    top-k slot of every lane in use, 512-entry dispatch histograms, with 4-
    and 16-token top-k + dispatch workgroups."""
    s = W["tiny"].replace(name=f"max_e_k_{tokens}", act_dtype="bf16", experts=512, top_k=16,
                          tokens=tokens)
    _run(s)


@pytest.mark.parametrize("tokens", [40, 1100])
@pytest.mark.parametrize("experts", [65, 128, 129, 320, 321])
def test_topk_slot_variants(experts, tokens):
    """Expert counts at the edges of the compiled top-k variants (1, 2, 5 or 8
    expert slots per lane, the smallest that holds E is launched), through the
    fused top-k + dispatch launch (40 tokens) and the separate top-k launch
    (1100 tokens)."""
    s = W["tiny"].replace(name=f"slots_{experts}_{tokens}", act_dtype="bf16", experts=experts,
                          top_k=8, tokens=tokens)
    _run(s)


# ----------------------------------------------------------------- full Step-3.5-Flash shapes

def _spread(T, n, seed=0):
    rng = np.random.default_rng(seed)
    pick = set([0, T - 1, T // 2]) | set(rng.choice(T, size=n, replace=False).tolist())
    return sorted(pick)


def test_decode_32():
    _run(W["decode"])


def test_verify_256_zipf():
    _, _, _, route, _ = _run(W["verify"])
    counts = route.expert_counts.cpu().numpy()
    assert counts.max() > 150 and (counts > 0).sum() > 200   # skewed and wide


@pytest.mark.parametrize("tokens", [128, 512])
def test_batch_sizes_around_the_second_stream(tokens):
    """Zipf-routed batches below and above 256 tokens, through a handle that
    owns a second stream: at 128 tokens everything runs in order on the
    caller's stream and equals, bit for bit, a handle without a second stream
    (max_tokens 128); at 512 tokens the hot experts' LDS-tiled GEMMs run on
    the second stream, overlapping the streaming GEMMs.  Both against the
    oracle on sampled tokens."""
    s = W["verify"].replace(name=f"verify_{tokens}_aux", tokens=tokens)
    inp = moe_synth.make_layer(s, seed=0, device="cuda")
    side = make_layer(s, max_tokens=1024)
    side.pack_inputs(inp)
    out, route = run_gpu(side, inp)
    _say(s.name, "handle with a second stream")
    if tokens < 256:
        inorder = make_layer(s, max_tokens=tokens)
        inorder.pack_inputs(inp)
        ref, _ = run_gpu(inorder, inp)
        assert torch.equal(out, ref)
    else:
        counts = route.expert_counts.cpu().numpy()
        assert (counts >= 32).sum() >= 3, counts    # hot experts: LDS tiles on the second stream
    res = compare(inp, out, route, sample=_spread(tokens, 24), strict=True)
    _say("ok", res)


def test_prefill_16384_sampled():
    """Every token at the first or last row of a 128-row and of a 256-row
    m-tile of every expert and of the shared expert (what both tiled GEMMs
    cover: every tile, ragged group tails, the last shared tile), plus a
    spread of others."""
    _run(W["prefill"], sample=_spread(16384, 24), edges={})


def test_max_tokens_sampled():
    """The largest batch a handle accepts (2^18 tokens) at the full layer shape:
    Y alone holds (P+T)*H ~ 2.4e9 elements, past 32-bit indexing.  The
    dispatch of every pair is compared bit for bit, routing and outputs on
    sampled tokens (the first, middle and last among them)."""
    T = 1 << 18
    s = W["prefill"].replace(name="max_tokens", tokens=T)
    _run(s, sample=_spread(T, 16), cmp_kw={"strict": True},
         edges={"heights": (256,), "tiles_per_group": 1})


def test_int4_decode_32():
    _run(W["int4_decode"])


@pytest.mark.parametrize("tokens", [1, 5, 17])
def test_decode_ragged(tokens):
    _run(W["decode"], tokens=tokens, max_tokens=32)


@pytest.mark.parametrize("tokens", [128, 257, 1024, 1025])
def test_mid_size_batches_sampled(tokens):
    """Batch sizes between decode and prefill at the full layer shape: 128
    (2 token groups per tile), 257 (first size on 16-token top-k + dispatch
    workgroups), 1024 (LDS-staged router; last size of the fused top-k +
    dispatch: 64 tokens per dispatching wave), 1025 (first size on the
    multi-workgroup dispatch)."""
    s = W["decode"].replace(name=f"mid_{tokens}", tokens=tokens)
    _run(s, sample=_spread(tokens, 10), edges={"heights": (128,)} if tokens >= 1024 else None)


def test_int4_two_token_groups_sampled():
    """INT4 weights with 2 token groups per tile (the INT4 kernels' other
    register budget)."""
    s = W["int4_decode"].replace(name="int4_256", tokens=256)
    _run(s, sample=_spread(256, 10))


# ----------------------------------------------------------------- further shapes from the pages

STEP3 = W["decode"].replace(name="step3", hidden=7168, experts=48, top_k=3, inter=5120,
                            shared_inter=5120, renormalize=False, tokens=8)


def test_step3_shape_decode():
    """Step-3's MoE shape (llm-atlas comparison table: hidden 7168, 48 experts,
    top-3, width 5120, norm_expert_weight false) through the same kernels."""
    _run(STEP3, cmp_kw=dict(renormalize=False))


def test_step3_shape_large_batch_sampled():
    s = STEP3.replace(name="step3_batch", tokens=1024)      # 64 rows per expert: tiled path
    _run(s, cmp_kw=dict(renormalize=False), sample=_spread(1024, 12), edges={"heights": (128,)})


@pytest.mark.parametrize("tokens", [32, 512])
def test_dense_ffn_as_one_expert(tokens):
    """The dense SwiGLU FFN of the first layers (intermediate_size 11264) as a
    one-expert layer: top-1 of 1 expert with renormalisation gives weight 1."""
    s = W["decode"].replace(name="dense_ffn", experts=1, top_k=1, inter=11264, shared_inter=0,
                            tokens=tokens)
    _run(s, sample=_spread(tokens, 8) if tokens > 64 else None)


@pytest.mark.parametrize("name,sampled", [("page_router_decode", 0), ("step3_decode", 0),
                                          ("step3_prefill", 12), ("dense_decode", 0),
                                          ("dense_prefill", 12)])
def test_next_row_workloads(name, sampled):
    """The benchmarked workloads of the widened rows, as bench.py times them:
    the page's router configuration, Step-3's shape, the dense FFN as one
    expert (every token, or sampled ones in the large batches)."""
    s = W[name]
    _run(s, sample=_spread(s.tokens, sampled) if sampled else None)


def test_page_router_selection_only_bias():
    """The page's router configuration at the full shape with the other
    reading of the router bias: it shifts the selection scores only, the
    weights come from the unbiased sigmoid scores."""
    s = W["page_router_decode"].replace(name="page_router_select", bias_mode="select")
    _run(s)


def test_dense_ffn_int4_decode():
    """The dense FFN as one expert with INT4-g32 weights at a decode batch:
    one expert of width 11264 through the INT4 streaming kernels."""
    s = W["dense_decode"].replace(name="dense_int4", weight_dtype="int4_g32")
    _run(s)


# ----------------------------------------------------------------- SwiGLU limits

LIMITS = dict(swiglu_limit=0.5, swiglu_limit_shared=0.75)   # act on N(0, 1) projections


@pytest.mark.parametrize("act,weights", [("f32", "bf16"), ("bf16", "bf16"), ("bf16", "int4_g32"),
                                         ("f32", "int4_g32")])
def test_tiny_swiglu_limits(act, weights):
    """Limits small enough that most up and a third of the gate projections
    are clamped, different for the routed and the shared expert, through each
    streaming-kernel variant (fp32 h, bf16 h + remainder, INT4)."""
    w = 128 if weights == "int4_g32" else 64
    s = W["tiny"].replace(name=f"tiny_limits_{act}_{weights}", act_dtype=act, weight_dtype=weights,
                          inter=w, shared_inter=w, **LIMITS)
    _run(s)


@pytest.mark.parametrize("tokens,inter,shared_inter", [(512, 64, 64), (4000, 96, 160)])
def test_tiled_swiglu_limits(tokens, inter, shared_inter):
    """The LDS-tiled GEMMs (128- and 256-row tiles) with both limits."""
    s = TILED_SMALL.replace(name=f"tiled_limits_{tokens}", inter=inter, shared_inter=shared_inter,
                            tokens=tokens, **LIMITS)
    _run(s)


def test_mtp_decode_32():
    """A last layer's limits (7 routed, 16 shared) at the full shape, on
    activations wide enough that both clamps act."""
    _run(W["mtp_decode"])


def test_mtp_decode_int4():
    s = W["mtp_decode"].replace(name="mtp_int4", weight_dtype="int4_g32")
    _run(s)


def test_mtp_large_batch_sampled():
    s = W["mtp_decode"].replace(name="mtp_4096", tokens=4096)   # ~114 rows per expert: tiled
    _run(s, sample=_spread(4096, 10))


def test_swiglu_limits_change_the_output():
    """The limits of the last layers must matter on these inputs: the same
    layer without them differs by far more than the tolerance."""
    s = W["mtp_decode"]
    inp = moe_synth.make_layer(s, seed=0, device="cuda")
    outs = []
    for lim in [(7.0, 16.0), (0.0, 0.0)]:
        layer = make_layer(s, swiglu_limit=lim[0], swiglu_limit_shared=lim[1])
        layer.pack_inputs(inp)
        out, _ = run_gpu(layer, inp)
        outs.append(out.float())
    diff = (outs[0] - outs[1]).abs().max().item()
    rms = outs[1].pow(2).mean().sqrt().item()
    _say("limits on vs off", diff / rms)
    assert diff > 0.2 * rms
