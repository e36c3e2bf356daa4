"""Pins the oracle to facts other than itself (CPU only).

Each check_* function is a pin; test_mutations_are_caught plants plausible
mistakes in the oracle (monkeypatched, on the CPU) and asserts that at least
one pin fails for each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe_oracle
import moe_synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _random_layer(rng, t=5, h=8, e=6, i=4, i_s=3):
    x = rng.standard_normal((t, h))
    wr = rng.standard_normal((e, h)) / math.sqrt(h)
    ex = [(rng.standard_normal((i, h)), rng.standard_normal((i, h)), rng.standard_normal((h, i)))
          for _ in range(e)]
    sh = (rng.standard_normal((i_s, h)), rng.standard_normal((i_s, h)), rng.standard_normal((h, i_s)))
    return x, wr, ex, sh


# ----------------------------------------------------------------------------- pins

def check_hand_case():
    """Hand-evaluated 2-expert layer (closed forms in tests/golden)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_two_expert.json")))
    ex = [(np.array(d["gate"]), np.array(d["up"]), np.array(d["down"])) for d in g["experts"]]
    sh = (np.array(g["shared"]["gate"]), np.array(g["shared"]["up"]), np.array(g["shared"]["down"]))
    s1 = 1.0 / (1.0 + math.exp(-1.0))          # silu(1) / 1 = sigmoid(1) = e/(1+e)
    closed = {"k2": [s1 + s1 * 2 * s1, s1 - (1 - s1) * (1 - s1)], "k1": [s1 + 2 * s1, s1]}
    for key, k in (("k2", 2), ("k1", 1)):
        y, idx, w, _ = oracle.forward(np.array(g["x"]), np.array(g["router_w"]), None,
                                      lambda e: ex[e], sh, k)
        exp = g["expected"][key]
        assert idx.tolist() == exp["idx"]
        np.testing.assert_allclose(w, exp["w"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(y, exp["y"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[0], closed[key], rtol=0, atol=1e-12)


def check_topk_bruteforce():
    """Selection = first k of a full sort by (-score, expert index)."""
    rng = _rng(1)
    for trial in range(60):
        t, e = rng.integers(1, 9), rng.integers(2, 20)
        k = int(rng.integers(1, e + 1))
        s = rng.standard_normal((t, e)).astype(np.float32)
        if trial % 3 == 0:      # forced exact ties: duplicate some columns
            src = rng.integers(0, e, size=e // 2)
            dst = rng.integers(0, e, size=e // 2)
            s[:, dst] = s[:, src]
        if trial % 5 == 0:      # quantised scores: many ties
            s = np.round(s * 2).astype(np.float32)
        got = oracle.select_topk(s, k)
        for r in range(t):
            order = np.lexsort((np.arange(e), -s[r].astype(np.float64)))
            assert got[r].tolist() == order[:k].tolist()


def check_weights_closed_form():
    rng = _rng(2)
    for _ in range(30):
        t, e = 4, int(rng.integers(2, 17))
        k = int(rng.integers(1, e + 1))
        l = (rng.standard_normal((t, e)) * 3).astype(np.float32)
        idx = oracle.select_topk(l, k)
        w = oracle.gate_weights(l, idx, "softmax", True, 1.0)
        sel = np.take_along_axis(l.astype(np.float64), idx, axis=1)
        np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.all(np.diff(w, axis=1) <= 1e-15)         # descending by rank
        w_raw = oracle.gate_weights(l, idx, "softmax", False, 1.0)
        full = scipy.special.softmax(l.astype(np.float64), axis=1)
        np.testing.assert_allclose(w_raw, np.take_along_axis(full, idx, axis=1), rtol=1e-12)
        # k = E: the renormalised weights are the full softmax
        idx_all = oracle.select_topk(l, e)
        w_all = oracle.gate_weights(l, idx_all, "softmax", True, 1.0)
        np.testing.assert_allclose(w_all, np.take_along_axis(full, idx_all, axis=1), rtol=1e-12)
        # k = 1: the single weight is 1
        np.testing.assert_allclose(oracle.gate_weights(l, idx[:, :1], "softmax", True, 1.0), 1.0)
        # sigmoid scoring, renormalised and scaled by 3
        ws = oracle.gate_weights(l, idx, "sigmoid", True, 3.0)
        sg = scipy.special.expit(sel)
        np.testing.assert_allclose(ws, 3.0 * sg / sg.sum(axis=1, keepdims=True), rtol=1e-12)


def _dense_swiglu_torch(x, wg, wu, wd):
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T) @ wd.T).numpy()


def check_identical_experts_dense():
    """All experts equal => routed part is one dense SwiGLU FFN (weights sum to 1)."""
    rng = _rng(3)
    x, wr, ex, sh = _random_layer(rng, t=7, h=12, e=9, i=5, i_s=4)
    same = ex[0]
    for k in (1, 3, 9):
        y, *_ = oracle.forward(x, wr, None, lambda e: same, sh, k)
        ref = _dense_swiglu_torch(x, *same) + _dense_swiglu_torch(x, *sh)
        np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)
    y0, *_ = oracle.forward(x, wr, None, lambda e: same, None, 2)
    np.testing.assert_allclose(y0, _dense_swiglu_torch(x, *same), rtol=1e-10, atol=1e-12)


def check_single_expert_contribution():
    """k = 1 and a router that prefers one expert: y = shared + that expert's FFN,
    evaluated by torch's library ops (catches swapped or transposed operands)."""
    rng = _rng(4)
    x, _, ex, sh = _random_layer(rng, t=3, h=6, e=4, i=5, i_s=2)
    for target in range(4):
        wr = np.zeros((4, 6))
        wr[target] = x.sum(axis=0) * 0 + 1.0     # logit of target = sum(x); others 0
        xx = np.abs(x) + 0.1                     # make sum(x) > 0 so target wins
        y, idx, w, _ = oracle.forward(xx, wr, None, lambda e: ex[e], sh, 1)
        assert (idx[:, 0] == target).all()
        ref = _dense_swiglu_torch(xx, *ex[target]) + _dense_swiglu_torch(xx, *sh)
        np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def check_relabel_and_token_independence():
    rng = _rng(5)
    x, wr, ex, sh = _random_layer(rng, t=9, h=10, e=7, i=3, i_s=2)
    y, idx, w, _ = oracle.forward(x, wr, None, lambda e: ex[e], sh, 3)
    perm = rng.permutation(7)                    # new expert e' = perm[e]
    wr2 = np.empty_like(wr)
    wr2[perm] = wr
    ex2 = [None] * 7
    for e in range(7):
        ex2[perm[e]] = ex[e]
    y2, idx2, w2, _ = oracle.forward(x, wr2, None, lambda e: ex2[e], sh, 3)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)
    assert (np.sort(idx2, axis=1) == np.sort(perm[idx], axis=1)).all()
    sub = [6, 1, 4]
    y3, *_ = oracle.forward(x[sub], wr, None, lambda e: ex[e], sh, 3)
    np.testing.assert_allclose(y3, y[sub], rtol=1e-12, atol=1e-14)


def check_router_bias_and_fp32_logits():
    rng = _rng(6)
    x = rng.standard_normal((5, 16))
    wr = rng.standard_normal((8, 16))
    b = rng.standard_normal(8).astype(np.float32)
    l = oracle.router_logits(x, wr, b)
    assert l.dtype == np.float32
    exact = [[math.fsum([x[t, h] * wr[e, h] for h in range(16)] + [float(b[e])]) for e in range(8)]
             for t in range(5)]
    np.testing.assert_array_equal(l, np.array(exact).astype(np.float32))
    # a large bias on one expert forces it into every token's selection
    b2 = np.zeros(8, np.float32)
    b2[5] = 100.0
    idx, w, _ = oracle.route(x, wr, b2, 2)
    assert (idx[:, 0] == 5).all()
    # selection-only bias: same selection, weights from unbiased logits
    idx_s, w_s, l_s = oracle.route(x, wr, b2, 2, bias_mode="select")
    assert (idx_s[:, 0] == 5).all()
    l_unb = oracle.router_logits(x, wr, None)
    sel = np.take_along_axis(l_unb.astype(np.float64), idx_s, axis=1)
    np.testing.assert_allclose(w_s, scipy.special.softmax(sel, axis=1), rtol=1e-12)


def check_dispatch():
    rng = _rng(7)
    for _ in range(20):
        t, e = int(rng.integers(1, 40)), int(rng.integers(2, 12))
        k = int(rng.integers(1, e + 1))
        idx = np.stack([rng.permutation(e)[:k] for _ in range(t)])
        counts, offsets, perm, inv = oracle.dispatch(idx, e)
        keys = sorted((int(idx[p // k, p % k]), p // k, p) for p in range(t * k))
        assert perm.tolist() == [p for _, _, p in keys]
        assert counts.sum() == t * k and offsets[-1] == t * k
        assert (np.diff(offsets) == counts).all()
        assert (inv[perm] == np.arange(t * k)).all()
        for r in range(t * k):
            p = perm[r]
            assert offsets[idx[p // k, p % k]] <= r < offsets[idx[p // k, p % k] + 1]


def check_int4():
    rng = _rng(8)
    w = torch.from_numpy(rng.standard_normal((6, 96)).astype(np.float32)).to(torch.bfloat16)
    w[0, :32] = 0.0                                     # an all-zero group: s = 0, q = 0
    packed, scales = moe_synth.quantize_int4_g32(w)
    deq = oracle.dequant_int4(packed.numpy(), scales.numpy())
    wf = w.double().numpy()
    s = np.repeat(scales.double().numpy(), 32, axis=1)
    q = moe_synth.unpack_int4(packed).numpy().astype(np.float64)
    np.testing.assert_array_equal(deq, s * q)           # exact dequantisation
    # byte layout: element k in byte k//2, low nibble for even k, offset binary
    pk = packed.numpy()
    for n in range(6):
        for k in range(96):
            nib = (pk[n, k // 2] >> (4 * (k % 2))) & 0xF
            assert deq[n, k] == float(scales[n, k // 32]) * (int(nib) - 8)
    # nearest code for unclipped elements (brute force over all 16 codes)
    codes = np.arange(-8, 8)
    for n in range(6):
        for k in range(96):
            sc = s[n, k]
            if sc == 0:
                assert q[n, k] == 0
                continue
            best = np.min(np.abs(wf[n, k] - sc * codes))
            assert abs(wf[n, k] - sc * q[n, k]) <= best + 1e-12
            if abs(wf[n, k] / sc) <= 7.0:
                assert abs(wf[n, k] - sc * q[n, k]) <= sc / 2 + 1e-12
    assert np.array_equal(moe_synth.unpack_int4(packed).numpy(), q.astype(np.int8))


def check_parameter_count():
    """The page shapes reproduce 196B total / 11B active (3 matrices per expert)."""
    H, E, K, I, Is, V = 4096, 288, 8, 1280, 1280, 128896
    moe_layers, dense_layers, layers, dense_i = 42, 3, 45, 11264
    q_heads, kv_groups, hd = 64, 8, 128
    attn = H * q_heads * hd * 2 + H * kv_groups * hd * 2
    expert = 3 * H * I
    total = (moe_layers * (E * expert + 3 * H * Is + E * H) + dense_layers * 3 * H * dense_i
             + layers * attn + 2 * V * H)
    active = (moe_layers * (K * expert + 3 * H * Is + E * H) + dense_layers * 3 * H * dense_i
              + layers * attn + 2 * V * H)
    assert abs(total / 1e9 - 196) < 1.0
    assert abs(active / 1e9 - 11) < 0.5


def check_swiglu_limit():
    """SwiGLU limits by hand: gate clamped from above only, up on both sides;
    routed and shared experts each take their own limit."""
    silu = lambda z: z / (1.0 + math.exp(-z))
    x = np.array([[1.0]])
    wd = np.array([[1.0]])
    # gate 10 > 7 -> 7, up -20 < -7 -> -7
    y = oracle.swiglu_ffn(x, np.array([[10.0]]), np.array([[-20.0]]), wd, limit=7.0)
    assert y[0, 0] == pytest.approx(silu(7.0) * -7.0, rel=1e-14)
    # gate -10 is not clamped from below; up 5 inside the limit
    y = oracle.swiglu_ffn(x, np.array([[-10.0]]), np.array([[5.0]]), wd, limit=7.0)
    assert y[0, 0] == pytest.approx(silu(-10.0) * 5.0, rel=1e-14)
    # no limit: untouched
    y = oracle.swiglu_ffn(x, np.array([[10.0]]), np.array([[-20.0]]), wd)
    assert y[0, 0] == pytest.approx(silu(10.0) * -20.0, rel=1e-14)
    # whole layer, one token, one expert (weight 1): routed limit 7, shared 16,
    # both projections at 10 -> routed clamped to (7, 7), shared untouched
    ex = (np.array([[10.0]]), np.array([[10.0]]), np.array([[1.0]]))
    y, idx, w, _ = oracle.forward(x, np.array([[1.0]]), None, lambda e: ex, ex, 1,
                                  swiglu_limit=7.0, swiglu_limit_shared=16.0)
    assert w[0, 0] == 1.0
    assert y[0, 0] == pytest.approx(silu(10.0) * 10.0 + silu(7.0) * 7.0, rel=1e-14)


def check_topk_gap_bruteforce():
    """topk_gap = (k-th - (k+1)-th) largest selection score per token, by a
    full sort written out per row; +inf when k equals the number of experts;
    exact ties give 0; the gap is the one at the selection boundary (a brute
    force over every expert of the selected and the rejected set)."""
    rng = _rng(9)
    for trial in range(60):
        t, e = int(rng.integers(1, 7)), int(rng.integers(2, 24))
        k = int(rng.integers(1, e + 1))
        s = rng.standard_normal((t, e)).astype(np.float32)
        if trial % 3 == 0:
            s = np.round(s * 2).astype(np.float32)       # many exact ties
        gap = oracle.topk_gap(s, k)
        for r in range(t):
            vals = sorted((float(v) for v in s[r]), reverse=True)
            want = math.inf if k == e else vals[k - 1] - vals[k]
            assert gap[r] == want, (trial, r, gap[r], want)
            if k < e:   # smallest selected minus largest rejected score
                sel = oracle.select_topk(s[r:r + 1], k)[0]
                rest = np.setdiff1d(np.arange(e), sel)
                assert gap[r] == float(s[r, sel].min()) - float(s[r, rest].max())
    # an exact tie at the boundary (experts 2 and 3 for k = 2): gap 0, and the
    # selection is still defined (the lower index); one past it (k = 3): gap 1
    s = np.array([[3.0, 1.0, 2.0, 2.0, 0.5]], np.float32)
    assert oracle.topk_gap(s, 2)[0] == 0.0 and oracle.topk_gap(s, 3)[0] == 1.0
    assert oracle.select_topk(s, 2)[0].tolist() == [0, 2]
    assert oracle.topk_gap(s, 1)[0] == 1.0 and oracle.topk_gap(s, 4)[0] == 0.5
    assert oracle.topk_gap(s, 5)[0] == math.inf


PINS = [check_hand_case, check_topk_bruteforce, check_topk_gap_bruteforce,
        check_weights_closed_form,
        check_identical_experts_dense, check_single_expert_contribution,
        check_relabel_and_token_independence, check_router_bias_and_fp32_logits,
        check_dispatch, check_int4, check_parameter_count, check_swiglu_limit]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------- planted mistakes

def _mut_swap_gate_up(m):
    orig = m.swiglu_ffn
    m.swiglu_ffn = lambda x, g, u, d, limit=0.0: orig(x, u, g, d, limit)


def _mut_no_renorm(m):
    orig = m.gate_weights
    m.gate_weights = lambda l, idx, score="softmax", renormalize=True, s=1.0: orig(l, idx, score, False, s)


def _mut_tie_high_index(m):
    def sel(scores, k):
        s = np.asarray(scores, np.float64)[:, ::-1]
        return (s.shape[1] - 1) - moe_oracle.select_topk.__wrapped__(s, k)
    sel.__wrapped__ = moe_oracle.select_topk
    m.select_topk = sel


def _mut_silu_sign(m):
    m.silu = lambda z: z / (1.0 + np.exp(z))


def _mut_down_transposed(m):
    def ffn(x, g, u, d, limit=0.0):
        x = np.asarray(x, np.float64)
        h = m.silu(x @ g.T) * (x @ u.T)
        return h @ np.asarray(d).reshape(d.shape[1], d.shape[0])
    m.swiglu_ffn = ffn


def _mut_softmax_no_max_shift_wrong(m):
    orig = m.gate_weights
    m.gate_weights = lambda l, idx, score="softmax", renormalize=True, s=1.0: orig(l * 0.5, idx, score, renormalize, s)


def _mut_shared_weighted(m):
    orig = m.forward

    def fwd(x, wr, b, experts, shared, k, *a, **kw):
        y, idx, w, l = orig(x, wr, b, experts, None, k, *a, **kw)
        if shared is not None:
            y = y + w[:, :1] * m.swiglu_ffn(np.asarray(x, np.float64), *shared)
        return y, idx, w, l
    m.forward = fwd


def _mut_int4_high_nibble_first(m):
    def deq(packed, scales):
        packed = np.asarray(packed, np.uint8)
        swapped = ((packed & 0xF) << 4) | (packed >> 4)
        return moe_oracle.dequant_int4.__wrapped__(swapped, scales)
    deq.__wrapped__ = moe_oracle.dequant_int4
    m.dequant_int4 = deq


def _mut_dispatch_unstable(m):
    orig = m.dispatch

    def disp(idx, e):
        counts, offsets, perm, inv = orig(idx, e)
        for ee in range(e):                   # reverse the order inside each group
            perm[offsets[ee]:offsets[ee + 1]] = perm[offsets[ee]:offsets[ee + 1]][::-1].copy()
        inv[perm] = np.arange(perm.shape[0])
        return counts, offsets, perm, inv
    m.dispatch = disp


def _mut_limit_gate_only(m):
    def ffn(x, g, u, d, limit=0.0):
        x = np.asarray(x, np.float64)
        gg = x @ np.asarray(g, np.float64).T
        if limit > 0:
            gg = np.minimum(gg, limit)
        return (m.silu(gg) * (x @ np.asarray(u, np.float64).T)) @ np.asarray(d, np.float64).T
    m.swiglu_ffn = ffn


def _mut_limit_shared_uses_routed(m):
    orig = m.forward

    def fwd(*a, swiglu_limit=0.0, swiglu_limit_shared=0.0, **kw):
        return orig(*a, swiglu_limit=swiglu_limit, swiglu_limit_shared=swiglu_limit, **kw)
    m.forward = fwd


def _mut_gap_off_by_one(m):
    def gap(scores32, k):
        s = np.sort(np.asarray(scores32, np.float64), axis=1)[:, ::-1]
        if k + 1 >= s.shape[1]:
            return np.full(s.shape[0], np.inf)
        return s[:, k] - s[:, k + 1]          # the (k+1)-th and (k+2)-th scores
    m.topk_gap = gap


def _mut_gap_ascending(m):
    def gap(scores32, k):
        s = np.sort(np.asarray(scores32, np.float64), axis=1)
        if k >= s.shape[1]:
            return np.full(s.shape[0], np.inf)
        return s[:, k] - s[:, k - 1]          # gap among the k smallest
    m.topk_gap = gap


MUTATIONS = [_mut_swap_gate_up, _mut_no_renorm, _mut_tie_high_index, _mut_silu_sign,
             _mut_down_transposed, _mut_softmax_no_max_shift_wrong, _mut_shared_weighted,
             _mut_int4_high_nibble_first, _mut_dispatch_unstable, _mut_limit_gate_only,
             _mut_limit_shared_uses_routed, _mut_gap_off_by_one, _mut_gap_ascending]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_mutations_are_caught(mutate, monkeypatch):
    import oracle as pkg
    saved = {n: getattr(moe_oracle, n) for n in dir(moe_oracle) if not n.startswith("_")}
    mutate(moe_oracle)
    for n in saved:                               # route the package names to the mutated ones
        monkeypatch.setattr(pkg, n, getattr(moe_oracle, n), raising=False)
    failed = []
    try:
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    finally:
        for n, v in saved.items():
            setattr(moe_oracle, n, v)
    assert failed, f"no pin caught {mutate.__name__}"
