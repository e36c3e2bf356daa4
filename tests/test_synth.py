"""Seeded input generator: shapes, dtypes, reproducibility (CPU)."""
import numpy as np
import torch

import moe_synth


def test_tiny_shapes_and_reproducible():
    s = moe_synth.WORKLOADS["tiny"]
    a = moe_synth.make_layer(s, seed=0)
    b = moe_synth.make_layer(s, seed=0)
    c = moe_synth.make_layer(s, seed=1)
    assert a.x.shape == (64, 256) and a.x.dtype == torch.float32
    assert a.router_w.shape == (16, 256) and a.router_w.dtype == torch.bfloat16
    assert a.w_gate.shape == (16, 64, 256) and a.w_down.shape == (16, 256, 64)
    assert a.s_gate.shape == (64, 256) and a.s_down.shape == (256, 64)
    assert a.router_bias is None
    assert torch.equal(a.w_up, b.w_up) and torch.equal(a.x, b.x)
    assert not torch.equal(a.w_up, c.w_up)
    # each expert has its own stream: experts differ from each other
    assert not torch.equal(a.w_gate[0], a.w_gate[1])
    # fan-in scaling: std of gate ~ 1/sqrt(H), of down ~ 1/sqrt(I)
    assert abs(a.w_gate.float().std().item() * 16 - 1) < 0.05
    assert abs(a.w_down.float().std().item() * 8 - 1) < 0.05


def test_int4_shape():
    s = moe_synth.WORKLOADS["tiny"].replace(weight_dtype="int4_g32", name="tiny_int4")
    a = moe_synth.make_layer(s, seed=0)
    qg, sg = a.q["gate"]
    assert qg.shape == (16, 64, 128) and qg.dtype == torch.uint8
    assert sg.shape == (16, 64, 8) and sg.dtype == torch.float16
    qd, sd = a.q["down"]
    assert qd.shape == (16, 256, 32) and sd.shape == (16, 256, 2)
    assert a.w_gate is None


def test_zipf_bias():
    b = moe_synth.zipf_bias(288)
    assert b.shape == (288,) and b.dtype == np.float32
    r = np.arange(1, 289)
    assert b[0] == b.max()
    assert np.corrcoef(b, -np.log(r))[0, 1] > 0.95   # popularity falls with rank
