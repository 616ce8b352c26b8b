"""Pins of the oracle's combine stage (orc_combine), the weighted un-permute of
lesson 10 of the expert-parallelism course ("第 10 课：专家并行 EP",
"核心概念" item 1: y is the gate-weighted sum of the chosen experts'
outputs; item 3: returned rows are multiplied by their saved gate weights and
summed), with the readings that a dropped slot adds nothing and the shared
expert adds its output with weight 1.

Two independent pins: a case worked by hand (two tokens, two heads, a dropped
slot, a token whose every slot on one head is dropped, a shared expert), and a
reassembly of the whole-layer oracle's output from expert rows computed by
dense numpy matmuls and placed at the layer's destination rows.
"""
import numpy as np
import pytest

from mixture_experts_layer_45_amd import inputs
from oracle import oracle as orc
from tests._np_ref import decode, ffn_dense, inputs_np


def _bf16_bits(v):
    """float values exactly representable in bf16 -> raw uint16 bits."""
    a = np.asarray(v, np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


# T = 2 tokens, H = 2 heads of d = 2, K = 2 slots per (token, head)
# sub-token s = 2t + g; its slots are dest_row[2s], dest_row[2s + 1]
DEST = np.array([0, 3,      # token 0, head 0: rows 0 and 3
                 1, -1,     # token 0, head 1: row 1, second slot dropped
                 -1, -1,    # token 1, head 0: both slots dropped
                 2, 4],     # token 1, head 1: rows 2 and 4
                np.int32)
W = np.array([[0.75, 0.25], [0.5, 0.5], [0.5, 0.5], [0.875, 0.125]])
YPERM = np.array([[1.0, -2.0],   # row 0
                  [4.0, 0.5],    # row 1
                  [-8.0, 2.0],   # row 2
                  [3.0, 6.0],    # row 3
                  [16.0, -4.0]])  # row 4
YSH = np.array([[0.5, 0.25, -1.0, 2.0],
                [1.0, -0.5, 0.125, 0.0]])
# worked by hand:
#   y[0, 0:2] = 0.75*(1, -2) + 0.25*(3, 6)          = (0.75 + 0.75, -1.5 + 1.5) = (1.5, 0)
#   y[0, 2:4] = 0.5*(4, 0.5)  (second slot dropped) = (2, 0.25)
#   y[1, 0:2] = nothing kept on head 0              = (0, 0)
#   y[1, 2:4] = 0.875*(-8, 2) + 0.125*(16, -4)      = (-7 + 2, 1.75 - 0.5) = (-5, 1.25)
ROUTED = np.array([[1.5, 0.0, 2.0, 0.25],
                   [0.0, 0.0, -5.0, 1.25]])
#   plus the shared expert's output, weight 1
WITH_SHARED = np.array([[2.0, 0.25, 1.0, 2.25],
                        [1.0, -0.5, -4.875, 1.25]])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_worked_by_hand(dtype):
    cfg = inputs.variant("multihead_h8_e32_top4", T=2, h=4, H=2, E=3, K=2, f=8, dtype=dtype, has_wo=0)
    enc = (lambda a: _bf16_bits(a)) if dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    y = orc.combine(cfg, DEST, W, enc(YPERM))
    assert np.array_equal(y, ROUTED)
    y = orc.combine(cfg, DEST, W, enc(YPERM), enc(YSH))
    assert np.array_equal(y, WITH_SHARED)


def test_combine_reassembles_the_layer():
    """orc_combine fed the layer's own routing and expert rows computed by
    dense numpy matmuls gives the whole-layer oracle's y (two heads, drops)."""
    H, E, d = 2, 6, 16
    cfg = inputs.variant("multihead_h8_e32_top4", T=64, h=H * d, H=H, E=E, K=2, f=24, dtype="f32", has_wo=0,
                         capacity_factor=0.75)
    inp = inputs_np(inputs.make_inputs(cfg))
    r = orc.layer_forward(cfg, inp, inp["x"])
    assert (r["dest_row"] < 0).any(), "the case should drop some assignments"
    X = decode(inp["x"])
    T, K = cfg["T"], cfg["K"]
    yp = np.zeros((r["n_kept"], d))
    idx = r["topk_idx"].ravel()
    for a, row in enumerate(r["dest_row"]):
        if row < 0:
            continue
        s = a // K
        t, g = divmod(s, H)
        e = idx[a]
        yp[row] = ffn_dense(X[t:t + 1, g * d:(g + 1) * d], inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e],
                            "swiglu")[0]
    y = orc.combine(cfg, r["dest_row"], r["topk_w"], yp.astype(np.float32))
    assert np.allclose(y, r["y"], rtol=1e-6, atol=1e-7 * np.abs(r["y"]).max())


def test_combine_reassembles_the_layer_with_shared_expert():
    """Same, one head and an always-on shared expert (sigmoid router)."""
    cfg = inputs.variant("sigmoid_top8_e256_shared", T=48, h=32, E=8, K=3, f=16, dtype="f32")
    inp = inputs_np(inputs.make_inputs(cfg))
    r = orc.layer_forward(cfg, inp, inp["x"])
    X = decode(inp["x"])
    K = cfg["K"]
    yp = np.zeros((r["n_kept"], cfg["h"]))
    idx = r["topk_idx"].ravel()
    for a, row in enumerate(r["dest_row"]):
        t, e = a // K, idx[a]
        yp[row] = ffn_dense(X[t:t + 1], inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e], "swiglu")[0]
    ysh = ffn_dense(X, inp["sh_gate"], inp["sh_up"], inp["sh_down"], "swiglu")
    y = orc.combine(cfg, r["dest_row"], r["topk_w"], yp.astype(np.float32), ysh.astype(np.float32))
    assert np.allclose(y, r["y"], rtol=1e-6, atol=1e-7 * np.abs(r["y"]).max())
    # without the shared output the difference is exactly that output (as stored)
    y0 = orc.combine(cfg, r["dest_row"], r["topk_w"], yp.astype(np.float32))
    assert np.allclose(y - y0, ysh.astype(np.float32), rtol=0, atol=1e-12)
