"""Fragment-ordered expert weights (moe_pack_weights, desc.packed = 1).

The packed forward kernels feed the MFMAs the same operands in the same order
as the row-major ones (the 4-wave kernel loads the weight fragments straight
into registers, the 64-wide kernel copies them into the same LDS layout), so
a forward pass on packed weights must give the row-major forward's output bit
for bit; the row-major forward is the one the parity tests hold to the
oracle.  The packing itself is checked against its definition in the header,
written out with numpy."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_45_amd as moe
from mixture_experts_layer_45_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()


def _reference_pack(w):
    """Piece ((nb * k/16 + s) * 64 + l) of a matrix = W[32 nb + l % 32][16 s + 8 (l / 32) + 0..7]."""
    m, n, k = w.shape
    b = w.reshape(m, n // 32, 32, k // 16, 2, 8)           # [mat, nb, l % 32, s, l / 32, j]
    return b.transpose(0, 1, 3, 4, 2, 5).reshape(m, n, k)  # [mat, nb, s, l / 32, l % 32, j]


@pytest.mark.parametrize("shape", [(3, 96, 128), (1, 32, 16), (2, 64, 4096)])
def test_pack_matches_definition(shape):
    G.log(f"[pack] shape={shape}")
    g = torch.Generator().manual_seed(11)
    w = torch.randn(shape, generator=g).to(torch.bfloat16).to(G.DEV)
    out = torch.full_like(w, 3.0)
    moe.moe_pack_weights(w, out)
    torch.cuda.synchronize()
    want = _reference_pack(w.view(torch.int16).cpu().numpy())
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), want)


def test_pack_empty_stack_is_a_no_op():
    w = torch.empty((0, 64, 64), dtype=torch.bfloat16, device=G.DEV)
    moe.moe_pack_weights(w, torch.empty_like(w))


def _ffn(cfg, counts, packed):
    H, E = cfg.get("H", 1), cfg["E"]
    dd, f = cfg["h"] // H, cfg["f"]
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(G.DEV)
    N = int(np.sum(counts))
    max_rows = N + 50
    inp = G.dev_inputs(dict(cfg, T=max(cfg["T"], 1)))
    xp = torch.randn((N, dd), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(G.DEV)
    w = moe.pack_weights(inp) if packed else inp
    d = moe.desc_from_cfg(dict(cfg, packed=int(packed)), T=(max_rows + H * cfg["K"] - 1) // (H * cfg["K"]))
    h_tmp = torch.full((max_rows, f), 5.0, dtype=torch.bfloat16, device=G.DEV)
    y_perm = torch.full((max_rows, dd), 7.0, dtype=torch.bfloat16, device=G.DEV)
    moe.moe_grouped_ffn(d, xp, offsets, max_rows, w["w_gate"], w["w_up"], w["w_down"], h_tmp, y_perm, 0,
                        moe.workspace(d, moe.MOE_WS_FFN))
    torch.cuda.synchronize()
    return h_tmp, y_perm


# the 4-wave kernel (256-row tiles, K >= 2048): gated and GELU products,
# plain products split along K in their last round; the 64-wide kernel:
# 128- and 256-row tiles, both schedule orders, K = 512 and 4096
FFN_CASES = {
    "w4_gated_then_split_plain": ("top2_e8_h4096", dict(E=2, K=1, h=2048, f=4096), [1100, 1300]),
    "w4_tail_only_plain": ("top2_e8_h4096", dict(E=2, K=1, h=1024, f=2048), [600, 700]),
    "w4_gelu": ("switch_top1_e64_zipf", dict(E=2, K=1, h=2048, f=1024), [700, 600]),
    "w4_gated_k4096_three_groups": ("top2_e8_h4096", dict(E=3, K=1, h=4096, f=512), [1100, 300, 1300]),
    "k64_paired_rows_swiglu": ("top2_e8_h4096", dict(E=6, K=1, h=512, f=1024), [130, 256, 300, 513, 0, 90]),
    "k64_paired_rows_gelu": ("switch_top1_e64_zipf", dict(E=5, K=1, h=512, f=1024), [512, 129, 0, 640, 384]),
    "k64_bm256_short_k": ("multihead_h8_e32_top4", dict(H=1, E=3, K=1, h=512, f=1024), [1030, 0, 990]),
}


@pytest.mark.parametrize("case", sorted(FFN_CASES))
def test_packed_grouped_ffn_is_bitwise_row_major(case):
    name, over, counts = FFN_CASES[case]
    cfg = inputs.variant(name, T=sum(counts), capacity_factor=0.0, **over)
    G.log(f"[packed ffn] {case} counts={counts} h={cfg['h']} f={cfg['f']}")
    h0, y0 = _ffn(cfg, counts, False)
    h1, y1 = _ffn(cfg, counts, True)
    N = int(np.sum(counts))
    assert torch.equal(h0[:N].view(torch.int16), h1[:N].view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))  # rows past the groups untouched in both


# the four bf16 layer families at small shapes with d and f multiples of 64,
# and the top-2 shape whose expert GEMMs both run on the 4-wave kernel
LAYER_CASES = {
    "top2": ("top2_e8_h4096", dict(T=600, h=512, f=320)),
    "top2_w4_both_gemms": ("top2_e8_h4096", dict(T=2048, f=2048)),
    "sigmoid_shared": ("sigmoid_top8_e256_shared", dict(T=96, h=256, f=128)),
    "sigmoid_shared_w4": ("sigmoid_top8_e256_shared", dict(T=1024, h=2048, f=128, E=16, K=4)),
    "switch_fused_unpermute": ("switch_top1_e64_zipf", dict(T=1000, h=128, f=256)),
    "multihead_wo": ("multihead_h8_e32_top4", dict(T=300, h=512, f=128)),
    "multihead_wo_w4": ("multihead_h8_e32_top4", dict(T=1024, h=2048, f=128)),
}


@pytest.mark.parametrize("case", sorted(LAYER_CASES))
def test_packed_layer_forward_is_bitwise_row_major(case):
    name, over = LAYER_CASES[case]
    cfg = inputs.variant(name, **over)
    G.log(f"[packed layer] {case} {over}")
    inp = G.dev_inputs(cfg)
    y0, aux0 = G.run_layer(cfg, inp)
    y1, aux1 = G.run_layer(dict(cfg, packed=1), moe.pack_weights(inp))
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    for k in ("topk_idx", "dest_row", "counts", "kept", "n_kept"):
        assert torch.equal(aux0[k], aux1[k]), k


@pytest.mark.parametrize("name", ["top2_e8_h4096", "sigmoid_top8_e256_shared", "switch_top1_e64_zipf",
                                  "multihead_h8_e32_top4"])
def test_packed_layer_full_size_is_bitwise_row_major(name):
    """The bf16 workloads at their full sizes, on the weights bench.py times
    (fragment order), against the same layer on row-major weights, which
    test_layer_full_size_sampled holds to the oracle."""
    cfg = inputs.CONFIGS[name]
    G.log(f"[packed layer full] {name}: generating inputs on the device")
    inp = inputs.make_inputs(cfg, G.DEV)
    y0, aux0 = G.run_layer(cfg, inp)
    packed = moe.pack_weights(inp)
    y1, aux1 = G.run_layer(dict(cfg, packed=1), packed)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    for k in ("topk_idx", "dest_row", "counts", "kept", "n_kept"):
        assert torch.equal(aux0[k], aux1[k]), k
    del inp, packed
    torch.cuda.empty_cache()
