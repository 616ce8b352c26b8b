"""Parity of the routing variants on the GPU (through the C ABI) with the CPU
oracle: group-limited top-K (lesson 10 "专家并行 EP", item 5: at most M nodes
per token), the hash gate ("HAI-LLM MoE" HashGate; "Multi-Head LatentMoE 与
Head 并行", "3. 理论基础"), the choice-major capacity queue and the evaluation
capacity factor ("HAI-LLM MoE", the (train, val) pair).

Routing from shared logits, the hash gate and the permutation must match bit
for bit; whole layers are compared within the stated bound, with the same
top-K margin exclusion as the plain router."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_45_amd as moe
from mixture_experts_layer_45_amd import inputs
from oracle import oracle as orc
from tests import _gpu as G
from tests._np_ref import to_np
from tests.test_gpu_parity import SMALL, _compare_layer, f32, i32, route_gpu

pytestmark = pytest.mark.gpu

# group-limited routers on each selection kernel: more than 64 experts (one
# wave per token), bf16 routers with at most 64 experts (one lane per token),
# fp32, several heads; the group counts leave 1 to 32 experts per group
GROUP_CASES = {
    "e256_k8_g8_m4_sigmoid": ("sigmoid_top8_e256_shared", dict(T=1500, n_groups=8, group_limit=4)),
    "e256_k8_g32_m2_sigmoid": ("sigmoid_top8_e256_shared", dict(T=700, n_groups=32, group_limit=2)),
    "e64_k6_g8_m3_softmax": ("top2_e8_h4096", dict(T=1100, E=64, K=6, n_groups=8, group_limit=3)),
    "e32_k4_g4_m2_sigmoid": ("sigmoid_top8_e256_shared", dict(T=999, E=32, K=4, n_groups=4, group_limit=2)),
    "e16_k2_g8_m1_softmax": ("top2_e8_h4096", dict(T=640, E=16, K=2, n_groups=8, group_limit=1)),
    "e96_k8_g12_m5_softmax": ("top2_e8_h4096", dict(T=500, E=96, K=8, n_groups=12, group_limit=5)),
    "f32_e16_k3_g4_m2": ("tiny_f32", dict(T=300, E=16, K=3, n_groups=4, group_limit=2)),
    "heads2_e24_k5_g6_m3": ("multihead_h8_e32_top4", dict(T=777, H=2, E=24, K=5, n_groups=6, group_limit=3)),
}


def _gcfg(case, **extra):
    base, over = GROUP_CASES[case]
    return inputs.variant(base, **dict(over, **extra))


@pytest.mark.parametrize("case", sorted(GROUP_CASES))
def test_group_limited_route_shared_logits_bit_exact(case):
    cfg = _gcfg(case)
    G.log(f"[group route shared-logits] {case}")
    lg = inputs.make_logits(cfg, "cpu", tie_every=5)
    b = inputs.make_biases(cfg, "cpu")
    bd = {k: (None if v is None else v.to(G.DEV)) for k, v in b.items()}
    g = route_gpu(cfg, logits=lg.to(G.DEV), biases=bd)
    r = orc.select(cfg, lg.numpy(), to_np(b["logit_bias"]), to_np(b["select_bias"]))
    plain = orc.select(dict(cfg, n_groups=0), lg.numpy(), to_np(b["logit_bias"]), to_np(b["select_bias"]))
    assert not np.array_equal(r["topk_idx"], plain["topk_idx"])  # the limit binds on these inputs
    assert np.array_equal(g["topk_idx"], r["topk_idx"])
    assert np.array_equal(g["counts"], r["counts"])
    assert np.abs(g["topk_w"] - r["topk_w"]).max() <= 2e-6
    assert np.allclose(g["P"], r["psum"] / cfg["T"], rtol=1e-4, atol=1e-7)


@pytest.mark.parametrize("case", ["e256_k8_g8_m4_sigmoid", "e64_k6_g8_m3_softmax", "e32_k4_g4_m2_sigmoid"])
def test_group_limited_route_logits_gemm(case):
    cfg = _gcfg(case, T=500)
    G.log(f"[group route gemm] {case}")
    inp = inputs.make_inputs(dict(cfg, f=8), "cpu")
    dv = {k: (None if v is None else v.to(G.DEV)) for k, v in inp.items()}
    g = route_gpu(cfg, x=dv["x"], w_router=dv["w_router"], biases=dv, want_logits=True)
    ref_lg = orc.logits(cfg, to_np(inp["x"]), to_np(inp["w_router"]))
    assert np.abs(g["logits"] - ref_lg).max() <= 5e-5
    r = orc.select(cfg, ref_lg, to_np(inp["logit_bias"]), to_np(inp["select_bias"]))
    ok = r["margin"] >= G.MARGIN
    assert ok.mean() > 0.5
    assert np.array_equal(g["topk_idx"][ok], r["topk_idx"][ok])
    assert np.abs(g["topk_w"][ok] - r["topk_w"][ok]).max() <= 1e-4


@pytest.mark.parametrize("E,H,T,keys", [(64, 1, 16384, None), (64, 1, 5000, "random"), (32, 8, 3001, "random"),
                                        (7, 3, 1000, None)])
def test_hash_route_bit_exact(E, H, T, keys):
    cfg = dict(inputs.CONFIGS["switch_top1_e64_zipf"], T=T, E=E, H=H, h=64 * H, gate="hash", K=1)
    G.log(f"[hash route] E={E} H={H} T={T} keys={keys}")
    k = None
    if keys == "random":
        k = np.random.default_rng(7).integers(-2 ** 31, 2 ** 31 - 1, size=T, dtype=np.int64).astype(np.int32)
        k[::13] = k[0]  # repeated keys
    d = moe.desc_from_cfg(cfg)
    S = T * H
    idx, w, counts = i32((S, 1)), f32((S, 1)), i32(H * E)
    moe.moe_route_hash(d, None if k is None else torch.from_numpy(k).to(G.DEV), idx, w, counts)
    torch.cuda.synchronize()
    r = orc.hash_select(cfg, hash_keys=k)
    assert np.array_equal(idx.cpu().numpy(), r["topk_idx"])
    assert np.all(w.cpu().numpy() == 1.0)
    assert np.array_equal(counts.cpu().numpy(), r["counts"])


@pytest.mark.parametrize("name,skew,capf", [
    ("top2_e8_h4096", 1.5, 1.0), ("top2_e8_h4096", 0.0, 0.9), ("sigmoid_top8_e256_shared", 0.8, 0.5),
    ("multihead_h8_e32_top4", 0.8, 0.7), ("tiny_f32", 1.0, 0.6),
])
def test_permute_choice_major_bit_exact(name, skew, capf):
    cfg = inputs.variant(name, queue="choice", capacity_factor=capf)
    T, H, K, E = cfg["T"], cfg.get("H", 1), cfg["K"], cfg["E"]
    G.log(f"[permute choice-major] {name} skew={skew} CF={capf}")
    idx = inputs.make_routing(cfg, "cpu", skew=skew)
    x = inputs.make_inputs(cfg, "cpu", with_weights=False)["x"].to(G.DEV)
    C = orc.capacity(cfg)
    d = moe.desc_from_cfg(cfg)
    assert moe.moe_capacity(d) == C
    A, Et, dd = T * H * K, H * E, cfg["h"] // H
    counts, kept, offsets, dest, src, nk = i32(Et), i32(Et), i32(Et + 1), i32(A), i32(A), i32(1)
    x_perm = torch.empty((A, dd), dtype=x.dtype, device=G.DEV)
    moe.moe_permute(d, idx.to(G.DEV), x, C, counts, kept, offsets, dest, src, x_perm, nk,
                    moe.workspace(d, moe.MOE_WS_PERMUTE))
    torch.cuda.synchronize()
    r = orc.permute(cfg, idx.numpy(), C)
    tok = orc.permute(dict(cfg, queue="token"), idx.numpy(), C)
    assert not np.array_equal(r["dest_row"], tok["dest_row"])  # the order matters on these inputs
    n = r["n_kept"]
    assert int(nk.item()) == n
    assert np.array_equal(kept.cpu().numpy(), r["kept"])
    assert np.array_equal(offsets.cpu().numpy(), r["offsets"])
    assert np.array_equal(dest.cpu().numpy(), r["dest_row"])
    assert np.array_equal(src.cpu().numpy()[:n], r["src_sub"])
    iv = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
    srcs = torch.from_numpy(r["src_sub"]).long().to(G.DEV)
    assert torch.equal(x_perm[:n].view(iv), x.view(T * H, dd)[srcs].view(iv))


LAYER_CASES = {
    "grouped_e256_g8_m4": ("sigmoid_top8_e256_shared", dict(n_groups=8, group_limit=4)),
    "grouped_e8_g4_m1": ("top2_e8_h4096", dict(n_groups=4, group_limit=1)),
    "hash_switch": ("switch_top1_e64_zipf", dict(gate="hash")),
    "hash_multihead": ("multihead_h8_e32_top4", dict(gate="hash", K=1)),
    "choice_queue_drops": ("top2_e8_h4096", dict(queue="choice", capacity_factor=0.8)),
    "eval_capacity": ("switch_top1_e64_zipf", dict(capacity_factor=2.0, capacity_factor_eval=0.5, eval=1)),
}


@pytest.mark.parametrize("case", sorted(LAYER_CASES))
def test_layer_routing_variants(case):
    name, over = LAYER_CASES[case]
    cfg = inputs.variant(name, **dict(SMALL[name], **over))
    G.log(f"[layer variant] {case}")
    inp = G.dev_inputs(cfg)
    y, aux = G.run_layer(cfg, inp)
    ref = orc.layer_forward(cfg, G.np_inputs(inp), to_np(inp["x"]))
    if cfg.get("gate") == "hash":
        assert np.all(ref["P"] == 0.0) and ref["l_aux"] == 0.0
    if case == "eval_capacity":
        assert ref["n_kept"] < cfg["T"]  # the evaluation factor binds
    st, n_ex = _compare_layer(cfg, y, aux, ref)
    G.log(f"   excluded={n_ex} {st}")


def test_layer_hash_keys():
    """The hash gate follows the caller's keys (e.g. vocabulary ids): tokens
    with equal keys go to the same expert."""
    cfg = inputs.variant("switch_top1_e64_zipf", **dict(SMALL["switch_top1_e64_zipf"], gate="hash"))
    G.log("[layer hash keys]")
    inp = G.dev_inputs(cfg)
    keys = np.random.default_rng(2).integers(0, 50, size=cfg["T"]).astype(np.int32)
    inp["hash_keys"] = torch.from_numpy(keys).to(G.DEV)
    y, aux = G.run_layer(cfg, inp)
    host = G.np_inputs(inp)
    ref = orc.layer_forward(cfg, host, host["x"])
    assert np.array_equal(aux["topk_idx"].cpu().numpy(), ref["topk_idx"])
    _compare_layer(cfg, y, aux, ref)


@pytest.mark.parametrize("case", ["grouped_e256_g8_m4", "hash_switch"])
def test_layer_variant_full_size_sampled(case):
    name, over = LAYER_CASES[case]
    cfg = inputs.variant(name, **over)
    T = cfg["T"]
    G.log(f"[layer variant full] {case}: generating inputs on the device")
    inp = inputs.make_inputs(cfg, G.DEV)
    y, aux = G.run_layer(cfg, inp)
    host_inp = {k: to_np(v) for k, v in inp.items()}
    rng = np.random.default_rng(4)
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 10, replace=False)])).astype(np.int32)
    G.log(f"[layer variant full] {case}: oracle on {tokens.size} sampled tokens")
    ref = orc.layer_forward(cfg, host_inp, host_inp["x"], tokens=tokens)
    st, n_ex = _compare_layer(cfg, y, aux, ref, tokens=tokens)
    G.log(f"   excluded={n_ex} of {T}; sampled {st}")
    del inp
    torch.cuda.empty_cache()
