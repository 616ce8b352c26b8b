"""Helpers of the GPU parity tests: device buffers, the stated tolerance, the
routing-margin exclusion, and calls through the C ABI binding."""
import json
import os
import sys

import numpy as np
import torch

import mixture_experts_layer_45_amd as moe
from mixture_experts_layer_45_amd import inputs
from tests import _bound as B
from tests._np_ref import to_np

DEV = "cuda"

# The stated bounds live in tests/_bound.py (bf16: half an ulp of the output,
# plus the larger of 2e-2 RMS and six standard deviations of the intermediate
# bf16 roundings, checked also against the first-order worst case, the
# aggregate RMS and the normalised mean square per row and column; fp32:
# 1e-5 RMS).  Tokens whose oracle top-K margin is under MARGIN are left out of
# end-to-end routing-sensitive comparisons.
MARGIN = 1e-3
ulp_bf16 = B.ulp_bf16


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    """device tensor -> numpy float64 (bf16 and fp32) or native ints."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float32, torch.float16):
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def assert_close(got, ref, dtype, what="", mag=None, sig=None, n_round=2, n_acc=0, rms_bound=B.RMS_BF16):
    """tests/_bound.py's check; returns its statistics."""
    return B.check(got, ref, dtype, what, mag=mag, sig=sig, n_round=n_round, n_acc=n_acc, rms_bound=rms_bound)


def n_acc(cfg):
    """longest fp32 sum of a layer evaluation: the GEMMs' reductions (d, f; h for W_o)"""
    return max(cfg["h"] // cfg.get("H", 1), cfg["f"], cfg["h"] if cfg.get("has_wo") else 0)


PARITY_RECORD = os.environ.get("MOE_PARITY_RECORD")


def record(what, stats):
    """Append one comparison's statistics to the JSON-lines file named by
    MOE_PARITY_RECORD (when set)."""
    if PARITY_RECORD:
        with open(PARITY_RECORD, "a") as fh:
            fh.write(json.dumps(dict(what=what, **stats)) + "\n")


def dev_inputs(cfg, seed=0, device=DEV):
    """Inputs generated on the host (small shapes) and copied to the device."""
    inp = inputs.make_inputs(cfg, "cpu", seed)
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def np_inputs(inp):
    return {k: to_np(v) for k, v in inp.items()}


def run_layer(cfg, inp, T=None):
    """moe_layer_forward through the C ABI; returns (y, aux) as device tensors."""
    T = cfg["T"] if T is None else T
    d = moe.desc_from_cfg(cfg, T)
    H, E, K = cfg.get("H", 1), cfg["E"], cfg["K"]
    S, Et = T * H, H * E
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    y = torch.empty((T, cfg["h"]), dtype=inputs.torch_dtype(cfg), device=DEV)
    aux = dict(topk_idx=torch.empty((S, K), **i32), topk_w=torch.empty((S, K), **f32),
               dest_row=torch.empty(S * K, **i32), counts=torch.empty(Et, **i32),
               kept=torch.empty(Et, **i32), n_kept=torch.empty(1, **i32), n_dropped=torch.empty(1, **i32),
               f=torch.empty(Et, **f32), P=torch.empty(Et, **f32), l_aux=torch.empty(1, **f32))
    ws = moe.workspace(d)
    moe.moe_layer_forward(d, inp, inp["x"], y, aux, ws)
    torch.cuda.synchronize()
    return y, aux


def excluded_tokens(cfg, ref, gpu_idx, gpu_dest):
    """Tokens left out of the end-to-end comparison: a head whose top-K margin
    (oracle key space) is under MARGIN, plus, where a capacity applies, any later
    token whose kept/dropped status differs because an excluded token earlier in
    the same expert's queue may have flipped.  Returns a bool mask over tokens."""
    T, H, K = cfg["T"], cfg.get("H", 1), cfg["K"]
    close = (ref["margin"] < MARGIN).reshape(T, H).any(1)
    excl = close.copy()
    ref_kept = (ref["dest_row"] >= 0).reshape(T, H * K)
    gpu_kept = (np.asarray(gpu_dest) >= 0).reshape(T, H * K)
    ridx = ref["topk_idx"].reshape(T, H * K)
    gidx = np.asarray(gpu_idx).reshape(T, H * K)
    cf = cfg.get("capacity_factor_eval", 0.0) if cfg.get("eval") else cfg.get("capacity_factor", 0.0)
    if cf > 0:
        touched = set()
        for t in np.nonzero(close)[0]:
            touched.update(ridx[t].tolist())
            touched.update(gidx[t].tolist())
        for t in range(T):
            if excl[t]:
                continue
            if not np.array_equal(ref_kept[t], gpu_kept[t]):
                assert set(ridx[t].tolist()) & touched, f"token {t}: drop status differs with no cause"
                excl[t] = True
    return excl
