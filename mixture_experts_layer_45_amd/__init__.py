"""MI355X-native forward pass of one sparse mixture-of-experts layer.

The layer runs as hand-written HIP kernels for gfx950 behind a C ABI
(include/moe.h, built into libmoe.so).  This module is the thin Python binding
over that ABI: each function has the name of its C entry point, turns torch
device tensors into pointers and the current torch stream into a hipStream_t,
and raises MoeError on a non-zero status.  It computes nothing itself; PyTorch
only supplies device memory and streams.
"""
import ctypes as C

from . import _ffi
from ._ffi import (INT32_MAX, MOE_BF16, MOE_F32, MOE_FFN_GEMM1, MOE_FFN_GEMM2, MOE_GELU,  # noqa: F401
                   MOE_GATE_HASH, MOE_GATE_TOPK, MOE_QUEUE_CHOICE, MOE_QUEUE_TOKEN, MOE_LOGITS_IN, MOE_LOGITS_OUT, MOE_SIGMOID, MOE_SOFTMAX, MOE_SWIGLU,
                   MOE_WS_BACKWARD, MOE_WS_FFN, MOE_WS_LAYER, MOE_WS_PERMUTE, MOE_WS_ROUTE, MoeAux, MoeDesc,
                   MoeGrads, MoeSaved, MoeWeights)

__all__ = [
    "MoeError", "MoeDesc", "desc_from_cfg", "moe_capacity", "moe_workspace_size", "moe_route",
    "moe_route_hash", "moe_permute", "moe_permute_noalloc", "moe_permute_noalloc_max_ints", "moe_grouped_ffn", "moe_grouped_ffn_rows", "moe_combine", "moe_layer_forward", "moe_version", "lib",
    "moe_max_rows", "moe_layer_forward_train", "moe_layer_backward", "SAVED_KEYS", "GRAD_KEYS",
    "alloc_saved", "alloc_grads",
    "workspace",
]


class MoeError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        name = _ffi.lib().moe_status_string(status).decode()
        super().__init__(f"{name} (status {status}): {detail}")


def lib():
    return _ffi.lib()


def moe_version():
    return lib().moe_version().decode()


def desc_from_cfg(cfg, T=None):
    """MoeDesc from a workload dict (keys as in inputs.CONFIGS)."""
    return MoeDesc(
        T=int(cfg["T"] if T is None else T), h=int(cfg["h"]), H=int(cfg.get("H", 1)),
        E=int(cfg["E"]), K=int(cfg["K"]), f=int(cfg["f"]), n_shared=int(cfg.get("n_shared", 0)),
        has_wo=int(cfg.get("has_wo", 0)), dtype=MOE_BF16 if cfg["dtype"] == "bf16" else MOE_F32,
        score=MOE_SIGMOID if cfg.get("score", "softmax") == "sigmoid" else MOE_SOFTMAX,
        act=MOE_GELU if cfg.get("act", "swiglu") == "gelu" else MOE_SWIGLU,
        capacity_factor=float(cfg.get("capacity_factor", 0.0)), aux_alpha=float(cfg.get("alpha", 0.01)),
        gate=MOE_GATE_HASH if cfg.get("gate", "topk") == "hash" else MOE_GATE_TOPK,
        n_groups=int(cfg.get("n_groups", 0)), group_limit=int(cfg.get("group_limit", 0)),
        queue=MOE_QUEUE_CHOICE if cfg.get("queue", "token") == "choice" else MOE_QUEUE_TOKEN,
        capacity_factor_eval=float(cfg.get("capacity_factor_eval", 0.0)), eval=int(cfg.get("eval", 0)),
        packed=int(cfg.get("packed", 0)),
    )


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def moe_capacity(desc):
    return int(lib().moe_capacity(C.byref(desc)))


def moe_workspace_size(desc, kind=MOE_WS_LAYER):
    n = C.c_size_t(0)
    _check(lib().moe_workspace_size(C.byref(desc), int(kind), C.byref(n)))
    return int(n.value)


def workspace(desc, kind=MOE_WS_LAYER, device="cuda"):
    """A device byte buffer of moe_workspace_size(desc, kind) bytes."""
    import torch
    return torch.empty(max(moe_workspace_size(desc, kind), 1), dtype=torch.uint8, device=device)


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def moe_route(desc, x, w_router, logit_bias, select_bias, logits, flags, topk_idx, topk_w,
              counts=None, prob_mean=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_route(C.byref(desc), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
                           _ptr(logits), int(flags), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                           _ptr(prob_mean), wp, wn, _stream(stream)))


def moe_route_hash(desc, hash_keys, topk_idx, topk_w, counts=None, stream=None):
    _check(lib().moe_route_hash(C.byref(desc), _ptr(hash_keys), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                                _stream(stream)))


def moe_permute(desc, topk_idx, x, capacity, counts, kept, offsets, dest_row, src_token, x_perm,
                n_kept=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_permute(C.byref(desc), _ptr(topk_idx), _ptr(x), int(capacity), _ptr(counts),
                             _ptr(kept), _ptr(offsets), _ptr(dest_row), _ptr(src_token), _ptr(x_perm),
                             _ptr(n_kept), wp, wn, _stream(stream)))


def moe_permute_noalloc(desc, topk_idx, x, capacity, counts, kept, offsets, dest_row, src_token, x_perm,
                        n_kept=None, stream=None):
    _check(lib().moe_permute_noalloc(C.byref(desc), _ptr(topk_idx), _ptr(x), int(capacity), _ptr(counts),
                                     _ptr(kept), _ptr(offsets), _ptr(dest_row), _ptr(src_token), _ptr(x_perm),
                                     _ptr(n_kept), _stream(stream)))


def moe_permute_noalloc_max_ints():
    return int(lib().moe_permute_noalloc_max_ints())


def moe_grouped_ffn(desc, x_perm, offsets, max_rows, w_gate, w_up, w_down, h_tmp, y_perm, flags=0,
                    ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_ffn(C.byref(desc), _ptr(x_perm), _ptr(offsets), int(max_rows), _ptr(w_gate),
                                 _ptr(w_up), _ptr(w_down), _ptr(h_tmp), _ptr(y_perm), int(flags), wp, wn,
                                 _stream(stream)))


def moe_grouped_ffn_rows(desc, x, src_token, offsets, max_rows, w_gate, w_up, w_down, h_tmp, y_perm, flags=0,
                         ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_ffn_rows(C.byref(desc), _ptr(x), _ptr(src_token), _ptr(offsets), int(max_rows),
                                      _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h_tmp), _ptr(y_perm), int(flags),
                                      wp, wn, _stream(stream)))


def moe_combine(desc, dest_row, topk_w, y_perm, y_shared, y, stream=None):
    _check(lib().moe_combine(C.byref(desc), _ptr(dest_row), _ptr(topk_w), _ptr(y_perm), _ptr(y_shared),
                             _ptr(y), _stream(stream)))


def moe_pack_weights(w, w_packed, stream=None):
    """w: bf16 device tensor [..., n_out, k] (a stack of row-major matrices);
    w_packed: a tensor of the same shape and dtype that receives them in
    fragment order."""
    if w.dim() < 2 or w.shape != w_packed.shape or w.dtype != w_packed.dtype:
        raise ValueError("w and w_packed must have one shape [..., n_out, k] and one dtype")
    import torch
    if w.dtype != torch.bfloat16:
        raise ValueError("fragment order is defined for bf16 weights")
    n_out, k = int(w.shape[-2]), int(w.shape[-1])
    n_mat = w.numel() // (n_out * k) if n_out * k else 0
    _check(lib().moe_pack_weights(_ptr(w), _ptr(w_packed), int(n_mat), n_out, k, _stream(stream)))


# the weights that desc.packed = 1 refers to
PACKED_KEYS = ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down", "w_o")


def pack_weights(weights, stream=None):
    """A copy of a weights dict with every expert weight of PACKED_KEYS in
    fragment order (new tensors; the rest shared)."""
    out = dict(weights)
    for key in PACKED_KEYS:
        w = weights.get(key)
        if w is not None:
            out[key] = w.new_empty(w.shape)
            moe_pack_weights(w, out[key], stream)
    return out


_WEIGHT_KEYS = ("w_router", "logit_bias", "select_bias", "w_gate", "w_up", "w_down", "sh_gate",
                "sh_up", "sh_down", "w_o", "hash_keys")
_AUX_KEYS = ("topk_idx", "topk_w", "dest_row", "counts", "kept", "n_kept", "n_dropped", "f", "P", "l_aux")


def moe_layer_forward(desc, weights, x, y, aux=None, ws=None, stream=None):
    """weights: dict with the keys of MoeWeights (missing = NULL); aux: dict with
    any of the keys of MoeAux (device tensors to fill) or None."""
    W = MoeWeights(**{k: _ptr(weights.get(k)) for k in _WEIGHT_KEYS})
    A = MoeAux(**{k: _ptr(aux.get(k)) for k in _AUX_KEYS}) if aux else None
    wp, wn = _ws(ws)
    _check(lib().moe_layer_forward(C.byref(desc), C.byref(W), _ptr(x), _ptr(y),
                                   C.byref(A) if A is not None else None, wp, wn, _stream(stream)))


SAVED_KEYS = tuple(n for n, _ in MoeSaved._fields_)
GRAD_KEYS = tuple(n for n, _ in MoeGrads._fields_)


def moe_max_rows(desc):
    return int(lib().moe_max_rows(C.byref(desc)))


def moe_layer_forward_train(desc, weights, x, y, saved, aux=None, ws=None, stream=None):
    """moe_layer_forward that also fills `saved` (dict with the keys of MoeSaved,
    device tensors; see include/moe.h for their shapes)."""
    W = MoeWeights(**{k: _ptr(weights.get(k)) for k in _WEIGHT_KEYS})
    A = MoeAux(**{k: _ptr(aux.get(k)) for k in _AUX_KEYS}) if aux else None
    Sv = MoeSaved(**{k: _ptr(saved.get(k)) for k in SAVED_KEYS})
    wp, wn = _ws(ws)
    _check(lib().moe_layer_forward_train(C.byref(desc), C.byref(W), _ptr(x), _ptr(y),
                                         C.byref(A) if A is not None else None, C.byref(Sv), wp, wn,
                                         _stream(stream)))


def moe_layer_backward(desc, weights, x, dy, saved, grads, aux_weight=1.0, ws=None, stream=None):
    """Gradients of sum(dy * y) + aux_weight * L_aux into `grads` (dict with the
    keys of MoeGrads: dx and one buffer per weight the layer has)."""
    W = MoeWeights(**{k: _ptr(weights.get(k)) for k in _WEIGHT_KEYS})
    Sv = MoeSaved(**{k: _ptr(saved.get(k)) for k in SAVED_KEYS})
    Gr = MoeGrads(**{k: _ptr(grads.get(k)) for k in GRAD_KEYS})
    wp, wn = _ws(ws)
    _check(lib().moe_layer_backward(C.byref(desc), C.byref(W), _ptr(x), _ptr(dy), C.byref(Sv), float(aux_weight),
                                    C.byref(Gr), wp, wn, _stream(stream)))


def alloc_saved(desc, device="cuda"):
    """Device buffers for the state of a training forward (the fields of
    MoeSaved that this layer uses), shaped as include/moe.h states."""
    import torch
    T, H, E, K, f, h = desc.T, desc.H, desc.E, desc.K, desc.f, desc.h
    d, S, Et, R = h // H, T * H, H * E, max(moe_max_rows(desc), 1)
    na = 1 if desc.act == MOE_GELU else 2
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    bf = dict(dtype=torch.bfloat16, device=device)
    sv = dict(topk_idx=torch.empty((S, K), **i32), topk_w=torch.empty((S, K), **f32),
              dest_row=torch.empty(S * K, **i32), src_token=torch.empty(S * K, **i32),
              offsets=torch.empty(Et + 1, **i32), counts=torch.empty(Et, **i32),
              logits=torch.empty((S, E), **f32), act_grad=torch.empty((R, na * f), **bf),
              h=torch.empty((R, f), **bf), y_perm=torch.empty((R, d), **bf))
    if desc.n_shared:
        sv.update(sh_act_grad=torch.empty((T, na * f), **bf), sh_h=torch.empty((T, f), **bf))
    if desc.has_wo:
        sv["y_cat"] = torch.empty((T, h), **bf)
    return sv


def alloc_grads(desc, weights, x):
    """Gradient buffers for moe_layer_backward: dx like x, and one like each
    weight the layer has (the router's only with the top-K gate)."""
    import torch
    gr = {"dx": torch.empty_like(x)}
    for k in ("w_router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down", "w_o"):
        if weights.get(k) is not None and not (k == "w_router" and desc.gate == MOE_GATE_HASH):
            gr[k] = torch.empty_like(weights[k])
    return gr
