"""Python face of the CPU oracle for the forward pass of one sparse MoE layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline may import this module; the product path (the HIP library and its
binding) never does.  The arithmetic lives in moe_oracle.c (plain C, fp64);
this module only marshals numpy arrays, plus the pure-Python load-imbalance
report of the worked example in lesson 10 of the expert-parallelism course
("第 10 课：专家并行 EP", learn.payai.win), section "具体演示与数值推演" and its
code exercise (expert-to-rank map, per-rank load, max/mean imbalance, routed
volume).

Parity unpinned (no page fixes them; checked through invariants only): P of
the sigmoid router and L_aux of the multi-head layer (see moe_oracle.c).

Arrays in bf16 are passed as numpy uint16 holding the raw bf16 bits.
A layer configuration is a plain dict with keys
  T, h, H, E, K, f, n_shared, has_wo, dtype ('f32'|'bf16'),
  score ('softmax'|'sigmoid'), act ('swiglu'|'gelu'), capacity_factor, alpha,
and optionally the routing variants
  gate ('topk'|'hash'), n_groups, group_limit, queue ('token'|'choice'),
  capacity_factor_eval, eval (0|1).
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB_PATH names another build of the oracle (the ASan/UBSan build
# of the CPU sanitizer test); by default the in-tree liboracle.so
LIB_PATH = os.environ.get("MOE_ORACLE_LIB_PATH") or os.path.join(HERE, "liboracle.so")


class OrcDesc(C.Structure):
    _fields_ = [
        ("T", C.c_int32), ("h", C.c_int32), ("H", C.c_int32), ("E", C.c_int32),
        ("K", C.c_int32), ("f", C.c_int32), ("n_shared", C.c_int32),
        ("has_wo", C.c_int32), ("dtype", C.c_int32), ("score", C.c_int32),
        ("act", C.c_int32), ("capacity_factor", C.c_float), ("alpha", C.c_float),
        ("gate", C.c_int32), ("n_groups", C.c_int32), ("group_limit", C.c_int32),
        ("queue", C.c_int32), ("capacity_factor_eval", C.c_float), ("eval", C.c_int32),
    ]


class OrcWeights(C.Structure):
    _fields_ = [
        ("w_router", C.c_void_p), ("logit_bias", C.c_void_p), ("select_bias", C.c_void_p),
        ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
        ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
        ("w_o", C.c_void_p), ("hash_keys", C.c_void_p),
    ]


class OrcGrads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up",
                                          "dsh_down", "dw_o", "dlogits", "dtopk_w")]


class OrcAux(C.Structure):
    _fields_ = [
        ("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("margin", C.c_void_p),
        ("counts", C.c_void_p), ("kept", C.c_void_p), ("offsets", C.c_void_p),
        ("dest_row", C.c_void_p), ("src_sub", C.c_void_p), ("n_kept", C.c_void_p),
        ("f", C.c_void_p), ("P", C.c_void_p), ("l_aux", C.c_void_p), ("logits", C.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            import importlib.util
            spec = importlib.util.spec_from_file_location("_oracle_build", os.path.join(HERE, "build.py"))
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.build()
        _lib = C.CDLL(LIB_PATH)
        _lib.orc_exp_spec.restype = C.c_float
        _lib.orc_exp_spec.argtypes = [C.c_float]
        _lib.orc_sigmoid_spec.restype = C.c_float
        _lib.orc_sigmoid_spec.argtypes = [C.c_float]
        _lib.orc_sigmoid_key.restype = C.c_float
        _lib.orc_sigmoid_key.argtypes = [C.c_float, C.c_float]
        _lib.orc_capacity.restype = C.c_int64
        _lib.orc_capacity.argtypes = [C.POINTER(OrcDesc)]
        _lib.orc_logits.restype = None
        _lib.orc_logits.argtypes = [C.POINTER(OrcDesc), C.c_void_p, C.c_void_p, C.c_void_p]
        _lib.orc_select.restype = None
        _lib.orc_select.argtypes = [C.POINTER(OrcDesc)] + [C.c_void_p] * 8
        _lib.orc_fmix32.restype = C.c_uint32
        _lib.orc_fmix32.argtypes = [C.c_uint32]
        _lib.orc_hash_select.restype = None
        _lib.orc_hash_select.argtypes = [C.POINTER(OrcDesc)] + [C.c_void_p] * 4
        _lib.orc_permute.restype = None
        _lib.orc_permute.argtypes = [C.POINTER(OrcDesc), C.c_void_p, C.c_int64] + [C.c_void_p] * 6
        _lib.orc_expert_ffn.restype = None
        _lib.orc_expert_ffn.argtypes = [C.c_int32] * 4 + [C.c_void_p] * 7
        _lib.orc_expert_ffn_rows.restype = None
        _lib.orc_expert_ffn_rows.argtypes = [C.c_int32] * 4 + [C.c_void_p] * 3 + [C.c_int64] + [C.c_void_p] * 4
        _lib.orc_combine.restype = None
        _lib.orc_combine.argtypes = [C.POINTER(OrcDesc)] + [C.c_void_p] * 5
        _lib.orc_layer_forward.restype = C.c_int
        _lib.orc_layer_forward.argtypes = [C.POINTER(OrcDesc), C.POINTER(OrcWeights), C.c_void_p,
                                           C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.POINTER(OrcAux)]
        _lib.orc_layer_backward.restype = C.c_int
        _lib.orc_layer_backward.argtypes = [C.POINTER(OrcDesc), C.POINTER(OrcWeights), C.c_void_p, C.c_void_p,
                                            C.c_double, C.c_int, C.POINTER(OrcGrads)]
        _lib.orc_num_threads.restype = C.c_int
        _lib.orc_num_threads.argtypes = []
        _lib.orc_set_num_threads.restype = None
        _lib.orc_set_num_threads.argtypes = [C.c_int]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def desc(cfg, T=None):
    return OrcDesc(
        T=int(cfg["T"] if T is None else T), h=int(cfg["h"]), H=int(cfg.get("H", 1)),
        E=int(cfg["E"]), K=int(cfg["K"]), f=int(cfg["f"]),
        n_shared=int(cfg.get("n_shared", 0)), has_wo=int(cfg.get("has_wo", 0)),
        dtype=1 if cfg["dtype"] == "bf16" else 0,
        score=1 if cfg.get("score", "softmax") == "sigmoid" else 0,
        act=1 if cfg.get("act", "swiglu") == "gelu" else 0,
        capacity_factor=float(cfg.get("capacity_factor", 0.0)),
        alpha=float(cfg.get("alpha", 0.01)),
        gate=1 if cfg.get("gate", "topk") == "hash" else 0,
        n_groups=int(cfg.get("n_groups", 0)), group_limit=int(cfg.get("group_limit", 0)),
        queue=1 if cfg.get("queue", "token") == "choice" else 0,
        capacity_factor_eval=float(cfg.get("capacity_factor_eval", 0.0)), eval=int(cfg.get("eval", 0)),
    )


def _elem(cfg):
    return np.uint16 if cfg["dtype"] == "bf16" else np.float32


def _chk(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


# ------------------------------------------------------------------ scalars
def exp_spec(x):
    """fp32 exp of the sigmoid routing key (Cody-Waite reduction + Taylor)."""
    x = np.asarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_exp_spec(float(v)) for v in x], dtype=np.float32)


def sigmoid_spec(x):
    x = np.asarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_sigmoid_spec(float(v)) for v in x], dtype=np.float32)


def sigmoid_key(l, b):
    return np.float32(lib().orc_sigmoid_key(float(l), float(b)))


def capacity(cfg, T=None):
    """C = CF*K*T/E rounded up (guarded); None means no limit."""
    c = lib().orc_capacity(C.byref(desc(cfg, T)))
    return None if c < 0 else int(c)


# ------------------------------------------------------------------ stages
def logits(cfg, x, w_router, T=None):
    d = desc(cfg, T)
    S = d.T * d.H
    x = _chk(x, _elem(cfg))
    w_router = _chk(w_router, _elem(cfg))
    out = np.empty((S, d.E), dtype=np.float32)
    lib().orc_logits(C.byref(d), _p(x), _p(w_router), _p(out))
    return out


def select(cfg, logits_, logit_bias=None, select_bias=None, T=None):
    d = desc(cfg, T)
    S = d.T * d.H
    lg = _chk(logits_, np.float32)
    assert lg.size == S * d.E
    lb = None if logit_bias is None else _chk(logit_bias, np.float32)
    sb = None if select_bias is None else _chk(select_bias, np.float32)
    idx = np.empty((S, d.K), dtype=np.int32)
    w = np.empty((S, d.K), dtype=np.float64)
    margin = np.empty(S, dtype=np.float64)
    counts = np.zeros(d.H * d.E, dtype=np.int32)
    psum = np.zeros(d.H * d.E, dtype=np.float64)
    lib().orc_select(C.byref(d), _p(lg), _p(lb), _p(sb), _p(idx), _p(w), _p(margin),
                     _p(counts), _p(psum))
    return dict(topk_idx=idx, topk_w=w, margin=margin, counts=counts, psum=psum)


def fmix32(v):
    """MurmurHash3's 32-bit finaliser, as the hash gate uses it."""
    return int(lib().orc_fmix32(int(v) & 0xFFFFFFFF))


def hash_select(cfg, hash_keys=None, T=None):
    """Hash gate (K = 1): expert ids [T*H, 1], weights (all 1) and counts."""
    d = desc(cfg, T)
    S = d.T * d.H
    keys = None if hash_keys is None else _chk(np.asarray(hash_keys, dtype=np.int32), np.int32)
    assert keys is None or keys.size == d.T
    idx = np.empty((S, 1), dtype=np.int32)
    w = np.empty((S, 1), dtype=np.float64)
    counts = np.zeros(d.H * d.E, dtype=np.int32)
    lib().orc_hash_select(C.byref(d), _p(keys), _p(idx), _p(w), _p(counts))
    return dict(topk_idx=idx, topk_w=w, counts=counts)


def permute(cfg, topk_idx, cap, T=None):
    """cap: int capacity or None for no limit."""
    d = desc(cfg, T)
    Et = d.H * d.E
    A = d.T * d.H * d.K
    idx = _chk(topk_idx, np.int32).ravel()
    assert idx.size == A
    counts = np.zeros(Et, dtype=np.int32)
    kept = np.zeros(Et, dtype=np.int32)
    offsets = np.zeros(Et + 1, dtype=np.int32)
    dest = np.empty(A, dtype=np.int32)
    src = np.full(max(A, 1), -1, dtype=np.int32)
    nk = np.zeros(1, dtype=np.int32)
    lib().orc_permute(C.byref(d), _p(idx), -1 if cap is None else int(cap), _p(counts), _p(kept),
                      _p(offsets), _p(dest), _p(src), _p(nk))
    n = int(nk[0])
    return dict(counts=counts, kept=kept, offsets=offsets, dest_row=dest, src_sub=src[:n], n_kept=n)


def expert_ffn(cfg, din, w1, w3, w2, xin, with_mag=False):
    """Rows xin [n, din] (float64) through one expert; returns [n, din] float64.
    With with_mag also the magnitude sum_j |hdn_j||W2[o][j]| per output and the
    standard deviation that rounding hdn to bf16 adds to each output
    (sqrt(sum_j W2[o][j]^2 ulp(hdn_j)^2 / 12); 0 for fp32): (out, mag, sig)."""
    el = _elem(cfg)
    act = 1 if cfg.get("act", "swiglu") == "gelu" else 0
    dt = 1 if cfg["dtype"] == "bf16" else 0
    w1 = _chk(w1, el)
    w2 = _chk(w2, el)
    w3 = None if act == 1 else _chk(w3, el)
    xin = np.ascontiguousarray(np.atleast_2d(xin), dtype=np.float64)
    f = w1.size // din
    out = np.empty_like(xin)
    mag = np.empty_like(xin)
    var = np.empty_like(xin)
    lib().orc_expert_ffn_rows(dt, act, din, f, _p(w1), _p(w3), _p(w2), xin.shape[0], _p(xin), _p(out), _p(mag),
                              _p(var))
    return (out, mag, np.sqrt(var)) if with_mag else out


def combine(cfg, dest_row, topk_w, y_perm, y_shared=None, T=None):
    """Gate-weighted combine of expert output rows; returns y [T, h] float64."""
    d = desc(cfg, T)
    el = _elem(cfg)
    dr = _chk(dest_row, np.int32).ravel()
    w = np.ascontiguousarray(topk_w, dtype=np.float64).ravel()
    yp = _chk(y_perm, el)
    ys = None if y_shared is None else _chk(y_shared, el)
    y = np.empty((d.T, d.h), dtype=np.float64)
    lib().orc_combine(C.byref(d), _p(dr), _p(w), _p(yp), _p(ys), _p(y))
    return y


def layer_forward(cfg, weights, x, tokens=None, T=None):
    """Whole layer.  weights: dict with numpy arrays (keys as in OrcWeights).
    Returns dict with y [n_tokens, h] float64 and the routing/aux arrays, plus
    the two scales of the bf16 parity bound (moe_oracle.c): ymag, the
    magnitude of the terms, and ysig, the standard deviation that the
    intermediate bf16 roundings add (0 for fp32 layers)."""
    d = desc(cfg, T)
    el = _elem(cfg)
    S = d.T * d.H
    A = S * d.K
    Et = d.H * d.E
    keep = []

    def ptr(name, dtype):
        a = weights.get(name)
        if a is None:
            return None
        a = _chk(a, dtype)
        keep.append(a)
        return a.ctypes.data

    W = OrcWeights(
        w_router=ptr("w_router", el), logit_bias=ptr("logit_bias", np.float32),
        select_bias=ptr("select_bias", np.float32), w_gate=ptr("w_gate", el),
        w_up=ptr("w_up", el), w_down=ptr("w_down", el), sh_gate=ptr("sh_gate", el),
        sh_up=ptr("sh_up", el), sh_down=ptr("sh_down", el), w_o=ptr("w_o", el),
        hash_keys=ptr("hash_keys", np.int32),
    )
    x = _chk(x, el)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    nt = d.T if tok is None else tok.size
    y = np.zeros((nt, d.h), dtype=np.float64)
    ymag = np.zeros((nt, d.h), dtype=np.float64)
    yvar = np.zeros((nt, d.h), dtype=np.float64)
    out = dict(
        topk_idx=np.empty((S, d.K), np.int32), topk_w=np.empty((S, d.K), np.float64),
        margin=np.empty(S, np.float64), counts=np.empty(Et, np.int32), kept=np.empty(Et, np.int32),
        offsets=np.empty(Et + 1, np.int32), dest_row=np.empty(A, np.int32),
        src_sub=np.full(max(A, 1), -1, np.int32), n_kept=np.zeros(1, np.int32),
        f=np.empty(Et, np.float64), P=np.empty(Et, np.float64), l_aux=np.zeros(1, np.float64),
        logits=np.empty((S, d.E), np.float32),
    )
    aux = OrcAux(**{k: _p(v) for k, v in out.items()})
    rc = lib().orc_layer_forward(C.byref(d), C.byref(W), _p(x), _p(tok), nt, _p(y), _p(ymag), _p(yvar),
                                 C.byref(aux))
    if rc != 0:
        raise ValueError("oracle rejected the layer description")
    out["n_kept"] = int(out["n_kept"][0])
    out["src_sub"] = out["src_sub"][: out["n_kept"]]
    out["l_aux"] = float(out["l_aux"][0])
    out["y"] = y
    out["ymag"] = ymag
    out["ysig"] = np.sqrt(yvar)
    return out


def _weights_struct(cfg, weights, keep):
    el = _elem(cfg)

    def ptr(name, dtype):
        a = weights.get(name)
        if a is None:
            return None
        a = _chk(a, dtype)
        keep.append(a)
        return a.ctypes.data

    return OrcWeights(
        w_router=ptr("w_router", el), logit_bias=ptr("logit_bias", np.float32),
        select_bias=ptr("select_bias", np.float32), w_gate=ptr("w_gate", el),
        w_up=ptr("w_up", el), w_down=ptr("w_down", el), sh_gate=ptr("sh_gate", el),
        sh_up=ptr("sh_up", el), sh_down=ptr("sh_down", el), w_o=ptr("w_o", el),
        hash_keys=ptr("hash_keys", np.int32),
    )


def layer_backward(cfg, weights, x, dy, c_aux=1.0, magnitude=False):
    """Gradients of L = sum(dy * y) + c_aux * L_aux with respect to x and every
    weight, in float64 (moe_oracle.c, orc_layer_backward).  With magnitude, the
    same sums taken over absolute values (the scale of rounding errors).
    Returns a dict with dx, dw_router, dw_gate, dw_up, dw_down, dsh_gate,
    dsh_up, dsh_down, dw_o (None where the layer has no such weight), dlogits
    [T*H, E] and dtopk_w [T*H, K]."""
    d = desc(cfg)
    S, Et, dd, f, h = d.T * d.H, d.H * d.E, d.h // d.H, d.f, d.h
    keep = []
    W = _weights_struct(cfg, weights, keep)
    x = _chk(x, _elem(cfg))
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    assert dy.shape == (d.T, h)
    gated = cfg.get("act", "swiglu") != "gelu"
    out = dict(
        dx=np.zeros((d.T, h)), dw_router=np.zeros((d.H, d.E, dd)) if cfg.get("gate", "topk") != "hash" else None,
        dw_gate=np.zeros((Et, f, dd)), dw_up=np.zeros((Et, f, dd)) if gated else None,
        dw_down=np.zeros((Et, dd, f)),
        dsh_gate=np.zeros((f, h)) if d.n_shared else None,
        dsh_up=np.zeros((f, h)) if d.n_shared and gated else None,
        dsh_down=np.zeros((h, f)) if d.n_shared else None,
        dw_o=np.zeros((h, h)) if d.has_wo else None,
        dlogits=np.zeros((S, d.E)), dtopk_w=np.zeros((S, d.K)),
    )
    G = OrcGrads(**{k: _p(v) for k, v in out.items()})
    rc = lib().orc_layer_backward(C.byref(d), C.byref(W), _p(x), _p(dy), float(c_aux), int(bool(magnitude)),
                                  C.byref(G))
    if rc != 0:
        raise ValueError("oracle rejected the layer description")
    return out


def num_threads():
    return int(lib().orc_num_threads())


def set_num_threads(n):
    lib().orc_set_num_threads(int(n))


# ------------------------------------------- expert-parallel load report
# The course's exercise: expert e lives on rank e // experts_per_rank, a rank's
# load is the sum of its experts' token counts, the imbalance ratio is
# max / mean of the per-rank loads, the routed volume (an upper bound on what
# crosses the network) is the total of the token counts, and the hardware
# utilisation when every rank waits for the slowest is sum / (ranks * max).
def expert_to_rank(num_experts, experts_per_rank):
    return {e: e // experts_per_rank for e in range(num_experts)}


def load_per_rank(tokens_per_expert, experts_per_rank):
    ranks = len(tokens_per_expert) // experts_per_rank
    loads = [0] * ranks
    owner = expert_to_rank(len(tokens_per_expert), experts_per_rank)
    for e, n in enumerate(tokens_per_expert):
        loads[owner[e]] += n
    return loads


def imbalance(loads):
    """Busiest rank's load over the average rank load (1.0 = perfectly even)."""
    n = len(loads)
    total = sum(loads)
    if n == 0 or total <= 0:
        raise ValueError(f"imbalance is undefined for {n} ranks carrying {total} tokens")
    return n * max(loads) / total


def routing_volume(tokens_per_expert):
    """Assignments that leave their token's rank, at most: one per (token, choice)."""
    vol = 0
    for n in tokens_per_expert:
        vol += int(n)
    return vol


def utilisation(loads):
    return sum(loads) / (len(loads) * max(loads))
