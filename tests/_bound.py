"""The stated parity bound for bf16 outputs against the unrounded fp64 oracle.

A bf16 evaluation of the layer rounds, to nearest, at fixed points: the FFN's
hidden activation H (the second GEMM's operand), each expert's output row (the
combine's input), the shared expert's output, the concatenated head outputs
before W_o, and the layer output y.  The oracle returns, per output element,
two scales (oracle/moe_oracle.c, orc_expert_ffn and orc_layer_forward):
  M (mag)  the magnitude of the terms, sum |H_j||W2_j| weighted as in y;
  sigma    the standard deviation those intermediate roundings add to y when
           each error is uniform on half an ulp either side and independent.

Per element (bf16), with RMS the root mean square of the reference:
  |y_gpu - y_ref| <= ulp(y)/2 + max(FLOOR * RMS, K_SIGMA * sigma) + 2^-20 * M
the first term the last rounding, FLOOR = 2e-2 the stated example bound, the
K_SIGMA = 6 standard deviations the intermediate roundings (a Gaussian passes
6 sigma about twice in 10^9 draws), the last fp32 accumulation and the fp32
exponential and reciprocal of the activation (relative 2^-22 or less, far
below bf16's 2^-8).  It must also hold the worst case, which needs no
statistics: each rounding moves a value by at most 2^-8 of itself, so
  |y_gpu - y_ref| <= ulp(y)/2 + (n_round * 2^-8 + n_acc * 2^-24) * M
with n_round the intermediate roundings on the path (2 for a layer output:
H and the expert row; 1 for an expert row) and n_acc the length of the
longest fp32 sum.  In aggregate, RMS(y_gpu - y_ref) <= RMS_BF16 * RMS(y_ref),
and the errors normalised by their expected spread sqrt(sigma^2 + ulp(y)^2/12)
have a mean square of at most Z2_MAX overall and in every row and column with
at least Z2_MIN_N samples (an error confined to one row or one column of a
tile shows there).  fp32 outputs: |dy| <= 1e-5 RMS elementwise.
"""
import math

import numpy as np

FLOOR = 2e-2
K_SIGMA = 6.0
ACC_SLACK = 2.0 ** -20
RMS_BF16 = 5e-3
Z2_MAX = 4.0
Z2_MIN_N = 32
FP32_REL = 1e-5
REPORT_REL = 2e-2


def ulp_bf16(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check(got, ref, dtype, what="", mag=None, sig=None, n_round=2, n_acc=0, rms_bound=RMS_BF16):
    """Elementwise and aggregate checks of got against ref (float arrays of
    one shape).  bf16 with mag and sig: the bound above; bf16 with mag alone:
    the worst case only (a backward-pass gradient), with n_round * 2^-8 as
    the unit; bf16 with neither: the last rounding of an fp32 sum only (the
    combine stage).  Returns the statistics (max_rel, rms_rel, n_over_2e2,
    worst ratio to the bound, mean z^2)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return {}
    rms = math.sqrt(float(np.mean(ref ** 2))) or 1.0
    err = np.abs(got - ref)
    stats = dict(max_rel=float(err.max() / rms), rms_rel=float(math.sqrt(np.mean(err ** 2)) / rms),
                 n_over_2e2=int((err > REPORT_REL * rms).sum()), n=int(ref.size))
    if dtype != "bf16":
        bounds = [("fp32", np.full(ref.shape, FP32_REL * rms))]
    else:
        half = 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref))) + 1e-6 * rms
        bounds = []
        if mag is not None:
            mag = np.asarray(mag, np.float64)
            bounds.append(("worst case", half + (n_round * 2.0 ** -8 + n_acc * 2.0 ** -24) * mag))
        if sig is not None:
            sig = np.asarray(sig, np.float64)
            bounds.append(("stated", half + np.maximum(FLOOR * rms, K_SIGMA * sig) + ACC_SLACK * mag))
        if not bounds:
            bounds = [("last rounding", half)]
    for name, bound in bounds:
        stats[f"worst_ratio_{name.replace(' ', '_')}"] = float((err / bound).max())
        bad = err > bound
        if bad.any():
            i = np.unravel_index(np.argmax(err - bound), err.shape)
            raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} elements over the {name} bound; worst at "
                                 f"{i}: got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}; {stats}")
    if dtype == "bf16" and sig is not None:
        spread = np.sqrt(sig ** 2 + ulp_bf16(ref) ** 2 / 12.0) + 1e-30
        z2 = (err / spread) ** 2
        stats["mean_z2"] = float(z2.mean())
        assert stats["mean_z2"] <= Z2_MAX, (what, "mean z^2 over all elements", stats)
        if z2.ndim == 2:
            for axis, name in ((1, "row"), (0, "column")):
                if z2.shape[axis] >= Z2_MIN_N:
                    m = z2.mean(axis=axis)
                    stats[f"max_{name}_z2"] = float(m.max())
                    assert m.max() <= Z2_MAX, (what, f"mean z^2 of {name} {int(m.argmax())}", stats)
    if dtype == "bf16" and mag is not None and ref.size >= 256 and rms_bound is not None:
        assert stats["rms_rel"] <= rms_bound, (what, stats)
    return stats
