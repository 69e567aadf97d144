"""Element-by-element comparison of GPU results with the fp64 oracle.

Tolerances (the readings the design documents give them):
* fp32 outputs: |gpu - y64| <= 1e-5 * ||x_r||_inf * log2(n), per row.
* bf16 outputs: |gpu - bf16(y64)| <= one bf16 ulp of bf16(y64); values whose
  bf16 ulp is finer than fp32 arithmetic can resolve (near zero) pass when
  |gpu - y64| <= 4 * ceil(log2 n) * 2^-24 * ||x_r||_2 -- counted separately.
* fp16 scales: bit-exact, except where the oracle's pre-rounding scale lies
  within 1e-6 (relative) of an fp16 rounding midpoint: either neighbour
  passes (counted).  Zero points: the oracle derives them again at the
  scale the GPU emitted; they must match except within 1e-6 (absolute) of a
  rounding boundary of -min/s.
* codes: the oracle re-quantizes its fp64 y at the scales (and zero points)
  the GPU emitted; codes must match bit for bit except where y64/scale lies
  within 1e-6 of a rounding boundary (counted).
* angle gradients: |gpu - dtheta64| <= 1e-5 * log2(n) * A, with A the sum of
  the magnitudes of the cancelling terms.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

U32 = 2.0 ** -24


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_to_f64(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_ulp(b: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid at each (finite) bf16 value."""
    v = np.abs(bf16_to_f64(b))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126)
    return np.where(v > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_f32(gpu: np.ndarray, y64: np.ndarray, x_inf: np.ndarray, n: int):
    bound = 1e-5 * x_inf[:, None] * math.log2(n)
    err = np.abs(gpu.astype(np.float64) - y64)
    bad = err > bound
    return {"ok": not bad.any(), "fails": int(bad.sum()),
            "max_rel_to_bound": float((err / np.maximum(bound, 1e-300)).max())}


def check_bf16(gpu_bits: np.ndarray, y64: np.ndarray, x_l2: np.ndarray, n: int):
    ref = oracle.round_bf16(y64)
    g = bf16_to_f64(gpu_bits)
    ulp = bf16_ulp(ref)
    within_ulp = np.abs(g - bf16_to_f64(ref)) <= ulp
    floor = 4 * math.ceil(math.log2(n)) * U32 * x_l2[:, None]
    within_floor = np.abs(g - y64) <= floor
    ok = within_ulp | within_floor
    return {"ok": bool(ok.all()), "fails": int((~ok).sum()),
            "exact": int((gpu_bits == ref).sum()), "by_floor": int((~within_ulp & within_floor).sum()),
            "total": int(ref.size)}


def _near_half(v: np.ndarray, win: float) -> np.ndarray:
    return np.abs(np.abs(v - np.floor(v)) - 0.5) <= win


def check_quant(y64: np.ndarray, codes: np.ndarray, scales: np.ndarray, zeros, bits: int,
                group: int, mode: int):
    """Compare GPU codes/scales/zeros with the oracle on fp64 rows y64."""
    ref = oracle.quantize(y64, bits, group, mode)
    res = {"ok": True}
    # scales
    s_pre = ref["s_pre"]
    s_pre_c = np.minimum(s_pre, 65504.0)
    sdiff = scales != ref["scales"]
    # rounding boundary of s_pre between the two fp16 neighbours
    lo = np.minimum(fp16_to_f64(scales), fp16_to_f64(ref["scales"]))
    hi = np.maximum(fp16_to_f64(scales), fp16_to_f64(ref["scales"]))
    adjacent = np.abs(scales.astype(np.int64) - ref["scales"].astype(np.int64)) == 1
    mid = (lo + hi) / 2
    in_win = adjacent & (np.abs(s_pre_c - mid) <= 1e-6 * np.abs(s_pre_c))
    res["scale_mismatch"] = int(sdiff.sum())
    res["scale_in_window"] = int((sdiff & in_win).sum())
    if (sdiff & ~in_win).any():
        res["ok"] = False
        res["scale_bad"] = int((sdiff & ~in_win).sum())
    if mode == oracle.ASYM:
        # zero points re-derived at the scales the GPU emitted (its own where
        # the scales agree), window 1e-6 on -min / scale
        zref = oracle.quantize(y64, bits, group, mode, scales=scales)
        zdiff = zeros != zref["zeros"]
        zin = _near_half(zref["z_pre"], 1e-6)
        res["zero_mismatch"] = int(zdiff.sum())
        res["zero_in_window"] = int((zdiff & zin).sum())
        if (zdiff & ~zin).any():
            res["ok"] = False
            res["zero_bad"] = int((zdiff & ~zin).sum())
    # codes at the GPU's own scales / zeros
    req = oracle.quantize(y64, bits, group, mode, scales=scales,
                          zeros=zeros if mode == oracle.ASYM else None, want_v=True)
    per = 8 // bits
    n = y64.shape[1]
    c_gpu = np.zeros(y64.shape, dtype=np.int64)
    c_ref = np.zeros(y64.shape, dtype=np.int64)
    for k in range(per):
        c_gpu[:, k::per] = (codes.astype(np.int64) >> (bits * k)) & ((1 << bits) - 1)
        c_ref[:, k::per] = (req["codes"].astype(np.int64) >> (bits * k)) & ((1 << bits) - 1)
    cdiff = c_gpu != c_ref
    win = _near_half(req["v"], 1e-6)
    res["code_mismatch"] = int(cdiff.sum())
    res["code_in_window"] = int(win.sum())
    res["code_bad"] = int((cdiff & ~win).sum())
    res["codes_total"] = int(n * y64.shape[0])
    if res["code_bad"]:
        res["ok"] = False
    return res


def check_dtheta(gpu: np.ndarray, d64: np.ndarray, dabs: np.ndarray, n: int):
    bound = 1e-5 * math.log2(n) * dabs
    err = np.abs(gpu.astype(np.float64) - d64)
    bad = err > bound
    return {"ok": not bad.any(), "fails": int(bad.sum()),
            "max_err_over_A": float((err / np.maximum(dabs, 1e-300)).max())}
