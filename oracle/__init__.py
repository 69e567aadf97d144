"""fp64 CPU oracle for the learnable butterfly rotation and its quantizer.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, by the smoke check and
by the CPU-baseline leg of the benchmark.  The product library never imports,
links or calls anything here, and nothing here imports the product package.

The arithmetic lives in ``bflyref.c`` (plain C, fp64, one loop iteration per
Givens pair); this module only builds it with gcc and marshals numpy arrays.
Each function cites the passage of the pages it follows:

* forward / kron_forward -- "ButterflyQuant" abstract (Fugu-MT page,
  arXiv 2509.09679): orthogonal Q from continuous Givens angles,
  n log n / 2 parameters, O(n log n) work; duidaima.com write-up, section
  "butterfly": Hadamard special case and the Kronecker composite for 5120.
* quantize -- WUSH page (gist.science), technical summary section 2: RTN
  quantizer with absmax block scaling; ButterflyQuant abstract: transforms
  are applied before quantization.
* backward -- ButterflyQuant abstract and duidaima.com section "training and
  results": the angles are learned by gradient descent.
* kron_backward -- gradients of the Kronecker composite (duidaima.com
  section "butterfly" for the composite, section "training and results" for
  learning the angles): dL/dz = (O^T kron I) G in fp64, then the butterfly
  backward on the rows * m segments.  The C backward reads its G in fp32,
  so dL/dz is rounded to fp32 first (2^-24 relative).
* calib_weight_loss_grad / calib_weight_step -- the same step with the
  layer's output as the reconstruction target (duidaima.com section
  "training and results"; ButterflyQuant abstract: computational invariance
  and 2-bit weights): numpy fp64 products of the rotated, quantized layer,
  the chain rule through both rotations with the quantizer's rounding
  passed straight through, and the C backward for each branch.
* calib_loss_grad / adam / calib_step -- one calibration step for the
  angles (duidaima.com section "training and results": a reconstruction
  loss plus the KL divergence between the rotated activations' distribution
  and the uniform one; ButterflyQuant abstract: uniformity regularisation,
  gradient descent on calibration samples).  numpy, fp64: the quantizer is
  ``quantize`` above, the histogram is linear interpolation onto bin
  centres, Adam is the textbook update.  The readings (which quantizer,
  how the histogram is made differentiable, which quantities are held
  constant, smoothing, the optimiser) are stated where the functions are.
* hadamard_matrix / hadamard / kron_hadamard -- the Hadamard special case
  (duidaima.com write-up, section "butterfly": H_n for n = 2^k is a butterfly
  with particular angles; ButterflyQuant abstract: Hadamard entries are +-1,
  coherence 1/sqrt(n)).  Written in numpy from the matrix's definition in
  Sylvester order, H_n[i][j] = (-1)^popcount(i AND j) / sqrt(n), applied by a
  dense product -- deliberately not by a butterfly, so that it checks one.
* dequantize / quant_matmul -- the consumer of the quantized weights:
  y = W x = (W Q^T)(Q x) with W Q^T stored as 2-bit (or 4-bit) group codes
  (ButterflyQuant abstract: computational invariance and 2-bit weights;
  duidaima.com section "training and results": W2A16).  Written in numpy:
  unpack the codes, s * q or s * (q - zero) per element in fp64, then one
  fp64 matrix product.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bflyref.c")
_LIB = os.path.join(_HERE, "libbflyref.so")

F32 = 0
BF16 = 1
SYM = 0
ASYM = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp, i64, i32, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.bflyref_forward.argtypes = [vp, ctypes.c_int, dp, i64, i32, vp]
        lib.bflyref_kron_forward.argtypes = [vp, ctypes.c_int, dp, i64, i32, i32, vp, vp]
        lib.bflyref_quantize.argtypes = [dp, i64, i32, i32, i32, i32, i32, vp, vp, vp, dp, dp, dp]
        lib.bflyref_backward.argtypes = [vp, vp, i64, i32, vp, dp, dp, dp, dp]
        lib.bflyref_round_bf16.argtypes = [dp, vp, i64]
        lib.bflyref_round_fp16.argtypes = [dp, vp, i64]
        lib.bflyref_fp16_value.argtypes = [ctypes.c_uint16]
        lib.bflyref_fp16_value.restype = ctypes.c_double
        lib.bflyref_num_threads.restype = ctypes.c_int
        lib.bflyref_set_num_threads.argtypes = [ctypes.c_int]
        for f in (lib.bflyref_forward, lib.bflyref_kron_forward, lib.bflyref_quantize,
                  lib.bflyref_backward):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _x_dtype(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits), got %s" % x.dtype)


def num_threads() -> int:
    return _load().bflyref_num_threads()


def set_num_threads(k: int) -> None:
    """Threads the oracle's parallel loops use from now on."""
    _load().bflyref_set_num_threads(int(k))


def forward(x: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """y = Q(theta) x for every row, fp64.  x: float32 or bf16 bits [rows][n];
    theta: float32 [log2 n][n/2]."""
    x = np.ascontiguousarray(x)
    theta = np.ascontiguousarray(theta, dtype=np.float32)
    rows, n = x.shape
    y = np.empty((rows, n), dtype=np.float64)
    rc = _load().bflyref_forward(_ptr(x), _x_dtype(x), _ptr(y), rows, n, _ptr(theta))
    if rc != 0:
        raise ValueError("bflyref_forward rejected its arguments")
    return y


def kron_forward(x: np.ndarray, theta_b: np.ndarray, mix: np.ndarray) -> np.ndarray:
    """y = (O kron B(theta_b)) x, index i = a*nb + b; fp64."""
    x = np.ascontiguousarray(x)
    theta_b = np.ascontiguousarray(theta_b, dtype=np.float32)
    mix = np.ascontiguousarray(mix, dtype=np.float32)
    m = mix.shape[0]
    rows, n = x.shape
    nb = n // m
    y = np.empty((rows, n), dtype=np.float64)
    rc = _load().bflyref_kron_forward(_ptr(x), _x_dtype(x), _ptr(y), rows, m, nb,
                                       _ptr(theta_b), _ptr(mix))
    if rc != 0:
        raise ValueError("bflyref_kron_forward rejected its arguments")
    return y


def quantize(y: np.ndarray, bits: int, group: int, mode: int, scales=None, zeros=None,
             want_v: bool = False):
    """Per-group RTN quantization of fp64 rows.

    Returns a dict with codes (uint8), scales (uint16 fp16 bits), zeros (asym),
    s_pre (fp64 scale before rounding), z_pre (asym) and optionally v (y/scale).
    If ``scales`` (and ``zeros``) are given, the codes are computed at those
    scales (and zero points) instead of the oracle's own; with ``scales``
    alone in asymmetric mode, the zero points are derived at those scales."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    rows, n = y.shape
    ng = n // group
    codes = np.zeros((rows, n * bits // 8), dtype=np.uint8)
    use_given = scales is not None
    given_zeros = use_given and mode == ASYM and zeros is not None
    sc = np.ascontiguousarray(scales, dtype=np.uint16).copy() if use_given else \
        np.zeros((rows, ng), dtype=np.uint16)
    if mode == ASYM:
        zr = np.ascontiguousarray(zeros, dtype=np.uint16).copy() if given_zeros else \
            np.zeros((rows, ng), dtype=np.uint16)
    else:
        zr = None
    how = 0 if not use_given else (1 if (mode == SYM or given_zeros) else 2)
    s_pre = np.empty((rows, ng), dtype=np.float64)
    z_pre = np.zeros((rows, ng), dtype=np.float64) if mode == ASYM else None
    v = np.empty((rows, n), dtype=np.float64) if want_v else None
    rc = _load().bflyref_quantize(_ptr(y), rows, n, group, bits, mode, how,
                                   _ptr(codes), _ptr(sc), _ptr(zr), _ptr(s_pre), _ptr(z_pre),
                                   _ptr(v))
    if rc != 0:
        raise ValueError("bflyref_quantize rejected its arguments")
    out = {"codes": codes, "scales": sc, "s_pre": s_pre}
    if mode == ASYM:
        out["zeros"] = zr
        out["z_pre"] = z_pre
    if want_v:
        out["v"] = v
    return out


def backward(x: np.ndarray, g: np.ndarray, theta: np.ndarray, want_y=True, want_dx=True):
    """Returns dict(y, dx, dtheta, dabs) in fp64 (see bflyref_backward)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    theta = np.ascontiguousarray(theta, dtype=np.float32)
    rows, n = x.shape
    L = theta.shape[0]
    y = np.empty((rows, n), dtype=np.float64) if want_y else None
    dx = np.empty((rows, n), dtype=np.float64) if want_dx else None
    dth = np.empty((L, n // 2), dtype=np.float64)
    dab = np.empty((L, n // 2), dtype=np.float64)
    rc = _load().bflyref_backward(_ptr(x), _ptr(g), rows, n, _ptr(theta), _ptr(y), _ptr(dx),
                                   _ptr(dth), _ptr(dab))
    if rc != 0:
        raise ValueError("bflyref_backward rejected its arguments")
    return {"y": y, "dx": dx, "dtheta": dth, "dabs": dab}


def round_bf16(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest even, directly from fp64."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    _load().bflyref_round_bf16(_ptr(y), _ptr(out), y.size)
    return out


def round_fp16(y: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 bits, round to nearest even, directly from fp64."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    _load().bflyref_round_fp16(_ptr(y), _ptr(out), y.size)
    return out


def fp16_value(h: int) -> float:
    return _load().bflyref_fp16_value(int(h))


def dense_q(theta: np.ndarray) -> np.ndarray:
    """Dense Q (n x n) built column by column from unit vectors: column k is
    Q e_k.  For tests at small n only."""
    theta = np.asarray(theta, dtype=np.float32)
    n = theta.shape[1] * 2
    eye = np.eye(n, dtype=np.float32)
    return forward(eye, theta).T.copy()


def widen(x: np.ndarray) -> np.ndarray:
    """float32 rows, or bf16 bit patterns (uint16), as fp64 (exact)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits), got %s" % x.dtype)


def hadamard_matrix(n: int) -> np.ndarray:
    """Orthonormal Sylvester-ordered Walsh-Hadamard matrix, fp64:
    entry (i, j) = (-1)^(number of bits set in i AND j) / sqrt(n)."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    idx = np.arange(n, dtype=np.int64)
    both = idx[:, None] & idx[None, :]
    parity = np.zeros_like(both)
    b = 1
    while b < n:
        parity ^= (both & b) != 0
        b <<= 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(float(n))


def hadamard(x: np.ndarray) -> np.ndarray:
    """y = H_n x for every row, fp64.  x: float32 or bf16 bits [rows][n]."""
    x = widen(np.ascontiguousarray(x))
    return x @ hadamard_matrix(x.shape[1]).T


def kron_hadamard(x: np.ndarray, mix: np.ndarray) -> np.ndarray:
    """y = (O kron H_nb) x, index i = a*nb + b, O = mix (m x m); fp64."""
    x = widen(np.ascontiguousarray(x))
    mix = np.asarray(mix, dtype=np.float32).astype(np.float64)
    m = mix.shape[0]
    nb = x.shape[1] // m
    return x @ np.kron(mix, hadamard_matrix(nb)).T


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros, bits: int, group: int, mode: int,
               n: int) -> np.ndarray:
    """Group-quantized rows back to fp64 values: codes u8 [rows][n*bits/8]
    (element e of a byte in bits [bits*e, bits*(e+1)); symmetric codes are
    two's-complement fields), scales / zeros fp16 bit patterns
    [rows][n/group].  Symmetric: s*q; asymmetric: s*(q - zero)."""
    per = 8 // bits
    c = np.asarray(codes).astype(np.int64)
    rows = c.shape[0]
    q = np.empty((rows, n), dtype=np.int64)
    for e in range(per):
        q[:, e::per] = (c >> (bits * e)) & ((1 << bits) - 1)
    if mode == SYM:
        q = np.where(q >= (1 << (bits - 1)), q - (1 << bits), q)
    s = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)
    s = np.repeat(s, group, axis=1)
    if mode == SYM:
        return s * q
    z = np.asarray(zeros, dtype=np.uint16).view(np.float16).astype(np.float64)
    return s * (q - np.repeat(z, group, axis=1))


def quant_matmul(a: np.ndarray, codes: np.ndarray, scales: np.ndarray, zeros, bits: int,
                 group: int, mode: int) -> np.ndarray:
    """y[m][o] = sum_k a[m][k] * w[o][k], w the dequantized weight rows; fp64.
    a: float32 or bf16 bits [M][K]; codes etc. as in dequantize, K = a's width."""
    a = widen(np.ascontiguousarray(a))
    w = dequantize(codes, scales, zeros, bits, group, mode, a.shape[1])
    return a @ w.T


def kron_backward(x: np.ndarray, g: np.ndarray, theta_b: np.ndarray, mix: np.ndarray):
    """Gradients of y = (O kron B(theta_b)) x with O = mix fixed: returns
    dict(dx (fp64 [rows][m*nb]), dtheta (fp64 [log2 nb][nb/2]), dabs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    mix64 = np.asarray(mix, dtype=np.float32).astype(np.float64)
    m = mix64.shape[0]
    rows, n = x.shape
    nb = n // m
    g3 = np.asarray(g, dtype=np.float32).astype(np.float64).reshape(rows, m, nb)
    # dL/dz[r][a'][b] = sum_a O[a][a'] G[r][a][b]
    gz = np.einsum("ab,rai->rbi", mix64, g3).reshape(rows * m, nb)
    out = backward(x.reshape(rows * m, nb), gz.astype(np.float32), theta_b, want_y=False)
    return {"dx": out["dx"].reshape(rows, n), "dtheta": out["dtheta"], "dabs": out["dabs"]}


CALIB_SMOOTH = 1e-6


def _group_absmax(y: np.ndarray, group: int) -> np.ndarray:
    rows, n = y.shape
    a = np.abs(y).reshape(rows, n // group, group).max(axis=2)
    return np.repeat(a, group, axis=1)


def calib_loss_grad(y: np.ndarray, bits: int, group: int, bins: int, lambda_kl: float,
                    with_rec: bool = True):
    """Loss and dL/dy of one calibration step at Y (fp64 [rows][n]).

    Readings: the reconstruction term is the group quantizer's error,
    L_rec = sum (y - y^)^2 / N with y^ = dequantized symmetric absmax RTN
    codes (held constant: no gradient through the rounding or the scale);
    the uniformity term is KL(p' || uniform) with p the distribution of
    u = y / a (a = the group's max |y|, held constant) on `bins` centres
    c_b = -1 + (b + 1/2) h, h = 2 / bins, each u giving linear-interpolation
    weights to its two nearest centres (u clamped to [c_0, c_{bins-1}];
    a clamped u has no gradient), p' = (p + 1e-6) / (1 + bins 1e-6).
    with_rec=False leaves the reconstruction term out of loss and g (the
    uniformity term alone, for the weight-side loss below).
    Returns dict(loss, rec, kl, g, t) with t = (u - c_0) / h (unclamped)."""
    y = np.asarray(y, dtype=np.float64)
    N = y.size
    q = quantize(y, bits, group, SYM)
    yhat = dequantize(q["codes"], q["scales"], None, bits, group, SYM, y.shape[1])
    rec = float(((y - yhat) ** 2).sum() / N)
    a = _group_absmax(y, group)
    u = np.divide(y, a, out=np.zeros_like(y), where=a > 0)
    h = 2.0 / bins
    t = (u + 1.0) / h - 0.5
    inside = (t >= 0) & (t <= bins - 1)
    tc = np.clip(t, 0, bins - 1)
    j = np.minimum(np.floor(tc).astype(np.int64), bins - 2)
    f = tc - j
    p = (np.bincount(j.ravel(), weights=(1 - f).ravel(), minlength=bins) +
         np.bincount((j + 1).ravel(), weights=f.ravel(), minlength=bins)) / N
    ps = (p + CALIB_SMOOTH) / (1 + bins * CALIB_SMOOTH)
    lb = np.log(bins * ps)
    kl = float((ps * lb).sum())
    g = 2.0 * (y - yhat) / N if with_rec else np.zeros_like(y)
    dkl = (lb[j + 1] - lb[j]) / (h * N * (1 + bins * CALIB_SMOOTH))
    g += lambda_kl * np.where(inside & (a > 0), dkl / np.where(a > 0, a, 1.0), 0.0)
    return {"loss": (rec if with_rec else 0.0) + lambda_kl * kl, "rec": rec, "kl": kl, "g": g,
            "t": t, "p": p, "yhat": yhat, "a": a}


def adam(theta, m, v, g, step: int, lr: float, beta1: float, beta2: float, eps: float):
    """The textbook Adam update (bias-corrected moments), fp64."""
    m = beta1 * np.asarray(m, np.float64) + (1 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1 - beta2) * g * g
    mh = m / (1 - beta1 ** step)
    vh = v / (1 - beta2 ** step)
    return np.asarray(theta, np.float64) - lr * mh / (np.sqrt(vh) + eps), m, v


def calib_step(x, theta, m, v, step, bits, group, bins, lambda_kl, lr, beta1, beta2, eps):
    """One calibration step: Y = Q X (fp64), loss and dL/dY, dtheta by the
    butterfly backward (its G read in fp32), one Adam update."""
    y = forward(x, theta)
    lg = calib_loss_grad(y, bits, group, bins, lambda_kl)
    bw = backward(x, lg["g"].astype(np.float32), theta, want_y=False, want_dx=False)
    th2, m2, v2 = adam(theta, m, v, bw["dtheta"], step, lr, beta1, beta2, eps)
    return dict(lg, y=y, dtheta=bw["dtheta"], dabs=bw["dabs"], theta=th2, m=m2, v=v2)


def calib_weight_loss_grad(x, w, theta, bits: int, group: int, mode: int, bins: int,
                           lambda_kl: float, wq=None):
    """Loss and dL/dtheta of one calibration step whose reconstruction term is
    the layer's output (duidaima.com write-up, section "training and
    results": the quantized model's output should match the original one;
    ButterflyQuant abstract: computational invariance W x = (W Q^T)(Q x) and
    2-bit weights).  fp64 throughout (x, w: float32 or bf16 bits).

    Readings:
      Xr = Q X (each row of X rotated), Wr = W Q^T (each row of W rotated),
      What = the group quantizer's value of Wr (bits, group, mode; or the
             codes, scales, zeros given as wq = (codes, scales, zeros)),
      Y = X W^T,  Yhat = Xr What^T,
      L_rec = sum (Yhat - Y)^2 / (rows * out),
      L = L_rec + lambda KL(Xr), the uniformity term of calib_loss_grad on Xr.
    The quantizer's rounding passes gradients straight through (What - Wr is
    held constant), so by the chain rule
      dL/dYhat = 2 (Yhat - Y) / (rows * out),
      dL/dXr = dL/dYhat What,   dL/dWr = dL/dYhat^T Xr,
    and dtheta is the butterfly backward of X with dL/dXr (plus the uniformity
    term's dL/dXr) added to the backward of W's rows with dL/dWr.
    Returns dict(loss, rec, kl, dtheta, dabs, gx, gw, r, e, xr, wr, what)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    n = x.shape[1]
    xr = forward(x, theta)
    wr = forward(w, theta)
    if wq is None:
        q = quantize(wr, bits, group, mode)
        wq = (q["codes"], q["scales"], q.get("zeros"))
    what = dequantize(wq[0], wq[1], wq[2], bits, group, mode, n)
    y = widen(x) @ widen(w).T
    yhat = xr @ what.T
    r = yhat - y
    n_rec = r.size
    rec = float((r * r).sum() / n_rec)
    kl = calib_loss_grad(xr, 4, group, bins, lambda_kl, with_rec=False)
    dyhat = 2.0 * r / n_rec
    gx = dyhat @ what + kl["g"]
    gw = dyhat.T @ xr
    bx = backward(widen(x).astype(np.float32), gx.astype(np.float32), theta, want_y=False,
                  want_dx=False)
    bw = backward(widen(w).astype(np.float32), gw.astype(np.float32), theta, want_y=False,
                  want_dx=False)
    return {"loss": rec + lambda_kl * kl["kl"], "rec": rec, "kl": kl["kl"],
            "dtheta": bx["dtheta"] + bw["dtheta"], "dabs": bx["dabs"] + bw["dabs"],
            "gx": gx, "gw": gw, "r": r, "e": what - wr, "xr": xr, "wr": wr, "what": what,
            "p": kl["p"], "a": kl["a"], "t": kl["t"]}


def calib_weight_step(x, w, theta, m, v, step, bits, group, mode, bins, lambda_kl, lr, beta1,
                      beta2, eps, wq=None):
    """One calibration step with the layer-output loss: calib_weight_loss_grad,
    then one Adam update of theta."""
    out = calib_weight_loss_grad(x, w, theta, bits, group, mode, bins, lambda_kl, wq)
    th2, m2, v2 = adam(theta, m, v, out["dtheta"], step, lr, beta1, beta2, eps)
    return dict(out, theta=th2, m=m2, v=v2)
