"""Seeded synthetic workloads.

Numpy only; this module holds no arithmetic of the rotation or the quantizer.
It draws angles, activations, weights, gradients and the Kronecker mixing
factor from fixed seeds so that the GPU path and the CPU oracle are fed the
same bytes.  The shapes follow the workloads the ButterflyQuant pages speak
of (LLaMA-2-7B hidden width 4096, LLaMA-2-13B width 5120, 2-bit weights,
128 calibration samples); no dataset or checkpoint is used.

Recipe (every tensor has its own child stream of
``SeedSequence(seed).spawn(k)``, drawn in fp64 and then cast):

* angles: uniform on [-pi, pi), cast to fp32, shape [log2 n][n/2];
* activations: N(0, 1); ``round(0.001 * n)`` outlier channels, chosen
  without replacement per seed and shared by all rows, are multiplied by 50;
  then cast to the storage dtype;
* weights: N(0, 0.02^2), no outliers;
* gradients: N(0, 1);
* Kronecker mixing factor: Q of the QR decomposition of an m x m N(0, 1) draw,
  with column signs chosen so that diag(R) > 0, cast to fp32.

bf16 storage is fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest
even on the fp32 bit pattern); the stored bits ARE the input, so the double
rounding is part of the recipe, not an error.
"""
from __future__ import annotations

import math

import numpy as np


def _streams(seed: int, k: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(k)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (storage cast)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def angles(rng, n: int) -> np.ndarray:
    L = int(round(math.log2(n)))
    assert 1 << L == n
    return rng.uniform(-math.pi, math.pi, size=(L, n // 2)).astype(np.float32)


def outlier_columns(rng, n: int) -> np.ndarray:
    k = int(round(0.001 * n))
    return np.sort(rng.choice(n, size=k, replace=False))


def activations(rng, rows: int, n: int, cols: np.ndarray, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=(rows, n))
    if cols is not None and len(cols):
        x[:, cols] *= 50.0
    x32 = x.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def mixing_factor(rng, m: int) -> np.ndarray:
    a = rng.standard_normal(size=(m, m))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


# ---------------------------------------------------------------------------
# The workloads.  Each returns a dict of numpy arrays plus metadata.
# ``rows`` may be lowered to draw the leading rows of the same workload: the
# row draws are sequential, so the first r rows are identical whatever the
# total.
# ---------------------------------------------------------------------------

def tiny_fp32(rows: int = 64, n: int = 256, seed: int = 0):
    """n=256 butterfly, fp32 rows ~ N(0,1), no quantization."""
    r_theta, r_x = _streams(seed, 2)
    theta = angles(r_theta, n)
    x = r_x.standard_normal(size=(rows, n)).astype(np.float32)
    return {"name": "tiny_n256_fp32", "n": n, "rows": rows, "theta": theta, "x": x,
            "x_dtype": "f32"}


def act_int4(rows: int = 8192, n: int = 4096, seed: int = 1):
    """LLaMA-2-7B-width activations, bf16 with 0.1% x50 outlier channels;
    symmetric absmax INT4, group 128, fp16 scales."""
    r_theta, r_x, r_cols = _streams(seed, 3)
    theta = angles(r_theta, n)
    cols = outlier_columns(r_cols, n)
    x = activations(r_x, rows, n, cols, "bf16")
    return {"name": "act_n4096_bf16_int4", "n": n, "rows": rows, "theta": theta, "x": x,
            "x_dtype": "bf16", "outliers": cols, "bits": 4, "group": 128, "mode": "sym"}


def weight_int2(rows1: int = 4096, rows2: int = 11008, n: int = 4096, seed: int = 2):
    """W Q^T for two LLaMA-2-7B weight shapes (4096x4096, 11008x4096), bf16
    N(0, 0.02^2); asymmetric min-max INT2, group 128, fp16 scale + zero."""
    r_theta, r_w1, r_w2 = _streams(seed, 3)
    theta = angles(r_theta, n)
    w1 = f32_to_bf16_bits((0.02 * r_w1.standard_normal(size=(rows1, n))).astype(np.float32))
    w2 = f32_to_bf16_bits((0.02 * r_w2.standard_normal(size=(rows2, n))).astype(np.float32))
    return {"name": "weight_n4096_bf16_int2", "n": n, "theta": theta, "w1": w1, "w2": w2,
            "x_dtype": "bf16", "bits": 2, "group": 128, "mode": "asym"}


def kron_int4(rows: int = 8192, m: int = 5, nb: int = 1024, seed: int = 3):
    """LLaMA-2-13B width 5120 = 5 x 1024: O5 (x) B1024, bf16 activations with
    0.1% x50 outliers; symmetric INT4 group 128."""
    r_theta, r_mix, r_x, r_cols = _streams(seed, 4)
    theta_b = angles(r_theta, nb)
    mix = mixing_factor(r_mix, m)
    n = m * nb
    cols = outlier_columns(r_cols, n)
    x = activations(r_x, rows, n, cols, "bf16")
    return {"name": "kron_n5120_bf16_int4", "n": n, "m": m, "nb": nb, "rows": rows,
            "theta_b": theta_b, "mix": mix, "x": x, "x_dtype": "bf16", "outliers": cols,
            "bits": 4, "group": 128, "mode": "sym"}


def kron_wide_int4(rows: int = 8192, m: int = 43, nb: int = 256, seed: int = 6):
    """LLaMA-2-7B MLP width 11008 = 43 x 256 (the down projection's input):
    O43 (x) B256, bf16 activations with 0.1% x50 outliers; symmetric INT4
    group 128."""
    r_theta, r_mix, r_x, r_cols = _streams(seed, 4)
    theta_b = angles(r_theta, nb)
    mix = mixing_factor(r_mix, m)
    n = m * nb
    cols = outlier_columns(r_cols, n)
    x = activations(r_x, rows, n, cols, "bf16")
    return {"name": "kron_n11008_bf16_int4", "n": n, "m": m, "nb": nb, "rows": rows,
            "theta_b": theta_b, "mix": mix, "x": x, "x_dtype": "bf16", "outliers": cols,
            "bits": 4, "group": 128, "mode": "sym"}


class CalibFP32:
    """Calibration forward+backward: 128 samples x 2048 tokens = 262144 rows of
    n=4096 fp32 (N(0,1) with 0.1% x50 outlier channels) and an upstream
    gradient of the same shape ~ N(0,1).  Rows come in blocks of BLOCK rows;
    block k of X and of G is drawn from its own child stream, so blocks can be
    drawn in any order or in parallel and the 4 GiB tensors never have to sit
    in host memory at once."""

    BLOCK = 4096

    def __init__(self, rows: int = 128 * 2048, n: int = 4096, seed: int = 4):
        self.rows, self.n, self.seed = rows, n, seed
        s_theta, s_x, s_cols, s_g = np.random.SeedSequence(seed).spawn(4)
        self.theta = angles(np.random.Generator(np.random.PCG64(s_theta)), n)
        self.outliers = outlier_columns(np.random.Generator(np.random.PCG64(s_cols)), n)
        nblocks = (rows + self.BLOCK - 1) // self.BLOCK
        self._xs = s_x.spawn(nblocks)
        self._gs = s_g.spawn(nblocks)
        self.nblocks = nblocks
        self.name = "calib_n4096_fp32_fwd_bwd"

    def block(self, k: int):
        """(row0, x, g) float32 arrays of block k."""
        r0 = k * self.BLOCK
        m = min(self.BLOCK, self.rows - r0)
        x = np.random.Generator(np.random.PCG64(self._xs[k])).standard_normal(size=(m, self.n))
        x[:, self.outliers] *= 50.0
        g = np.random.Generator(np.random.PCG64(self._gs[k])).standard_normal(size=(m, self.n))
        return r0, x.astype(np.float32), g.astype(np.float32)

    def blocks(self, limit_rows: int | None = None, threads: int = 8):
        """Yield (row0, x, g) for the leading blocks, in order, drawing up to
        `threads` blocks concurrently."""
        from concurrent.futures import ThreadPoolExecutor
        total = self.rows if limit_rows is None else min(limit_rows, self.rows)
        nb = (total + self.BLOCK - 1) // self.BLOCK
        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            futs = [ex.submit(self.block, k) for k in range(min(nb, threads))]
            for k in range(nb):
                r0, x, g = futs[k].result()
                futs[k] = None
                if k + threads < nb:
                    futs.append(ex.submit(self.block, k + threads))
                m = min(x.shape[0], total - r0)
                yield r0, x[:m], g[:m]
