"""GPU parity of bfly_quant_matmul (y = a w^T with w's rows as group codes)
against the fp64 oracle: ragged small shapes element by element, and the
full 8192 x 4096 x 11008 W2A16 product (activations of the headline batch
against the 11008 x 4096 weight) on sampled rows.

Tolerance (derived from each kernel's arithmetic; a sum whose terms pass
through at most D fp32 roundings is within D * 2^-24 * sum |terms| of the
exact sum):
* MFMA tiles (more than 64 rows): every product a * (q - zero) is exact in
  fp32; one group's products summed in fp32 (at most `group` roundings),
  times the group's scale (1), added over the k / group groups:
  D = group + k / group + 2, on the terms |a| |w|.
* few-row kernel (64 rows or fewer): per group the matrix cores sum the
  exact products a q' (q' the code as offset binary, q' - z = w / s; at most
  `group` roundings) and, alongside, the activations S = sum a; the group
  adds s (C - z S) (one rounding for the zero point, one for the
  accumulation over at most k / group groups), and at most 16 waves' sums
  are added: D = group + k / group + 18, on the terms |a| s (q' + z), which
  bound both sums (s (q' + z) <= |w| + 2 s |z|).
bf16 outputs add half a bf16 ulp of the result."""
import math

import numpy as np
import pytest

import oracle
import learnable_butterfly_rotation_amd as B
from learnable_butterfly_rotation_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def dev_u16(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(dtype)


def host_bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rand_codes(rng, n_out, k, bits, group, mode):
    """Random code bytes (every pattern is a valid code), fp16 scales over
    four decades and integer zero points."""
    codes = rng.integers(0, 256, size=(n_out, k * bits // 8), dtype=np.uint8)
    s = (rng.uniform(0.5, 1.5, (n_out, k // group)) * 10.0 ** rng.integers(-3, 1, (n_out, 1)))
    scales = s.astype(np.float16).view(np.uint16)
    zeros = None
    if mode == oracle.ASYM:
        zeros = rng.integers(0, 1 << bits, (n_out, k // group)).astype(np.float16).view(np.uint16)
    return codes, scales, zeros


def run(a_bits, codes, scales, zeros, bits, group, mode, y_dtype):
    rows, k = a_bits.shape
    n_out = codes.shape[0]
    y = torch.empty((rows, n_out), dtype=y_dtype, device="cuda")
    B.bfly_quant_matmul(dev_u16(a_bits, torch.bfloat16), torch.from_numpy(codes).cuda(),
                        dev_u16(scales, torch.float16),
                        dev_u16(zeros, torch.float16) if zeros is not None else None, y,
                        bits=bits, group=group, mode=mode)
    if y_dtype == torch.float32:
        torch.cuda.synchronize()
        return y.cpu().numpy().astype(np.float64)
    return (host_bits(y).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rounding_depth(call_rows, k, group):
    """D of the kernel that a call with `call_rows` rows runs (see above)."""
    if call_rows > 64:
        return group + k // group + 2
    return group + k // group + 18


def term_bound(w, scales, zeros, bits, group, mode, call_rows):
    """Per-element weight magnitude of the bound's terms (see above)."""
    if call_rows > 64:
        return np.abs(w)
    s = np.repeat(np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64), group, 1)
    if mode == oracle.ASYM:
        z = np.repeat(np.asarray(zeros, dtype=np.uint16).view(np.float16).astype(np.float64), group, 1)
    else:
        z = float(1 << (bits - 1))
    return np.abs(w) + 2.0 * np.abs(s) * np.abs(z)


def check(got, a_bits, codes, scales, zeros, bits, group, mode, bf16_out, rows=None):
    a = inputs.bf16_bits_to_f32(a_bits).reshape(a_bits.shape).astype(np.float64)
    call_rows = a.shape[0]
    if rows is not None:
        a = a[rows]
        got = got[rows]
    w = oracle.dequantize(codes, scales, zeros, bits, group, mode, a.shape[1])
    y64 = a @ w.T
    k = a.shape[1]
    wt = term_bound(w, scales, zeros, bits, group, mode, call_rows)
    bound = rounding_depth(call_rows, k, group) * U * (np.abs(a) @ wt.T)
    if bf16_out:
        mag = np.maximum(np.abs(got), np.abs(y64))
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
        bound = bound + np.where(mag > 0, 2.0 ** (np.maximum(e, -126) - 8), 0.0)
    err = np.abs(got - y64)
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), float((err / np.maximum(bound, 1e-300)).max()))
    return float((err / np.maximum(bound, 1e-300)).max())


@pytest.mark.parametrize("bits,mode", [(2, oracle.ASYM), (2, oracle.SYM), (4, oracle.SYM),
                                       (4, oracle.ASYM)])
@pytest.mark.parametrize("y_dt", ["f32", "bf16"])
def test_small_shapes(bits, mode, y_dt):
    rng = np.random.default_rng(100 + 10 * bits + mode + (5 if y_dt == "bf16" else 0))
    # few-row kernel: 1, 2, 3-4 rows (activations staged in LDS), 5-16 and
    # more (16-row slices); one pass per wave (k up to 1024 per wave), a
    # partial last segment (k = 64, 2112), several passes (k = 11008 at
    # group 64 with eight waves); every group size
    for rows, n_out, k, group in [(1, 128, 64, 64), (37, 256, 128, 128), (300, 384, 640, 64),
                                  (257, 128, 1024, 256), (513, 256, 512, 512), (4, 384, 2112, 64),
                                  (16, 128, 1024, 512), (64, 256, 4096, 128), (65, 128, 256, 128),
                                  (2, 128, 4096, 256), (3, 256, 11008, 128), (5, 128, 16384, 64),
                                  (20, 128, 3072, 256), (1, 256, 11008, 64)]:
        a = inputs.f32_to_bf16_bits(rng.standard_normal((rows, k)).astype(np.float32) * 3)
        codes, scales, zeros = rand_codes(rng, n_out, k, bits, group, mode)
        got = run(a, codes, scales, zeros, bits, group, mode,
                  torch.float32 if y_dt == "f32" else torch.bfloat16)
        check(got, a, codes, scales, zeros, bits, group, mode, y_dt == "bf16")


def test_unit_codes_pick_columns():
    """A weight row with a single code of value 1 (scale 1) copies one
    activation column exactly; all others zero -- checks the row/column
    placement of every output tile (bit-exact)."""
    rows, n_out, k, group = 300, 256, 128, 64
    rng = np.random.default_rng(5)
    a = inputs.f32_to_bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
    pick = rng.integers(0, k, n_out)
    q = np.zeros((n_out, k), dtype=np.int64)
    q[np.arange(n_out), pick] = 1
    codes = np.zeros((n_out, k // 4), dtype=np.uint8)
    for e in range(4):
        codes |= (q[:, e::4] << (2 * e)).astype(np.uint8)
    scales = np.full((n_out, k // group), 0x3C00, dtype=np.uint16)
    got = run(a, codes, scales, None, 2, group, oracle.SYM, torch.float32)
    want = inputs.bf16_bits_to_f32(a).reshape(a.shape)[:, pick]
    assert np.array_equal(got, want.astype(np.float64))


def test_w2a16_full_size_sampled():
    """8192 rotated activation rows (bf16) x the 11008 x 4096 weight rotated
    and quantized to asym INT2 g128 by the oracle, in the configuration the
    benchmark times; rows sampled across tiles, including the last."""
    w = inputs.act_int4()
    ww = inputs.weight_int2()
    th = w["theta"]
    a = oracle.round_bf16(oracle.forward(w["x"], th))
    q = oracle.quantize(oracle.forward(ww["w2"], ww["theta"]), 2, 128, oracle.ASYM)
    got = run(a, q["codes"], q["scales"], q["zeros"], 2, 128, oracle.ASYM, torch.bfloat16)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, 8190, 8191],
                                     rng.integers(0, 8192, 41)]))
    r = check(got, a, q["codes"], q["scales"], q["zeros"], 2, 128, oracle.ASYM, True, rows=rows)
    print("w2a16 8192x4096x11008 sampled rows: max err / bound", r)
    # a 300-row slice computes the same values (tile placement is row-independent)
    part = run(a[:300], q["codes"], q["scales"], q["zeros"], 2, 128, oracle.ASYM, torch.bfloat16)
    assert np.array_equal(part, got[:300])


@pytest.mark.parametrize("rows", [1, 16])
def test_w2a16_decode_full_width(rows):
    """Few rows (decode time) against the full 11008 x 4096 asym INT2 g128
    weight, quantized by the oracle: every output."""
    ww = inputs.weight_int2()
    q = oracle.quantize(oracle.forward(ww["w2"], ww["theta"]), 2, 128, oracle.ASYM)
    rng = np.random.default_rng(11 + rows)
    a = inputs.f32_to_bf16_bits(rng.standard_normal((rows, 4096)).astype(np.float32))
    got = run(a, q["codes"], q["scales"], q["zeros"], 2, 128, oracle.ASYM, torch.bfloat16)
    check(got, a, q["codes"], q["scales"], q["zeros"], 2, 128, oracle.ASYM, True)


@pytest.mark.parametrize("rows,bits,mode,k,group",
                         [(1, 2, oracle.ASYM, 65536, 512), (300, 4, oracle.SYM, 65536, 512),
                          (16, 4, oracle.ASYM, 65536, 512), (3, 2, oracle.SYM, 16384, 128)])
def test_longest_k(rows, bits, mode, k, group):
    """k = 65536 (the largest accepted): 1024 chunks through the MFMA tiles;
    in the few-row kernel four passes per wave for one row (16 waves), eight
    for 16 rows (8 waves, activations read from memory), and several passes
    with the activations staged in LDS (3 rows, k = 16384, 8 waves)."""
    rng = np.random.default_rng(21 + rows)
    n_out = 128
    a = inputs.f32_to_bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
    codes, scales, zeros = rand_codes(rng, n_out, k, bits, group, mode)
    got = run(a, codes, scales, zeros, bits, group, mode, torch.float32)
    check(got, a, codes, scales, zeros, bits, group, mode, False)
