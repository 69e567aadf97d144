"""GPU parity: libbfly's HIP kernels against the fp64 oracle, element by
element, on seeded inputs -- small shapes spanning several tiles with ragged
tails, every edge case, and the five workloads at full size in the launch
configuration the benchmark times.  Every call goes through the C ABI."""
import math

import numpy as np
import pytest

import oracle
import learnable_butterfly_rotation_amd as B
from learnable_butterfly_rotation_amd import inputs

from parity import check_bf16, check_dtheta, check_f32, check_quant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


def dev(a: np.ndarray):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def row_norms(x: np.ndarray):
    xf = inputs.bf16_bits_to_f32(x).reshape(x.shape) if x.dtype == np.uint16 else x
    xf = xf.astype(np.float64)
    return np.abs(xf).max(axis=1), np.linalg.norm(xf, axis=1)


def rand_theta(rng, n):
    return inputs.angles(rng, n)


def run_quant(x, theta, bits, group, mode, y_dtype=torch.bfloat16, with_y=True, coeffs=False):
    rows, n = x.shape
    xd = dev(x)
    y = empty((rows, n), y_dtype) if with_y else None
    codes = torch.zeros((rows, n * bits // 8), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, n // group), dtype=torch.float16, device="cuda")
    zeros = torch.zeros((rows, n // group), dtype=torch.float16, device="cuda") if mode else None
    th = dev(theta)
    if coeffs:
        tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
        B.bfly_prepare(th, n, tab)
        B.bfly_forward_quant(xd, y, codes, scales, zeros, coeffs=tab, bits=bits, group=group,
                             mode=mode)
    else:
        B.bfly_forward_quant(xd, y, codes, scales, zeros, theta=th, bits=bits, group=group,
                             mode=mode)
    out = {"codes": host(codes), "scales": host(scales)}
    if zeros is not None:
        out["zeros"] = host(zeros)
    if y is not None:
        out["y"] = host(y)
    return out


def assert_forward(y_gpu, y64, x, n):
    xinf, xl2 = row_norms(x)
    if y_gpu.dtype == np.uint16:
        r = check_bf16(y_gpu, y64, xl2, n)
    else:
        r = check_f32(y_gpu, y64, xinf, n)
    assert r["ok"], r
    return r


def assert_quant(out, y64, bits, group, mode):
    r = check_quant(y64, out["codes"], out["scales"], out.get("zeros"), bits, group, mode)
    assert r["ok"], r
    return r


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def test_tiny_fp32_workload_full():
    w = inputs.tiny_fp32()
    x, th = w["x"], w["theta"]
    y = empty(x.shape, torch.float32)
    B.bfly_forward(dev(x), y, theta=dev(th))
    y_gpu = host(y)
    r = assert_forward(y_gpu, oracle.forward(x, th), x, 256)
    print("tiny n=256 fp32:", r)
    # a prepared table gives bit-identical results
    tab = torch.empty(B.bfly_coeff_bytes(256), dtype=torch.uint8, device="cuda")
    B.bfly_prepare(dev(th), 256, tab)
    y2 = empty(x.shape, torch.float32)
    B.bfly_forward(dev(x), y2, coeffs=tab)
    assert np.array_equal(host(y2), y_gpu)


@pytest.mark.parametrize("n", [64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("x_dt,y_dt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
                                       ("f32", "bf16")])
def test_forward_sizes_and_dtypes(n, x_dt, y_dt):
    rng = np.random.default_rng(1000 + n)
    th = rand_theta(rng, n)
    for rows in (1, 37, 301):
        xf = (rng.standard_normal((rows, n)) * 3).astype(np.float32)
        x = inputs.f32_to_bf16_bits(xf) if x_dt == "bf16" else xf
        y = empty((rows, n), torch.bfloat16 if y_dt == "bf16" else torch.float32)
        B.bfly_forward(dev(x), y, theta=dev(th))
        assert_forward(host(y), oracle.forward(x, th), x, n)


@pytest.mark.parametrize("n", [64, 256, 1024, 4096])
@pytest.mark.parametrize("bits,mode", [(4, 0), (2, 1), (4, 1), (2, 0)])
def test_forward_quant_modes(n, bits, mode):
    rng = np.random.default_rng(7 * n + bits + 10 * mode)
    th = rand_theta(rng, n)
    for group in sorted(g for g in {8, 32, 128, 512, n} if g <= min(n, 512)):
        rows = 67
        xf = (rng.standard_normal((rows, n)) * np.exp(rng.uniform(-4, 4, (rows, 1)))).astype(np.float32)
        x = inputs.f32_to_bf16_bits(xf)
        out = run_quant(x, th, bits, group, mode)
        y64 = oracle.forward(x, th)
        assert_forward(out["y"], y64, x, n)
        assert_quant(out, y64, bits, group, mode)


def test_act_int4_workload_full():
    """n=4096, 8192 bf16 rows with outlier channels, sym INT4 g128: all rows."""
    w = inputs.act_int4()
    x, th = w["x"], w["theta"]
    out = run_quant(x, th, 4, 128, 0)
    y64 = oracle.forward(x, th)
    rf = assert_forward(out["y"], y64, x, 4096)
    rq = assert_quant(out, y64, 4, 128, 0)
    print("act n=4096 bf16 int4:", rf, rq)
    # deterministic, independent of the prepared/unprepared path and of the
    # batch a row is computed in
    again = run_quant(x, th, 4, 128, 0, coeffs=True)
    for k in out:
        assert np.array_equal(out[k], again[k]), k
    part = run_quant(x[:37], th, 4, 128, 0)
    for k in out:
        assert np.array_equal(out[k][:37], part[k]), k


def test_weight_int2_workload_full():
    """W Q^T for 4096x4096 and 11008x4096 bf16 weights, asym INT2 g128."""
    w = inputs.weight_int2()
    for name in ("w1", "w2"):
        x = w[name]
        out = run_quant(x, w["theta"], 2, 128, 1)
        y64 = oracle.forward(x, w["theta"])
        rf = assert_forward(out["y"], y64, x, 4096)
        rq = assert_quant(out, y64, 2, 128, 1)
        print("weight", name, rf, rq)
        codes_only = run_quant(x, w["theta"], 2, 128, 1, with_y=False)
        for k in ("codes", "scales", "zeros"):
            assert np.array_equal(out[k], codes_only[k]), k


def test_computational_invariance_on_gpu():
    """(W Q^T)(Q x) = W x with both rotations computed by the library (fp32)."""
    rng = np.random.default_rng(5)
    n = 1024
    th = rand_theta(rng, n)
    w = rng.standard_normal((96, n)).astype(np.float32)
    x = rng.standard_normal((33, n)).astype(np.float32)
    wq = empty(w.shape, torch.float32)
    qx = empty(x.shape, torch.float32)
    B.bfly_forward(dev(w), wq, theta=dev(th))
    B.bfly_forward(dev(x), qx, theta=dev(th))
    lhs = host(qx).astype(np.float64) @ host(wq).astype(np.float64).T
    rhs = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(lhs - rhs).max() <= 1e-5 * math.log2(n) * np.abs(rhs).max()


# ---------------------------------------------------------------------------
# Kronecker composite
# ---------------------------------------------------------------------------

def run_kron(x, th, mix, quant=True, bits=4, group=128, mode=0):
    rows, n = x.shape
    y = empty((rows, n), torch.bfloat16)
    args = {}
    if quant:
        args = dict(codes=torch.zeros((rows, n * bits // 8), dtype=torch.uint8, device="cuda"),
                    scales=torch.zeros((rows, n // group), dtype=torch.float16, device="cuda"),
                    zeros=torch.zeros((rows, n // group), dtype=torch.float16, device="cuda")
                    if mode else None)
    B.bfly_kron_forward(dev(x), y, dev(mix), theta_b=dev(th), bits=bits, group=group, mode=mode,
                        **args)
    out = {"y": host(y)}
    if quant:
        out["codes"] = host(args["codes"])
        out["scales"] = host(args["scales"])
        if mode:
            out["zeros"] = host(args["zeros"])
    return out


def test_kron_workload_full():
    """n=5120 = O5 (x) B1024, 8192 bf16 rows with outliers, sym INT4 g128."""
    w = inputs.kron_int4()
    x = w["x"]
    out = run_kron(x, w["theta_b"], w["mix"])
    y64 = oracle.kron_forward(x, w["theta_b"], w["mix"])
    rf = assert_forward(out["y"], y64, x, 5120)
    rq = assert_quant(out, y64, 4, 128, 0)
    print("kron n=5120:", rf, rq)


@pytest.mark.parametrize("m,nb", [(m, nb) for m in (1, 2, 3, 5, 8) for nb in (256, 1024)] +
                         [(2, 2048), (3, 2048), (2, 4096)])
def test_kron_shapes(m, nb):
    rng = np.random.default_rng(100 * m + nb)
    th = rand_theta(rng, nb)
    mix = inputs.mixing_factor(rng, m)
    rows = 45
    x = inputs.f32_to_bf16_bits(rng.standard_normal((rows, m * nb)).astype(np.float32))
    for quant, mode in ((False, 0), (True, 0), (True, 1)):
        out = run_kron(x, th, mix, quant=quant, bits=4, group=64, mode=mode)
        y64 = oracle.kron_forward(x, th, mix)
        assert_forward(out["y"], y64, x, m * nb)
        if quant:
            assert_quant(out, y64, 4, 64, mode)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def test_rows_zero_is_noop():
    y = torch.full((4, 256), 7.0, device="cuda")
    x = torch.zeros((0, 256), device="cuda")
    B.bfly_forward(x, y[:0], theta=dev(np.zeros((8, 128), np.float32)))
    assert (host(y) == 7.0).all()


def test_in_place():
    rng = np.random.default_rng(3)
    th = rand_theta(rng, 1024)
    x = rng.standard_normal((50, 1024)).astype(np.float32)
    xd = dev(x)
    B.bfly_forward(xd, xd, theta=dev(th))
    assert_forward(host(xd), oracle.forward(x, th), x, 1024)


def _right_angles(rng, n):
    """Angles of exactly +-pi/2 (as fp32) on every pair: the table then marks
    the scaled form unusable and the forward runs the three-shear form."""
    L = int(math.log2(n))
    return np.where(rng.random((L, n // 2)) < 0.5, np.float32(math.pi / 2),
                    np.float32(-math.pi / 2)).astype(np.float32)


@pytest.mark.parametrize("n", [256, 1024, 4096])
def test_in_place_three_shear_form(n):
    """y == x with the three-shear fallback: the kernel decides on the form
    after its first row group, so no output of that group may reach memory
    before the fallback re-reads the group's input (fp32 forward, and bf16
    rows with INT4 codes).  Three stages of exact right angles put the table
    on the fallback; the other stages' angles are uniform, so that the rows
    are genuinely rotated (all right angles would only permute bf16 values,
    piling the codes' pre-round values onto rounding boundaries)."""
    rng = np.random.default_rng(90 + n)
    L = int(math.log2(n))
    th = inputs.angles(rng, n)
    right = _right_angles(rng, n)
    for s in (0, 1, 2):   # scales shrink by ~4e-8 per such stage: below 2^-64 after three
        th[s] = right[s]
    assert not _table_uses_scaled_form(th, n)
    # more row groups than workgroups, so every workgroup's first group is in play
    rows = 3 * 256 * max(1, 256 // (n // 8)) + 29
    x = rng.standard_normal((rows, n)).astype(np.float32)
    xd = dev(x)
    B.bfly_forward(xd, xd, theta=dev(th))
    assert_forward(host(xd), oracle.forward(x, th), x, n)

    xb = inputs.f32_to_bf16_bits(x)
    xbd = dev(xb)
    codes = torch.zeros((rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
    B.bfly_forward_quant(xbd, xbd, codes, scales, theta=dev(th), bits=4, group=128, mode=0)
    y64 = oracle.forward(xb, th)
    assert_forward(host(xbd), y64, xb, n)
    assert_quant({"codes": host(codes), "scales": host(scales)}, y64, 4, 128, 0)


def test_timed_forward_launch_is_the_same_kernel():
    # events attached to the dispatch: same outputs bit for bit, a positive
    # kernel time, and the arming is consumed by that one launch
    rng = np.random.default_rng(11)
    n, rows = 4096, 512
    th = dev(rand_theta(rng, n))
    x = dev(inputs.f32_to_bf16_bits(rng.standard_normal((rows, n)).astype(np.float32)))
    tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    B.bfly_prepare(th, n, tab)
    outs = []
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for armed in (False, True, False):
        y = empty((rows, n), torch.bfloat16)
        codes = torch.zeros((rows, n // 2), dtype=torch.uint8, device="cuda")
        scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
        if armed:
            ev[0].record()
            ev[1].record()
            torch.cuda.synchronize()
            B.bfly_time_next_forward(ev[0].cuda_event, ev[1].cuda_event)
        B.bfly_forward_quant(x, y, codes, scales, coeffs=tab, bits=4, group=128, mode=0)
        torch.cuda.synchronize()
        if armed:
            ms = ev[0].elapsed_time(ev[1])
            assert 0.0 < ms < 100.0, ms
        outs.append((host(y), host(codes), host(scales)))
    assert ev[0].elapsed_time(ev[1]) == ms  # the later launch left the events alone
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    for a, b in zip(outs[0], outs[2]):
        assert np.array_equal(a, b)


def _fq(x, th, ws=None, coeffs=None, noalloc=False):
    rows, n = x.shape
    y = empty((rows, n), torch.bfloat16)
    codes = torch.zeros((rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
    if noalloc:
        B.bfly_forward_quant_noalloc(x, y, codes, scales, theta=th, bits=4, group=128, mode=0)
    elif coeffs is not None:
        B.bfly_forward_quant(x, y, codes, scales, coeffs=coeffs, bits=4, group=128, mode=0)
    else:
        B.bfly_forward_quant(x, y, codes, scales, theta=th, bits=4, group=128, mode=0,
                             workspace=ws)
    return y, codes, scales


@pytest.mark.parametrize("n,rows", [(4096, 512), (4096, 383), (1024, 640), (256, 300)])
def test_forward_from_angles_with_a_reused_workspace(n, rows):
    """From angles, the call prepares its table into the caller's workspace.
    One workspace, whatever it held before (zeros, ones, an earlier call's
    table), serves calls with different angles in turn; each matches the
    call on the table bfly_prepare made, bit for bit (and so does the entry
    point without allocation), and the oracle."""
    rng = np.random.default_rng(4000 + n + rows)
    x = dev(inputs.f32_to_bf16_bits(rng.standard_normal((rows, n)).astype(np.float32)))
    thetas = [dev(rand_theta(rng, n)) for _ in range(2)]
    refs = []
    for th in thetas:
        tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
        B.bfly_prepare(th, n, tab)
        refs.append([host(t) for t in _fq(x, th, coeffs=tab)])
    ws = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    for fill in (0, 255):
        ws.fill_(fill)
        for k in (0, 1, 0, 0, 1):
            got = [host(t) for t in _fq(x, thetas[k], ws=ws)]
            for a, b in zip(got, refs[k]):
                assert np.array_equal(a, b), (fill, k)
    got = [host(t) for t in _fq(x, thetas[1], noalloc=True)]
    for a, b in zip(got, refs[1]):
        assert np.array_equal(a, b)
    th64 = host(thetas[0])
    xb = host(x)
    y64 = oracle.forward(xb, th64)
    assert_forward(refs[0][0], y64, xb, n)


def test_forward_from_angles_under_stream_capture():
    """A captured forward from angles (the prepare kernel, then the fused
    kernel) is replayed with the angles changed in place between replays,
    with eager work and synchronisations in between; every replay matches
    the eager call with those angles.  Both the workspace entry point and
    the one without allocation are captured."""
    rng = np.random.default_rng(4100)
    n, rows = 4096, 512
    x = dev(inputs.f32_to_bf16_bits(rng.standard_normal((rows, n)).astype(np.float32)))
    th = dev(rand_theta(rng, n))
    ws = torch.zeros(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    y = empty((rows, n), torch.bfloat16)
    codes = torch.zeros((rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
    for noalloc in (False, True):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # warm-up outside the capture
            if noalloc:
                B.bfly_forward_quant_noalloc(x, y, codes, scales, theta=th, bits=4, group=128,
                                             mode=0)
            else:
                B.bfly_forward_quant(x, y, codes, scales, theta=th, bits=4, group=128, mode=0,
                                     workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            if noalloc:
                B.bfly_forward_quant_noalloc(x, y, codes, scales, theta=th, bits=4, group=128,
                                             mode=0)
            else:
                B.bfly_forward_quant(x, y, codes, scales, theta=th, bits=4, group=128, mode=0,
                                     workspace=ws)
        for rep in range(4):
            th.copy_(dev(rand_theta(rng, n)))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (host(y), host(codes), host(scales))
            tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
            B.bfly_prepare(th, n, tab)
            want = [host(t) for t in _fq(x, th, coeffs=tab)]
            for a, b in zip(got, want):
                assert np.array_equal(a, b), (noalloc, rep)
        del g


# ---------------------------------------------------------------------------
# n = 8192: two passes (stages 0..11 on each half, then stage 12 with the
# output and the quantizer)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows", [1, 37, 300])
@pytest.mark.parametrize("x_dt,y_dt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_forward_8192(rows, x_dt, y_dt):
    """Every row against the oracle; the call from angles and the call on the
    table bfly_prepare made agree bit for bit."""
    rng = np.random.default_rng(5000 + rows)
    n = 8192
    th = rand_theta(rng, n)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, x_dt)
    tdt = torch.float32 if y_dt == "f32" else torch.bfloat16
    y = empty((rows, n), tdt)
    B.bfly_forward(dev(x), y, theta=dev(th))
    got = host(y)
    y64 = oracle.forward(x, th)
    print("n=8192 forward", x_dt, y_dt, rows, assert_forward(got, y64, x, n))
    tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    B.bfly_prepare(dev(th), n, tab)
    y2 = empty((rows, n), tdt)
    B.bfly_forward(dev(x), y2, coeffs=tab)
    assert np.array_equal(got, host(y2))


@pytest.mark.parametrize("bits,group,mode", [(4, 128, 0), (2, 128, 1), (4, 8, 1), (2, 512, 0),
                                             (4, 64, 0)])
def test_forward_quant_8192(bits, group, mode):
    rng = np.random.default_rng(5100 + bits * 1000 + group + mode)
    n, rows = 8192, 301
    th = rand_theta(rng, n)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, "bf16")
    out = run_quant(x, th, bits, group, mode)
    y64 = oracle.forward(x, th)
    rf = assert_forward(out["y"], y64, x, n)
    rq = assert_quant(out, y64, bits, group, mode)
    print("n=8192 quant", bits, group, mode, rf, rq)
    codes_only = run_quant(x, th, bits, group, mode, with_y=False)
    for k in codes_only:
        assert np.array_equal(codes_only[k], out[k]), k


def test_forward_quant_8192_batch():
    """2048 bf16 rows of n = 8192 with outlier channels, sym INT4 g128: every
    row, element by element (the headline's format at twice the width)."""
    rng = np.random.default_rng(5200)
    n, rows = 8192, 2048
    th = rand_theta(rng, n)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, "bf16")
    out = run_quant(x, th, 4, 128, 0)
    y64 = oracle.forward(x, th)
    print("n=8192 batch:", assert_forward(out["y"], y64, x, n), assert_quant(out, y64, 4, 128, 0))
    part = run_quant(x[:5], th, 4, 128, 0)
    for k in part:
        assert np.array_equal(out[k][:5], part[k]), k


def test_forward_8192_in_place_and_hadamard():
    rng = np.random.default_rng(5300)
    n, rows = 8192, 64
    th = rand_theta(rng, n)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    xd = dev(x)
    B.bfly_forward(xd, xd, theta=dev(th))
    assert_forward(host(xd), oracle.forward(x, th), x, n)
    # H_8192 from its table: the halves' tables start with the diagonal's
    # signs, the last stage is pi/4 from exact constants
    tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    B.bfly_prepare_hadamard(n, tab)
    xs = x[:8]
    y = empty((8, n), torch.float32)
    B.bfly_forward(dev(xs), y, coeffs=tab)
    assert_forward(host(y), oracle.hadamard(xs), xs, n)


def test_zero_angles_identity_bit_exact():
    rng = np.random.default_rng(4)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((20, 512)).astype(np.float32))
    y = empty((20, 512), torch.bfloat16)
    B.bfly_forward(dev(x), y, theta=dev(np.zeros((9, 256), np.float32)))
    assert np.array_equal(host(y), x)


def test_quarter_pi_is_hadamard():
    n = 256
    th = np.full((8, 128), math.pi / 4, dtype=np.float32)
    h = np.array([[1.0]])
    for _ in range(8):
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    h /= math.sqrt(n)
    d = np.array([(-1.0) ** bin(i).count("1") for i in range(n)])
    rng = np.random.default_rng(9)
    x = rng.standard_normal((16, n)).astype(np.float32)
    y = empty(x.shape, torch.float32)
    B.bfly_forward(dev(x), y, theta=dev(th))
    want = (x.astype(np.float64) * d) @ h.T
    assert np.abs(host(y) - want).max() < 1e-5


# ---------------------------------------------------------------------------
# the Hadamard special case: table of H_n = Q(pi/4) D from exact constants
# ---------------------------------------------------------------------------

def hadamard_table(n):
    tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    B.bfly_prepare_hadamard(n, tab)
    return tab


def _scaled_block(tab, n):
    L, half = int(math.log2(n)), n // 2
    raw = tab.cpu().numpy()
    return raw[half * 8 * L: half * 8 * (2 * L - 1)].view(np.float32)


@pytest.mark.parametrize("n", [64, 128, 256, 512, 1024, 2048, 4096])
def test_hadamard_forward(n):
    rng = np.random.default_rng(2000 + n)
    tab = hadamard_table(n)
    assert not np.isnan(_scaled_block(tab, n)).any()
    for rows in (1, 37, 301):
        xf = (rng.standard_normal((rows, n)) * 3).astype(np.float32)
        y = empty((rows, n), torch.float32)
        B.bfly_forward(dev(xf), y, coeffs=tab)
        assert_forward(host(y), oracle.hadamard(xf), xf, n)
        xb = inputs.f32_to_bf16_bits(xf)
        yb = empty((rows, n), torch.bfloat16)
        B.bfly_forward(dev(xb), yb, coeffs=tab)
        assert_forward(host(yb), oracle.hadamard(xb), xb, n)


def test_hadamard_closed_forms_on_gpu():
    """H e_0 = 1/sqrt(n) everywhere; H applied twice is the identity."""
    n = 1024
    tab = hadamard_table(n)
    e = torch.zeros((1, n), device="cuda")
    e[0, 0] = 1.0
    y = empty((1, n), torch.float32)
    B.bfly_forward(e, y, coeffs=tab)
    assert np.abs(host(y) - 1 / 32).max() < 1e-7
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, n)).astype(np.float32)
    y1 = empty(x.shape, torch.float32)
    y2 = empty(x.shape, torch.float32)
    B.bfly_forward(dev(x), y1, coeffs=tab)
    B.bfly_forward(y1, y2, coeffs=tab)
    assert np.abs(host(y2) - x).max() < 1e-5 * math.log2(n) * np.abs(x).max()


def test_hadamard_act_int4_workload_full():
    """H_4096 fused with sym INT4 g128 on the 8192-row bf16 activation batch
    with outlier channels (the learned rotation's workload, angles fixed)."""
    w = inputs.act_int4()
    x = w["x"]
    rows, n = x.shape
    tab = hadamard_table(n)
    y = empty((rows, n), torch.bfloat16)
    codes = torch.zeros((rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
    B.bfly_forward_quant(dev(x), y, codes, scales, coeffs=tab, bits=4, group=128, mode=0)
    out = {"y": host(y), "codes": host(codes), "scales": host(scales)}
    y64 = oracle.hadamard(x)
    rf = assert_forward(out["y"], y64, x, n)
    rq = assert_quant(out, y64, 4, 128, 0)
    print("hadamard n=4096 bf16 int4:", rf, rq)


@pytest.mark.parametrize("bits,mode", [(2, 1), (4, 1), (2, 0)])
def test_hadamard_quant_modes(bits, mode):
    rng = np.random.default_rng(40 + bits + 10 * mode)
    for n in (256, 4096):
        tab = hadamard_table(n)
        rows = 67
        xf = (rng.standard_normal((rows, n)) * np.exp(rng.uniform(-4, 4, (rows, 1)))).astype(np.float32)
        x = inputs.f32_to_bf16_bits(xf)
        y = empty((rows, n), torch.bfloat16)
        codes = torch.zeros((rows, n * bits // 8), dtype=torch.uint8, device="cuda")
        scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
        zeros = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda") if mode else None
        B.bfly_forward_quant(dev(x), y, codes, scales, zeros, coeffs=tab, bits=bits, group=128,
                             mode=mode)
        out = {"y": host(y), "codes": host(codes), "scales": host(scales)}
        if mode:
            out["zeros"] = host(zeros)
        y64 = oracle.hadamard(x)
        assert_forward(out["y"], y64, x, n)
        assert_quant(out, y64, bits, 128, mode)


@pytest.mark.parametrize("m,nb", [(5, 1024), (3, 256), (2, 4096)])
def test_kron_hadamard(m, nb):
    """(O kron H_nb) with the Hadamard table as the butterfly factor."""
    rng = np.random.default_rng(3000 + 10 * m + nb)
    mix = inputs.mixing_factor(rng, m)
    rows = 301
    x = inputs.f32_to_bf16_bits(rng.standard_normal((rows, m * nb)).astype(np.float32))
    n = m * nb
    tab = hadamard_table(nb)
    y = empty((rows, n), torch.bfloat16)
    codes = torch.zeros((rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, n // 128), dtype=torch.float16, device="cuda")
    B.bfly_kron_forward(dev(x), y, dev(mix), codes=codes, scales=scales, coeffs_b=tab, bits=4,
                        group=128, mode=0)
    out = {"y": host(y), "codes": host(codes), "scales": host(scales)}
    y64 = oracle.kron_hadamard(x, mix)
    assert_forward(out["y"], y64, x, n)
    assert_quant(out, y64, 4, 128, 0)


def _table_uses_scaled_form(theta, n):
    """Whether the prepared table keeps the scaled (two-FMA) rotation form.
    Reads the (beta, gamma) part of the table's scaled-form block (after the
    (cos, sin) block; (log2 n - 1) x n/2 float2, in the forward kernel's
    thread order) and looks for the NaN marker."""
    L, half = int(math.log2(n)), n // 2
    tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
    B.bfly_prepare(dev(theta), n, tab)
    raw = tab.cpu().numpy()
    fg = raw[half * 8 * L: half * 8 * (2 * L - 1)].view(np.float32)
    return not np.isnan(fg).any()


@pytest.mark.parametrize("n", [128, 256, 4096])
def test_three_shear_form_for_right_angles(n):
    """Angles of exactly +-pi/2 (as fp32) on every pair: the scaled form's
    scales would shrink by ~4e-8 per stage, so the table falls back to the
    three-shear form; results must still match the oracle."""
    L = int(math.log2(n))
    rng = np.random.default_rng(70 + n)
    th = np.where(rng.random((L, n // 2)) < 0.5, np.float32(math.pi / 2),
                  np.float32(-math.pi / 2)).astype(np.float32)
    assert not _table_uses_scaled_form(th, n)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((45, n)).astype(np.float32))
    out = run_quant(x, th, 4, 128, 0)
    y64 = oracle.forward(x, th)
    assert_forward(out["y"], y64, x, n)
    assert_quant(out, y64, 4, 128, 0)
    xf = rng.standard_normal((33, n)).astype(np.float32)
    y = empty(xf.shape, torch.float32)
    B.bfly_forward(dev(xf), y, theta=dev(th))
    assert_forward(host(y), oracle.forward(xf, th), xf, n)


@pytest.mark.parametrize("n", [128, 256, 1024, 4096])
def test_scaled_form_with_near_right_angles(n):
    """Three stages of angles 1e-3..3e-3 away from +-pi/2 (scales shrink by
    ~1e-3 per such stage, still in range), on register and lane-mapped bits
    of the forward's two phases: the scaled form stays in use, with
    coefficients up to ~1e3 times larger; results must match the oracle."""
    L = int(math.log2(n))
    rng = np.random.default_rng(80 + n)
    th = inputs.angles(rng, n)
    for s in sorted({0, 4, L - 3}):
        off = rng.uniform(1e-3, 3e-3, n // 2) * np.sign(rng.standard_normal(n // 2))
        th[s] = (np.sign(rng.standard_normal(n // 2)) * (math.pi / 2) + off).astype(np.float32)
    assert _table_uses_scaled_form(th, n)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((45, n)).astype(np.float32))
    out = run_quant(x, th, 4, 128, 0)
    y64 = oracle.forward(x, th)
    assert_forward(out["y"], y64, x, n)
    assert_quant(out, y64, 4, 128, 0)
    out = run_quant(x, th, 2, 128, 1)
    assert_quant(out, y64, 2, 128, 1)
    xf = rng.standard_normal((33, n)).astype(np.float32)
    y = empty(xf.shape, torch.float32)
    B.bfly_forward(dev(xf), y, theta=dev(th))
    assert_forward(host(y), oracle.forward(xf, th), xf, n)


def test_degenerate_groups():
    """All-zero rows (scale 0 -> codes 0), constant rows in asym mode, and
    values so large that the fp16 scale saturates."""
    n = 256
    th = np.zeros((8, 128), np.float32)  # identity: groups keep their shape
    x = np.zeros((3, n), np.float32)
    x[1] = 3.0
    x[2, ::2] = 1e9
    x[2, 1::2] = -1e9
    for bits, mode in ((4, 0), (2, 1)):
        out = run_quant(x, th, bits, 32, mode, y_dtype=torch.float32)
        y64 = oracle.forward(x, th)
        assert_quant(out, y64, bits, 32, mode)
        assert not out["codes"][0].any() and not out["scales"][0].any()
        assert (out["scales"][2] == 0x7BFF).all()


@pytest.mark.parametrize("n", [256, 4096])
def test_fixed_formats_scale_edges(n):
    """The fixed formats (sym INT4 and asym INT2, groups of 128, bf16 rows)
    skip the code clamp in waves where no group's fp16 scale lost precision.
    Groups here have fp16-subnormal scales (codes that must saturate), a
    saturated scale, zero, or ordinary values, side by side in some rows;
    the last two rows hold only ordinary groups."""
    rng = np.random.default_rng(70 + n)
    L = int(math.log2(n))
    th = np.zeros((L, n // 2), np.float32)  # identity: each group keeps its values
    rows, ng = 6, n // 128
    x = rng.standard_normal((rows, n)).astype(np.float32)
    tiny = 2.0 ** -24  # fp16's smallest subnormal
    for r in range(rows - 2):
        for gi in range(ng):
            grp = x[r, gi * 128:(gi + 1) * 128]
            kind = (r + gi) % 4
            if kind == 1:  # max|y| / 7 between 0.4 and 3 subnormal steps
                grp *= rng.uniform(3.0, 20.0) * tiny / np.abs(grp).max()
            elif kind == 2:
                grp *= 1e9 / np.abs(grp).max()
            elif kind == 3:
                grp[:] = 0.0
    xb = inputs.f32_to_bf16_bits(x)
    y64 = oracle.forward(xb, th)
    for bits, mode in ((4, 0), (2, 1)):
        out = run_quant(xb, th, bits, 128, mode)
        assert_forward(out["y"], y64, xb, n)
        assert_quant(out, y64, bits, 128, mode)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def run_backward(x, g, th, with_y=True, coeffs=False):
    rows, n = x.shape
    ws = torch.empty(B.bfly_backward_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    y = empty((rows, n), torch.float32) if with_y else None
    dx = empty((rows, n), torch.float32)
    dth = torch.full(th.shape, float("nan"), device="cuda")
    if coeffs:
        tab = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
        B.bfly_prepare(dev(th), n, tab)
        B.bfly_backward(dev(x), dev(g), y, dx, dth, ws, coeffs=tab)
    else:
        B.bfly_backward(dev(x), dev(g), y, dx, dth, ws, theta=dev(th))
    return {"y": host(y) if with_y else None, "dx": host(dx), "dtheta": host(dth)}


@pytest.mark.parametrize("n", [64, 256, 1024, 4096])
def test_backward_small(n):
    rng = np.random.default_rng(50 + n)
    th = rand_theta(rng, n)
    for rows in (1, 29, 515):
        x = (rng.standard_normal((rows, n)) * 2).astype(np.float32)
        g = rng.standard_normal((rows, n)).astype(np.float32)
        out = run_backward(x, g, th)
        ref = oracle.backward(x, g, th)
        assert check_f32(out["y"], ref["y"], np.abs(x).max(1), n)["ok"]
        assert check_f32(out["dx"], ref["dx"], np.abs(g).max(1), n)["ok"]
        r = check_dtheta(out["dtheta"], ref["dtheta"], ref["dabs"], n)
        assert r["ok"], r
    again = run_backward(x, g, th, with_y=False, coeffs=True)
    assert np.array_equal(again["dtheta"], out["dtheta"])
    assert np.array_equal(again["dx"], out["dx"])


def test_backward_rows_zero_zeroes_dtheta():
    n = 256
    out = run_backward(np.zeros((0, n), np.float32), np.zeros((0, n), np.float32),
                       np.ones((8, 128), np.float32))
    assert (out["dtheta"] == 0).all()


def test_backward_invariant_g_equals_y():
    """G = Y: the loss does not depend on theta, so dtheta ~ 0 relative to the
    term magnitudes, and dX = X."""
    rng = np.random.default_rng(11)
    n = 1024
    th = rand_theta(rng, n)
    x = rng.standard_normal((200, n)).astype(np.float32)
    g = oracle.forward(x, th).astype(np.float32)
    out = run_backward(x, g, th)
    ref = oracle.backward(x, g, th)
    assert np.abs(out["dtheta"]).max() <= 1e-5 * math.log2(n) * ref["dabs"].max()
    assert np.abs(out["dx"] - x).max() <= 1e-5 * math.log2(n) * np.abs(x).max()


@pytest.mark.timeout(900)
def test_calibration_workload_full():
    """262144 x 4096 fp32 forward + backward; dtheta over all rows against the
    oracle (streamed by blocks), Y and dX on sampled blocks."""
    c = inputs.CalibFP32()
    n = c.n
    X = torch.empty((c.rows, n), dtype=torch.float32, device="cuda")
    G = torch.empty((c.rows, n), dtype=torch.float32, device="cuda")
    d64 = np.zeros(c.theta.shape)
    dabs = np.zeros(c.theta.shape)
    sampled = {0, c.nblocks // 2, c.nblocks - 1}
    keep = {}
    for r0, x, g in c.blocks(threads=8):
        X[r0:r0 + x.shape[0]].copy_(torch.from_numpy(x))
        G[r0:r0 + x.shape[0]].copy_(torch.from_numpy(g))
        k = r0 // c.BLOCK
        want = k in sampled
        ref = oracle.backward(x, g, c.theta, want_y=want, want_dx=want)
        d64 += ref["dtheta"]
        dabs += ref["dabs"]
        if want:
            keep[k] = (r0, x, g, ref["y"], ref["dx"])
    ws = torch.empty(B.bfly_backward_workspace_bytes(c.rows, n), dtype=torch.uint8, device="cuda")
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    dth = torch.empty(c.theta.shape, dtype=torch.float32, device="cuda")
    B.bfly_backward(X, G, Y, dX, dth, ws, theta=dev(c.theta))
    r = check_dtheta(host(dth), d64, dabs, n)
    print("calib dtheta:", r)
    assert r["ok"], r
    for k, (r0, x, g, y64, dx64) in keep.items():
        m = x.shape[0]
        assert check_f32(host(Y[r0:r0 + m]), y64, np.abs(x).max(1), n)["ok"]
        assert check_f32(host(dX[r0:r0 + m]), dx64, np.abs(g).max(1), n)["ok"]


# ---------------------------------------------------------------------------
# Kronecker backward
# ---------------------------------------------------------------------------

# m <= 5 out of place: one pass (the O^T mix formed in the backward's loads);
# in place and m > 5: the mixing pass, then the backward.  Both give the same bits.
@pytest.mark.parametrize("m,nb,rows", [(5, 1024, 37), (2, 256, 300), (3, 2048, 9), (8, 1024, 64),
                                       (43, 256, 21), (9, 512, 40), (16, 1024, 7), (64, 256, 5),
                                       (4, 512, 50), (2, 4096, 11), (5, 256, 3), (3, 1024, 1)])
def test_kron_backward(m, nb, rows):
    rng = np.random.default_rng(5000 + 10 * m + nb + rows)
    th = rand_theta(rng, nb)
    mix = inputs.mixing_factor(rng, m)
    n = m * nb
    x = rng.standard_normal((rows, n)).astype(np.float32)
    g = rng.standard_normal((rows, n)).astype(np.float32)
    ref = oracle.kron_backward(x, g, th, mix)
    xd, gd = dev(x), dev(g)
    dx = empty((rows, n), torch.float32)
    dth = empty(th.shape, torch.float32)
    ws = torch.empty(B.bfly_kron_backward_workspace_bytes(rows, m, nb), dtype=torch.uint8,
                     device="cuda")
    B.bfly_kron_backward(xd, gd, dx, dth, dev(mix), ws, theta_b=dev(th))
    # dx against the fp32 bound with x := G: 1e-5 * ||g_r||_inf * log2(m nb)
    r = check_f32(host(dx), ref["dx"], np.abs(g).max(axis=1), n)
    assert r["ok"], r
    r = check_dtheta(host(dth), ref["dtheta"], ref["dabs"], nb)
    assert r["ok"], r
    # in place on g gives the same bits, dx and dtheta; a second call (same
    # workspace) too
    dth1 = host(dth)
    B.bfly_kron_backward(xd, gd, gd, dth, dev(mix), ws, theta_b=dev(th))
    assert np.array_equal(host(gd), host(dx))
    assert np.array_equal(host(dth), dth1)


@pytest.mark.timeout(900)
def test_kron_backward_workload_full():
    """The Kronecker backward at its benchmark shape and call: 32768 fp32 rows
    of n = 5120 = O5 (x) B1024 (the composite's theta_b and O5 from its seed),
    x and G ~ N(0, 1) drawn by blocks of 2048 rows; the one-pass kernel.
    dtheta_b over all rows against the oracle (summed block by block), dX on
    three sampled blocks."""
    w = inputs.kron_int4(rows=16)
    th, mix = w["theta_b"], w["mix"]
    rows, m, nb, blk = 32768, 5, 1024, 2048
    n = m * nb
    X = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    G = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    d64 = np.zeros(th.shape)
    dabs = np.zeros(th.shape)
    sampled = {0, rows // blk // 2, rows // blk - 1}
    keep = {}
    for k in range(rows // blk):
        rng = np.random.default_rng(71000 + k)
        x = rng.standard_normal((blk, n)).astype(np.float32)
        g = rng.standard_normal((blk, n)).astype(np.float32)
        X[k * blk:(k + 1) * blk].copy_(torch.from_numpy(x))
        G[k * blk:(k + 1) * blk].copy_(torch.from_numpy(g))
        ref = oracle.kron_backward(x, g, th, mix)
        d64 += ref["dtheta"]
        dabs += ref["dabs"]
        if k in sampled:
            keep[k] = (np.abs(g).max(axis=1), ref["dx"])
    ws = torch.empty(B.bfly_kron_backward_workspace_bytes(rows, m, nb), dtype=torch.uint8,
                     device="cuda")
    dX = torch.empty_like(X)
    dth = torch.empty(th.shape, dtype=torch.float32, device="cuda")
    B.bfly_kron_backward(X, G, dX, dth, dev(mix), ws, theta_b=dev(th))
    r = check_dtheta(host(dth), d64, dabs, nb)
    print("kron backward dtheta:", r)
    assert r["ok"], r
    for k, (gmax, dx64) in keep.items():
        r = check_f32(host(dX[k * blk:(k + 1) * blk]), dx64, gmax, n)
        assert r["ok"], (k, r)


# ---------------------------------------------------------------------------
# wide Kronecker composites (m up to 64): mix pass, then the fused butterfly
# ---------------------------------------------------------------------------

def run_kron_wide(x, th, mix, quant=True, bits=4, group=128, mode=0, y_dtype=torch.bfloat16,
                  coeffs=False, with_y=True):
    rows, n = x.shape
    m = mix.shape[0]
    y = empty((rows, n), y_dtype) if with_y else None
    ws = torch.empty(B.bfly_kron_forward_wide_workspace_bytes(rows, m, n // m), dtype=torch.uint8,
                     device="cuda")
    args = {}
    if quant:
        args = dict(codes=torch.zeros((rows, n * bits // 8), dtype=torch.uint8, device="cuda"),
                    scales=torch.zeros((rows, n // group), dtype=torch.float16, device="cuda"),
                    zeros=torch.zeros((rows, n // group), dtype=torch.float16, device="cuda")
                    if mode else None)
    if coeffs:
        tab = torch.empty(B.bfly_coeff_bytes(n // m), dtype=torch.uint8, device="cuda")
        B.bfly_prepare(dev(th), n // m, tab)
        args["coeffs_b"] = tab
    else:
        args["theta_b"] = dev(th)
    B.bfly_kron_forward_wide(dev(x), y, dev(mix), ws, bits=bits, group=group, mode=mode, **args)
    out = {"y": host(y)} if with_y else {}
    if quant:
        out["codes"] = host(args["codes"])
        out["scales"] = host(args["scales"])
        if mode:
            out["zeros"] = host(args["zeros"])
    return out


# m spans every matrix-core tiling of the mixing step (one or two 32-row
# tiles; one to four 16-deep k steps) and its edges (17, 32, 33, 48, 49).
@pytest.mark.parametrize("m,nb", [(43, 256), (9, 512), (16, 1024), (64, 256), (2, 4096),
                                  (5, 1024), (16, 4096), (17, 256), (32, 512), (33, 256),
                                  (48, 256), (49, 512), (2, 256), (16, 256)])
def test_kron_wide_shapes(m, nb):
    rng = np.random.default_rng(7000 + 10 * m + nb)
    th = rand_theta(rng, nb)
    mix = inputs.mixing_factor(rng, m)
    rows = 37
    x = inputs.f32_to_bf16_bits(rng.standard_normal((rows, m * nb)).astype(np.float32))
    y64 = oracle.kron_forward(x, th, mix)
    for quant, mode in ((False, 0), (True, 0), (True, 1)):
        out = run_kron_wide(x, th, mix, quant=quant, mode=mode)
        assert_forward(out["y"], y64, x, m * nb)
        if quant:
            assert_quant(out, y64, 4, 128, mode)
    xf = rng.standard_normal((5, m * nb)).astype(np.float32)
    out = run_kron_wide(xf, th, mix, quant=False, y_dtype=torch.float32, coeffs=True)
    assert_forward(out["y"], oracle.kron_forward(xf, th, mix), xf, m * nb)


@pytest.mark.parametrize("m", [2, 16, 43, 64])
def test_kron_wide_one_pass(m):
    """bf16 rows with nb = 256 take the one-pass kernel (mix on the matrix
    cores into LDS, butterfly and quantizer per segment): fp32, bf16 and no
    output, groups of 8 to 256, both modes and widths, in place."""
    rng = np.random.default_rng(7500 + m)
    nb, rows = 256, 45
    th = rand_theta(rng, nb)
    mix = inputs.mixing_factor(rng, m)
    cols = inputs.outlier_columns(rng, m * nb)
    x = inputs.activations(rng, rows, m * nb, cols, "bf16")
    y64 = oracle.kron_forward(x, th, mix)
    out = run_kron_wide(x, th, mix, quant=False, y_dtype=torch.float32)
    print("one pass m=%d fp32:" % m, assert_forward(out["y"], y64, x, m * nb))
    for bits, group, mode in ((4, 8, 1), (2, 64, 0), (2, 256, 1), (4, 128, 0)):
        out = run_kron_wide(x, th, mix, bits=bits, group=group, mode=mode)
        assert_forward(out["y"], y64, x, m * nb)
        print("one pass m=%d" % m, bits, group, mode, assert_quant(out, y64, bits, group, mode))
        only = run_kron_wide(x, th, mix, bits=bits, group=group, mode=mode, with_y=False)
        for k in only:
            assert np.array_equal(only[k], out[k]), k
    # in place
    xd = dev(x)
    ws = torch.empty(B.bfly_kron_forward_wide_workspace_bytes(rows, m, nb), dtype=torch.uint8,
                     device="cuda")
    B.bfly_kron_forward_wide(xd, xd, dev(mix), ws, theta_b=dev(th))
    ref = run_kron_wide(x, th, mix, quant=False)
    assert np.array_equal(host(xd), ref["y"])


def test_kron_wide_workload_full():
    """n=11008 = O43 (x) B256 (the LLaMA-2-7B down projection's input), 8192
    bf16 rows with outliers, sym INT4 g128: all rows."""
    w = inputs.kron_wide_int4()
    x = w["x"]
    out = run_kron_wide(x, w["theta_b"], w["mix"])
    y64 = oracle.kron_forward(x, w["theta_b"], w["mix"])
    rf = assert_forward(out["y"], y64, x, 11008)
    rq = assert_quant(out, y64, 4, 128, 0)
    print("kron n=11008:", rf, rq)
