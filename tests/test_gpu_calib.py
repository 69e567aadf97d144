"""GPU parity of bfly_calib_step (one step of learning the angles: loss,
dL/dY, the butterfly backward, Adam) against the fp64 oracle.

The gradient is checked against the oracle fed the GPU's own Y (the same
forward kernel and table the step runs), so that the quantizer's and the
histogram's decisions are taken on the same values on both sides.  What
remains is arithmetic:
* loss terms to 1e-4 relative: fp32 partial sums of ~1e6 terms in fixed
  order, and a bin coordinate formed in fp32 (one element that lands on the
  other side of a bin boundary moves the KL by ~1e-6 / KL);
* dtheta (read back from Adam's first moment, m = (1 - beta1) dtheta at
  step 1): the fp32 backward's bound 1e-5 log2(n) A (A = the magnitude sum
  of the cancelling terms) for at least 95 % of the angles; every angle
  within that plus F = 4 flipped decisions.  A flip happens where the
  backward's recomputed Y (a few ulps from the forward's) and the forward's
  Y straddle a rounding or bin boundary; it moves one element of dL/dY by
  delta (one quantization step 2 s / N, or the KL slope's jump), and one
  element's change moves any angle's gradient by at most
  delta (|v_i| + |v_j|) <= 2 delta ||x_r||_2 (the stage outputs are
  orthogonal images of x_r);
* the updated angles, for every angle whose gradient is within the tight
  bound and larger than twice it, against Adam's first step from the
  oracle's gradient (the bound follows from the step lr g / (|g| + eps))."""
import numpy as np
import pytest

import oracle
import learnable_butterfly_rotation_amd as B
from learnable_butterfly_rotation_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def run(x, th, steps, bits, group, bins, lam, lr=1e-3):
    rows, n = x.shape
    cfg = B.bfly_calib_config(bits, group, bins, lam, lr, 0.9, 0.999, 1e-8)
    xd = torch.from_numpy(x).cuda()
    thd = torch.from_numpy(th.copy()).cuda()
    m = torch.zeros_like(thd)
    v = torch.zeros_like(thd)
    loss = torch.zeros(3, device="cuda")
    ws = torch.empty(B.bfly_calib_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    losses = []
    for step in range(1, steps + 1):
        B.bfly_calib_step(xd, thd, m, v, step, cfg, loss, ws)
        losses.append(loss.cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    return thd.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), losses


@pytest.mark.parametrize("n,rows,group,bits,bins", [(256, 300, 32, 4, 16), (1024, 77, 128, 2, 8),
                                                    (64, 1, 64, 4, 32), (4096, 257, 128, 4, 16)])
def test_calib_step_first_step(n, rows, group, bits, bins):
    rng = np.random.default_rng(9000 + n + rows)
    th = inputs.angles(rng, n)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, "f32")
    lam, lr = 0.1, 1e-3
    th1, m1, v1, losses = run(x, th, 1, bits, group, bins, lam, lr)
    ref = oracle.calib_step(x, th, np.zeros_like(th), np.zeros_like(th), 1, bits, group, bins,
                            lam, lr, 0.9, 0.999, 1e-8)
    got = losses[0]
    # the oracle on the GPU's own Y
    yd = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    B.bfly_forward(torch.from_numpy(x).cuda(), yd, theta=torch.from_numpy(th).cuda())
    y_gpu = yd.cpu().numpy().astype(np.float64)
    lg = oracle.calib_loss_grad(y_gpu, bits, group, bins, lam)
    bw = oracle.backward(x, lg["g"].astype(np.float32), th, want_y=False, want_dx=False)
    for k, name in enumerate(("loss", "rec", "kl")):
        for want in (ref[name], lg[name]):
            assert abs(got[k] - want) <= 1e-4 * abs(want) + 1e-12, (name, got[k], want)
    dth = m1.astype(np.float64) / 0.1
    d64, dabs = bw["dtheta"], bw["dabs"]
    tight = 1e-5 * np.log2(n) * dabs
    # one flipped decision: the larger of a quantization step and the KL
    # slope's jump, at the element where it is largest
    N = rows * n
    q = oracle.quantize(y_gpu, bits, group, oracle.SYM)
    step = np.repeat(q["scales"].view(np.float16).astype(np.float64), group, axis=1)
    lb = np.log(bins * (lg["p"] + oracle.CALIB_SMOOTH) / (1 + bins * oracle.CALIB_SMOOTH))
    jump = np.abs(np.diff(lb, 2)).max() if bins > 2 else 0.0
    a = np.where(lg["a"] > 0, lg["a"], np.inf)
    delta = np.maximum(2 * step / N, lam * jump / ((2.0 / bins) * N * (1 + bins * 1e-6)) / a).max()
    flips = 4 * delta * 2 * np.linalg.norm(x.astype(np.float64), axis=1).max()
    err = np.abs(dth - d64)
    within = err <= tight
    print("dtheta: %.4f of the angles within 1e-5 log2(n) A; max err / (tight + flips) %.3g"
          % (within.mean(), float((err / (tight + flips)).max())))
    assert within.mean() >= 0.95, within.mean()
    assert (err <= tight + flips).all(), float((err / (tight + flips)).max())
    cos = (dth * d64).sum() / np.sqrt((dth * dth).sum() * (d64 * d64).sum())
    assert cos > 0.99999
    # Adam's first step, lr g / (|g| + eps), from the oracle's gradient: for
    # an angle whose gradient is within `tight` of the oracle's, the steps
    # differ by at most lr eps tight / (|g| (|g| - tight)), plus the fp32
    # rounding of theta and of the update (a few ulps of theta)
    th_ref = oracle.adam(th, np.zeros_like(d64), np.zeros_like(d64), d64, 1, lr, 0.9, 0.999,
                         1e-8)[0]
    clear = within & (np.abs(d64) > 2 * tight)
    assert clear.mean() > 0.5, clear.mean()
    g = np.abs(d64)
    step_bound = (lr * 1e-8 * tight / (g * np.maximum(g - tight, 1e-300))
                  + 4 * np.spacing(np.abs(th).astype(np.float32)).astype(np.float64))
    assert (np.abs(th1 - th_ref) <= step_bound)[clear].all(), \
        float((np.abs(th1 - th_ref) / step_bound)[clear].max())
    # Adam's first step moves each angle by at most lr (plus fp32 rounding of theta)
    assert np.abs(th1 - th).max() <= lr * (1 + 1e-5) + 2 * np.spacing(np.abs(th).max())


def test_calib_steps_follow_the_oracle_and_repeat_bitwise():
    """Twenty steps on an outlier-heavy batch: the GPU's loss sequence
    follows the oracle's own twenty steps, the loss goes down, and the same
    run again gives the same bits (fixed-order reductions)."""
    rng = np.random.default_rng(9100)
    n, rows, lr = 1024, 2048, 1e-3
    th = (inputs.angles(rng, n) * 0.05).astype(np.float32)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, "f32")
    a = run(x, th, 20, 4, 128, 16, 0.05, lr=lr)
    b = run(x, th, 20, 4, 128, 16, 0.05, lr=lr)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    t, m, v = th.copy(), np.zeros_like(th, dtype=np.float64), np.zeros_like(th, dtype=np.float64)
    ref = []
    for step in range(1, 21):
        o = oracle.calib_step(x, t, m, v, step, 4, 128, 16, 0.05, lr, 0.9, 0.999, 1e-8)
        ref.append(o["loss"])
        t, m, v = o["theta"].astype(np.float32), o["m"], o["v"]
    got = np.array([l[0] for l in a[3]])
    assert np.abs(got - np.array(ref)).max() <= 1e-3 * ref[0], (got, ref)
    assert got[-1] < 0.99 * got[0]
