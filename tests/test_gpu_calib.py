"""GPU parity of bfly_calib_step (one step of learning the angles: loss,
dL/dY, the butterfly backward, Adam) against the fp64 oracle.

Tolerances: the loss terms to 1e-4 relative (fp32 sums of ~1e6 terms in
fixed order, fp64 final sums); dtheta (read back from Adam's first moment,
m = (1 - beta1) dtheta at step 1) to 1e-4 of the magnitude sum `dabs` plus
2e-3 of max |dtheta| -- a quantization or bin decision that lies within
fp32 rounding of its boundary moves one element of dL/dY, which the fp64
oracle takes the other way; the updated angles where the gradient is
clearly nonzero to 1e-6 (Adam's first step is lr * sign)."""
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
    for k, name in enumerate(("loss", "rec", "kl")):
        assert abs(got[k] - ref[name]) <= 1e-4 * abs(ref[name]) + 1e-12, (name, got[k], ref[name])
    dth = m1 / 0.1
    d64 = ref["dtheta"]
    bound = 1e-4 * ref["dabs"] + 2e-3 * np.abs(d64).max()
    assert (np.abs(dth - d64) <= bound).all(), float((np.abs(dth - d64) / bound).max())
    cos = (dth * d64).sum() / np.sqrt((dth * dth).sum() * (d64 * d64).sum())
    assert cos > 0.99999
    clear = np.abs(d64) > 10 * bound
    assert clear.sum() >= 10
    assert np.abs(th1 - ref["theta"])[clear].max() < 1e-6
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
