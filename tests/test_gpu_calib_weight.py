"""GPU parity of bfly_calib_step_weight (the layer-output loss: Xr = Q X,
Wr = W Q^T quantized to What, L = ||Xr What^T - X W^T||^2 / N + lambda KL(Xr),
the quantizer's rounding passed straight through) against the fp64 oracle.

The oracle is given the quantizer's decisions the GPU took (its codes,
scales and zero points for Wr, from bfly_forward_quant with the same angles:
the kernel and table the step runs), so that both sides quantize alike.
What remains is fp32 arithmetic, bounded to first order:
* Xr and Wr carry the forward's rounding error, at most
  4 ceil(log2 n) 2^-24 ||row||_2 per element (L Givens stages in fp32 with
  rounded coefficients; the bound the bf16 checks use); the products
  R = Xr E^T and G = 2 R E / N add (k + 2) 2^-24 of their magnitude sums
  (k the contraction length); so, element by element,
    |dR| <= |dXr| |E|^T + |Xr| |dE|^T + (n + 2) u |Xr| |E|^T,
    |dG| <= 2 / N (|dR| |E| + |R| |dE| + (out + 2) u |R| |E|);
* dtheta[s][p] = sum_r g_j v_i - g_i v_j is linear in G through g = M_s G
  (M_s the transpose of the stages after s): a change dG moves it by at most
  sum_r |v_i M_s[j, :] - v_j M_s[i, :]| |dG_r|, computed here from the
  dense stage matrices;
* the fp32 backward itself: 1e-5 log2(n) A (A the magnitude sum of the
  cancelling terms, from the oracle's single-backward form);
* the uniformity term's bin decisions: at least 95 % of the angles within
  the arithmetic bound above, every angle within it plus four flipped
  elements (as in the activation-side step).
The loss terms match to 1e-4 relative (fp32 partial sums in fixed order)."""
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


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(x, w, th, steps, cfg):
    rows, n = x.shape
    out = w.shape[0]
    xd, wd = dev(x), dev(w)
    thd = torch.from_numpy(th.copy()).cuda()
    m, v = torch.zeros_like(thd), torch.zeros_like(thd)
    loss = torch.zeros(3, device="cuda")
    ws = torch.empty(B.bfly_calib_step_weight_workspace_bytes(rows, out, n), dtype=torch.uint8,
                     device="cuda")
    losses = []
    for step in range(1, steps + 1):
        B.bfly_calib_step_weight(xd, wd, thd, m, v, step, cfg, loss, ws)
        losses.append(loss.cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    return thd.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), losses


def gpu_decisions(w, th, bits, group, mode):
    out, n = w.shape
    codes = torch.zeros((out, n * bits // 8), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((out, n // group), dtype=torch.float16, device="cuda")
    zeros = torch.zeros((out, n // group), dtype=torch.float16, device="cuda") if mode else None
    B.bfly_forward_quant(dev(w), None, codes, scales, zeros, theta=dev(th), bits=bits, group=group,
                         mode=mode)
    torch.cuda.synchronize()
    h = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return codes.cpu().numpy(), h(scales), h(zeros) if zeros is not None else None


def stage_matrices(th):
    """Dense B_s (stage s alone) for every stage."""
    mats = []
    for s in range(th.shape[0]):
        t = np.zeros_like(th)
        t[s] = th[s]
        mats.append(oracle.dense_q(t))
    return mats


def dtheta_sensitivity(x64, th, dG):
    """sum_r |v_i M_s[j, :] - v_j M_s[i, :]| dG_r for every angle [s][p]:
    the most a change of G bounded by dG (elementwise) moves dtheta."""
    L, half = th.shape
    n = 2 * half
    Bs = stage_matrices(th)
    out = np.zeros((L, half))
    v = x64.copy()                                   # rows x n, stage inputs
    for s in range(L):
        v = v @ Bs[s].T                              # stage-s outputs
        M = np.eye(n)
        for t in range(s + 1, L):                    # M_s = B_{s+1}^T ... B_{L-1}^T
            M = M @ Bs[t].T
        i = np.array([((p >> s) << (s + 1)) | (p & ((1 << s) - 1)) for p in range(half)])
        j = i + (1 << s)
        # per angle: sum_r sum_k |v[r, i] M[j, k] - v[r, j] M[i, k]| dG[r, k]
        for p in range(half):
            coef = np.abs(v[:, i[p], None] * M[j[p]][None, :] - v[:, j[p], None] * M[i[p]][None, :])
            out[s, p] = (coef * dG).sum()
    return out


@pytest.mark.parametrize("n,rows,out,bits,group,mode,w_dt",
                         [(256, 64, 48, 2, 32, oracle.ASYM, "bf16"),
                          (128, 33, 32, 4, 64, oracle.SYM, "f32"),
                          (256, 80, 16, 2, 128, oracle.ASYM, "f32")])
def test_calib_step_weight_first_step(n, rows, out, bits, group, mode, w_dt):
    rng = np.random.default_rng(9300 + n + rows + out)
    th = inputs.angles(rng, n)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, "f32")
    wf = (rng.standard_normal((out, n)) * 0.02).astype(np.float32)
    w = inputs.f32_to_bf16_bits(wf) if w_dt == "bf16" else wf
    bins, lam, lr = 16, 0.1, 1e-3
    cfg = B.bfly_calib_weight_config(bits, group, mode, bins, lam, lr, 0.9, 0.999, 1e-8)
    th1, m1, _, losses = run(x, w, th, 1, cfg)
    wq = gpu_decisions(w, th, bits, group, mode)
    ref = oracle.calib_weight_loss_grad(x, w, th, bits, group, mode, bins, lam, wq=wq)
    got = losses[0]
    for k, name in enumerate(("loss", "rec", "kl")):
        assert abs(got[k] - ref[name]) <= 1e-4 * abs(ref[name]) + 1e-12, (name, got[k], ref[name])

    # the single-backward form of the same gradient, for the backward's bound
    N = rows * out
    r, e, xr = ref["r"], ref["e"], ref["xr"]
    kl = oracle.calib_loss_grad(xr, 4, group, bins, lam, with_rec=False)
    g = 2.0 * r @ e / N + kl["g"]
    single = oracle.backward(x, g.astype(np.float32), th, want_y=False, want_dx=False)
    d64, dabs = single["dtheta"], single["dabs"]
    assert np.abs(d64 - ref["dtheta"]).max() <= 1e-6 * np.abs(d64).max()

    # first-order bound of the fp32 products' error (see the module doc)
    x64 = x.astype(np.float64)
    w64 = inputs.bf16_bits_to_f32(w).reshape(w.shape).astype(np.float64) if w.dtype == np.uint16 \
        else w.astype(np.float64)
    fe = 4 * math.ceil(math.log2(n)) * U
    dxr = fe * np.linalg.norm(x64, axis=1, keepdims=True) * np.ones((1, n))
    de = fe * np.linalg.norm(w64, axis=1, keepdims=True) * np.ones((1, n))
    ae, axr, ar = np.abs(e), np.abs(xr), np.abs(r)
    dr = dxr @ ae.T + axr @ de.T + (n + 2) * U * (axr @ ae.T)
    dg = 2.0 / N * (dr @ ae + ar @ de + (out + 2) * U * (ar @ ae))
    # four flipped bin decisions of the uniformity term
    lb = np.log(bins * (kl["p"] + oracle.CALIB_SMOOTH) / (1 + bins * oracle.CALIB_SMOOTH))
    jump = np.abs(np.diff(lb, 2)).max()
    a = np.where(kl["a"] > 0, kl["a"], np.inf)
    delta = (lam * jump / ((2.0 / bins) * rows * n * (1 + bins * 1e-6)) / a).max()
    flips = 4 * delta * 2 * np.linalg.norm(x64, axis=1).max()
    tight = 1e-5 * math.log2(n) * dabs + dtheta_sensitivity(x64, th, dg)

    dth = m1.astype(np.float64) / 0.1
    err = np.abs(dth - d64)
    within = err <= tight
    print("weight-loss dtheta: %.4f of the angles within the arithmetic bound; max err / (bound + "
          "flips) %.3g, max err / max|dtheta| %.3g"
          % (within.mean(), float((err / (tight + flips)).max()), float(err.max() / np.abs(d64).max())))
    # a flipped bin decision moves one element of the gradient by as much as
    # the uniformity term's whole per-element slope, so flips are allowed for
    # every angle but expected in few of them
    assert within.mean() >= 0.95, within.mean()
    assert (err <= tight + flips).all(), float((err / (tight + flips)).max())
    cos = (dth * d64).sum() / np.sqrt((dth * dth).sum() * (d64 * d64).sum())
    assert cos > 0.99999
    # Adam's first step from the oracle's gradient (bound as in the activation-side test)
    th_ref = oracle.adam(th, np.zeros_like(d64), np.zeros_like(d64), d64, 1, lr, 0.9, 0.999, 1e-8)[0]
    gabs = np.abs(d64)
    clear = within & (gabs > 2 * tight)
    assert clear.mean() > 0.5, clear.mean()
    step_bound = (lr * 1e-8 * tight / (gabs * np.maximum(gabs - tight, 1e-300))
                  + 4 * np.spacing(np.abs(th).astype(np.float32)).astype(np.float64))
    assert (np.abs(th1 - th_ref) <= step_bound)[clear].all(), \
        float((np.abs(th1 - th_ref) / step_bound)[clear].max())


def test_calib_step_weight_steps_follow_the_oracle_and_repeat():
    """Twenty steps on an outlier-heavy batch: the GPU's loss terms follow
    the oracle's own twenty steps (each side quantizing with its own
    decisions, so to 1e-3 of the first loss), the layer-output loss goes
    down, and a second run gives the same bits (fixed-order reductions)."""
    rng = np.random.default_rng(9400)
    n, rows, out = 256, 512, 64
    th = (inputs.angles(rng, n) * 0.05).astype(np.float32)
    cols = inputs.outlier_columns(rng, n)
    x = inputs.activations(rng, rows, n, cols, "f32")
    w = inputs.f32_to_bf16_bits((rng.standard_normal((out, n)) * 0.02).astype(np.float32))
    hp = (2, 64, oracle.ASYM, 16, 0.05, 2e-3, 0.9, 0.999, 1e-8)
    cfg = B.bfly_calib_weight_config(*hp)
    a = run(x, w, th, 20, cfg)
    b = run(x, w, th, 20, cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    t, m, v = th.copy(), np.zeros_like(th, dtype=np.float64), np.zeros_like(th, dtype=np.float64)
    ref = []
    for step in range(1, 21):
        o = oracle.calib_weight_step(x, w, t, m, v, step, *hp)
        ref.append((o["loss"], o["rec"], o["kl"]))
        t, m, v = o["theta"].astype(np.float32), o["m"], o["v"]
    got, ref = np.array(a[3]), np.array(ref)
    print("layer-output loss over 20 steps:", got[0, 1], "->", got[-1, 1], "(oracle", ref[-1, 1], ")")
    assert (np.abs(got - ref) <= 1e-3 * ref[0]).all(), (got, ref)
    assert got[-1, 1] < got[0, 1]
