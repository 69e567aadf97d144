"""The oracle's pins catch plausible mistakes: each case plants one mistake in
a private copy of the oracle (C or Python), on the CPU, and runs the pins of
tests/test_oracle_pins.py against that copy; at least one pin must fail.  A
mistake that every pin lets through would mean that part of the oracle is not
pinned.  The repository's oracle itself is never modified."""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, file, text to find exactly once, replacement)
MUTATIONS = [
    ("rotation sign", "bflyref.c",
     "        u[i] = c * ui - sn * uj;\n        u[j] = sn * ui + c * uj;",
     "        u[i] = c * ui + sn * uj;\n        u[j] = -sn * ui + c * uj;"),
    ("pair rank", "bflyref.c",
     "        int p = ((i >> (s + 1)) << s) + (i & (half - 1));\n        double c = c_s[p], sn = s_s[p];\n        double ui",
     "        int p = i >> 1;\n        double c = c_s[p], sn = s_s[p];\n        double ui"),
    ("stage order", "bflyref.c",
     "    for (int s = 0; s < L; ++s)\n        stage_forward(u,",
     "    for (int s = L - 1; s >= 0; --s)\n        stage_forward(u,"),
    ("cos and sin swapped", "bflyref.c",
     "        (*cs)[k] = cos((double)theta[k]);\n        (*sn)[k] = sin((double)theta[k]);",
     "        (*cs)[k] = sin((double)theta[k]);\n        (*sn)[k] = cos((double)theta[k]);"),
    ("Kronecker factor transposed", "bflyref.c",
     "acc += (double)mix[a * m + a2] * u[(int64_t)a2 * nb + b];",
     "acc += (double)mix[a2 * m + a] * u[(int64_t)a2 * nb + b];"),
    ("symmetric range 8", "bflyref.c",
     "const int qmax = (1 << (bits - 1)) - 1;", "const int qmax = (1 << (bits - 1));"),
    ("ties away from zero", "bflyref.c",
     "return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;", "return f + 1.0;"),
    ("divide by the unrounded scale", "bflyref.c",
     "double sc = bflyref_fp16_value(s16);", "double sc = use_given ? bflyref_fp16_value(s16) : spre;"),
    ("zero point sign", "bflyref.c", "zp = -lo; /* divided", "zp = lo; /* divided"),
    ("asymmetric levels", "bflyref.c",
     "const int levels = (1 << bits) - 1;", "const int levels = (1 << bits);"),
    ("packing order", "bflyref.c",
     "<< (bits * (e % per_byte)));", "<< (bits * (per_byte - 1 - e % per_byte)));"),
    ("gradient sign", "bflyref.c",
     "pd[(int64_t)s * (n / 2) + p] += t1 - t2;", "pd[(int64_t)s * (n / 2) + p] += t2 - t1;"),
    ("gradient at the stage input", "bflyref.c",
     "const double* v = V + (int64_t)(s + 1) * n; /* stage-s output */",
     "const double* v = V + (int64_t)s * n;"),
    ("transposed stage not transposed", "bflyref.c",
     "        g[i] = c * gi + sn * gj;\n        g[j] = -sn * gi + c * gj;",
     "        g[i] = c * gi - sn * gj;\n        g[j] = sn * gi + c * gj;"),
    ("bf16 rounding precision", "bflyref.c",
     "round_to_format(x, 8, -126, maxf)", "round_to_format(x, 9, -126, maxf)"),
    ("fp16 subnormal range", "bflyref.c",
     "round_to_format(x, 11, -14, 65504.0)", "round_to_format(x, 11, -15, 65504.0)"),
    ("Adam bias correction power", "__init__.py",
     "mh = m / (1 - beta1 ** step)", "mh = m / (1 - beta1 ** 1)"),
    ("Adam second moment not square-rooted", "__init__.py",
     "lr * mh / (np.sqrt(vh) + eps)", "lr * mh / (vh + eps)"),
    ("KL without the bin count", "__init__.py",
     "lb = np.log(bins * ps)", "lb = np.log(ps)"),
    ("histogram weights swapped", "__init__.py",
     "p = (np.bincount(j.ravel(), weights=(1 - f).ravel(), minlength=bins) +\n"
     "         np.bincount((j + 1).ravel(), weights=f.ravel(), minlength=bins)) / N",
     "p = (np.bincount(j.ravel(), weights=f.ravel(), minlength=bins) +\n"
     "         np.bincount((j + 1).ravel(), weights=(1 - f).ravel(), minlength=bins)) / N"),
    ("reconstruction gradient halved", "__init__.py",
     "g = 2.0 * (y - yhat) / N", "g = (y - yhat) / N"),
    ("dequantize zero point sign", "__init__.py",
     "return s * (q - np.repeat(z, group, axis=1))", "return s * (q + np.repeat(z, group, axis=1))"),
    ("Hadamard signs", "__init__.py",
     "return np.where(parity == 1, -1.0, 1.0) / np.sqrt(float(n))",
     "return np.where(parity == 1, 1.0, -1.0) / np.sqrt(float(n))"),
    ("Kronecker backward mixes with O, not its transpose", "__init__.py",
     'gz = np.einsum("ab,rai->rbi", mix64, g3)', 'gz = np.einsum("ab,rbi->rai", mix64, g3)'),
    ("layer-output gradient through the unquantized weights", "__init__.py",
     'gx = dyhat @ what + kl["g"]', 'gx = dyhat @ wr + kl["g"]'),
    ("layer-output residual sign", "__init__.py", "    r = yhat - y\n", "    r = y - yhat\n"),
    ("weight branch against the unrotated activations", "__init__.py",
     "gw = dyhat.T @ xr", "gw = dyhat.T @ widen(x)"),
    ("layer-output mean over rows only", "__init__.py", "n_rec = r.size", "n_rec = r.shape[0]"),
]


def _run_with_mutation(case):
    name, fname, old, new = case
    tmp = tempfile.mkdtemp(prefix="bflyref_mut_")
    try:
        dst = os.path.join(tmp, "oracle")
        os.makedirs(dst)
        for f in ("__init__.py", "bflyref.c"):
            shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, f))
        path = os.path.join(dst, fname)
        text = open(path).read()
        if text.count(old) != 1:
            return name, "anchor", "the text to mutate occurs %d times" % text.count(old)
        open(path, "w").write(text.replace(old, new))
        env = dict(os.environ, OMP_NUM_THREADS="1",
                   PYTHONPATH=os.pathsep.join([tmp, ROOT, os.environ.get("PYTHONPATH", "")]))
        # cwd = the copy's parent: `import oracle` finds the mutated copy first
        r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider",
                            "-m", "not gpu"], cwd=tmp, env=env, capture_output=True, text=True,
                           timeout=600)
        tail = (r.stdout + r.stderr).strip().splitlines()[-1:] or [""]
        return name, r.returncode, tail[0]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_every_planted_mistake_fails_a_pin():
    workers = min(8, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run_with_mutation, MUTATIONS))
    bad = [(n, rc, t) for n, rc, t in results if rc != 1]
    assert not bad, "mistakes no pin caught (or that did not apply): %s" % bad


def test_unmutated_copy_passes_its_pins():
    """The harness itself: the same copy with no mistake passes."""
    name, rc, tail = _run_with_mutation(("none", "__init__.py", "import ctypes\n", "import ctypes\n"))
    assert rc == 0, tail
