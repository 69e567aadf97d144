"""The C-ABI library loads, exports every symbol include/bfly.h declares, and
rejects bad arguments with the documented codes -- all before any HIP call,
so these run on a machine without a GPU.  No compute call is made."""
import ctypes
import os
import re

import pytest

import learnable_butterfly_rotation_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfly.h")

OK, NULL, SIZE, DTYPE, ALIGN, QUANT, WORKSPACE, UNSUPPORTED, HIP = range(9)

# fake, well-aligned device addresses: validation never dereferences them
X, Y, C, S, Z, TH, MIX, WS, CO = (ctypes.c_void_p(a) for a in
                                  (0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000,
                                   0x70000, 0x80000, 0x90000))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bfly_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.library_path):
        pytest.skip("libbfly.so not built")
    return B.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"bfly_forward", "bfly_forward_quant", "bfly_kron_forward", "bfly_backward",
            "bfly_prepare", "bfly_prepare_hadamard", "bfly_coeff_bytes", "bfly_backward_workspace_bytes",
            "bfly_status_string", "bfly_last_hip_error"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(9):
        assert B.bfly_status_string(s)
    assert B.bfly_status_string(99) == "unknown status"
    assert B.bfly_last_hip_error() == 0


def test_time_next_forward_arming(L):
    # makes no HIP call: fake handles are armed, then disarmed (both NULL)
    assert L.bfly_time_next_forward(None, 0x1000) == 1      # BFLY_ERR_NULL
    assert L.bfly_time_next_forward(0x1000, None) == 1
    assert L.bfly_time_next_forward(0x1000, 0x2000) == 0
    assert L.bfly_time_next_forward(None, None) == 0


def test_sizes(L):
    # (cos, sin) [L][n/2] + three-shear (p, u) [L-1][n/2] + last stage 4 x [n/2], fp32
    # per pair: (cos, sin) for every stage, two coefficient pairs (scaled and
    # three-shear form) and a sign product for stages 0..L-2, two
    # 4-coefficient last stages
    assert B.bfly_coeff_bytes(4096) == (12 * 2 + 2 * (12 - 1) * 2 + (12 - 1) + 2 * 4) * 2048 * 4
    assert B.bfly_coeff_bytes(256) == (8 * 2 + 2 * 7 * 2 + 7 + 2 * 4) * 128 * 4
    assert B.bfly_coeff_bytes(100) == 0
    assert B.bfly_coeff_bytes(32) == 0
    ws = B.bfly_backward_workspace_bytes(262144, 4096)
    assert ws >= B.bfly_coeff_bytes(4096) + 12 * 2048 * 4  # table + at least one partial slot
    assert B.bfly_backward_workspace_bytes(10, 4096) < ws
    assert B.bfly_backward_workspace_bytes(-1, 4096) == 0
    assert B.bfly_backward_workspace_bytes(100, 8192) == 0


def fwd(L, x=X, xd=0, y=Y, yd=0, rows=4, n=256, th=TH, co=None, ws=WS, wsb=None):
    if wsb is None:
        wsb = B.bfly_coeff_bytes(n)
    return L.bfly_forward(x, xd, y, yd, rows, n, th, co, ws, wsb, None)


def test_forward_validation(L):
    assert fwd(L, rows=0) == OK                       # valid, nothing to do
    assert fwd(L, rows=0, x=None, y=None) == OK       # empty tensors carry NULL
    assert fwd(L, x=None) == NULL
    assert fwd(L, y=None) == NULL
    assert fwd(L, th=None, co=None) == NULL
    assert fwd(L, th=None, co=CO, rows=0) == OK
    assert fwd(L, xd=2) == DTYPE
    assert fwd(L, yd=-1) == DTYPE
    assert fwd(L, rows=-1) == SIZE
    assert fwd(L, n=100) == SIZE
    assert fwd(L, n=0) == SIZE
    assert fwd(L, n=32) == UNSUPPORTED
    assert fwd(L, n=16384) == UNSUPPORTED
    # n = 8192 always needs its workspace: the table area, then the fp32 rows
    # between its two passes
    w8 = B.bfly_forward_workspace_bytes(4, 8192)
    assert w8 == (B.bfly_coeff_bytes(8192) + 255) // 256 * 256 + 4 * 8192 * 4
    assert B.bfly_coeff_bytes(8192) == 2 * B.bfly_coeff_bytes(4096) + 4096 * 8
    assert B.bfly_forward_workspace_bytes(4, 4096) == B.bfly_coeff_bytes(4096)
    assert B.bfly_forward_workspace_bytes(-1, 8192) == 0
    assert B.bfly_forward_workspace_bytes(4, 100) == 0
    assert fwd(L, n=8192, rows=0, wsb=w8) == OK
    assert fwd(L, n=8192, rows=0, co=CO, th=None, ws=None, wsb=0) == NULL
    assert fwd(L, n=8192, rows=4, wsb=w8 - 1) == WORKSPACE
    assert fwd(L, n=8192, rows=-1, wsb=w8) == SIZE
    assert fwd(L, n=8192, rows=0, x=ctypes.c_void_p(0x10008), wsb=w8) == ALIGN
    assert fwd(L, x=ctypes.c_void_p(0x10008)) == ALIGN
    assert fwd(L, y=ctypes.c_void_p(0x20004)) == ALIGN
    assert fwd(L, co=ctypes.c_void_p(0x90008), rows=0) == ALIGN
    # angles without a table: the table goes into the caller's workspace
    assert fwd(L, rows=0, ws=None) == NULL
    assert fwd(L, rows=0, wsb=B.bfly_coeff_bytes(256) - 1) == WORKSPACE
    assert fwd(L, rows=0, ws=ctypes.c_void_p(0x80008)) == ALIGN
    # with a table the workspace is not used
    assert fwd(L, rows=0, th=None, co=CO, ws=None, wsb=0) == OK
    assert fwd(L, rows=0, co=CO, ws=None, wsb=0) == OK


def fq(L, y=Y, c=C, s=S, z=None, bits=4, group=128, mode=0, n=4096, rows=0, ws=WS, wsb=None):
    if wsb is None:
        wsb = B.bfly_coeff_bytes(n)
    return L.bfly_forward_quant(X, 1, y, 1, c, s, z, rows, n, TH, None, bits, group, mode, ws, wsb,
                                None)


def test_forward_quant_validation(L):
    assert fq(L) == OK
    assert fq(L, y=None) == OK                        # codes only
    assert fq(L, c=None, rows=1) == NULL
    assert fq(L, c=None, s=None, y=None) == OK        # no rows: pointers unused
    assert fq(L, s=None, rows=1) == NULL
    assert fq(L, bits=3) == QUANT
    assert fq(L, bits=8) == QUANT
    assert fq(L, mode=2) == QUANT
    assert fq(L, mode=1, rows=1) == QUANT             # asym needs zeros
    assert fq(L, mode=1, z=Z) == OK
    assert fq(L, mode=0, z=Z) == QUANT                # sym must not get zeros
    assert fq(L, group=100) == QUANT
    assert fq(L, group=4) == QUANT
    assert fq(L, group=1024) == QUANT
    assert fq(L, group=512, n=256) == QUANT           # group larger than the row
    for g in (8, 16, 32, 64, 128, 256, 512):
        assert fq(L, group=g) == OK
        assert fq(L, group=g, n=8192, wsb=B.bfly_forward_workspace_bytes(0, 8192)) == OK
    assert fq(L, group=1024, n=8192, wsb=1 << 30) == QUANT
    assert fq(L, c=ctypes.c_void_p(0x30004)) == ALIGN
    assert fq(L, s=ctypes.c_void_p(0x40001)) == ALIGN
    assert fq(L, ws=None) == NULL
    assert fq(L, wsb=B.bfly_coeff_bytes(4096) - 1) == WORKSPACE
    assert fq(L, ws=ctypes.c_void_p(0x80004)) == ALIGN


def test_forward_quant_noalloc_validation(L):
    # validated like bfly_forward_quant (its scratch replaces the workspace);
    # rows == 0 returns before any HIP call
    def nq(y=Y, c=C, s=S, z=None, bits=4, group=128, mode=0, n=4096, rows=0, th=TH):
        return L.bfly_forward_quant_noalloc(X, 1, y, 1, c, s, z, rows, n, th, bits, group, mode,
                                            None)
    assert nq() == OK
    assert nq(y=None) == OK
    assert nq(th=None) == NULL
    assert nq(c=None, rows=1) == NULL
    assert nq(bits=3) == QUANT
    assert nq(mode=1, rows=1) == QUANT
    assert nq(mode=1, z=Z) == OK
    assert nq(n=100) == SIZE
    assert nq(n=32) == UNSUPPORTED
    assert nq(n=8192) == UNSUPPORTED
    assert nq(rows=-1) == SIZE
    assert nq(c=ctypes.c_void_p(0x30004)) == ALIGN
    for n in (64, 128, 256, 512, 1024, 2048, 4096):
        assert nq(n=n, group=min(128, n)) == OK


def kf(L, m=5, nb=1024, c=C, s=S, z=None, mix=MIX, group=128, rows=0, ws=WS, wsb=None, co=None):
    if wsb is None:
        wsb = B.bfly_coeff_bytes(nb)
    return L.bfly_kron_forward(X, 1, Y, 1, c, s, z, rows, m, nb, TH, co, mix, 4, group, 0, ws, wsb,
                               None)


def test_kron_validation(L):
    assert kf(L) == OK
    assert kf(L, c=None, s=None) == OK                # no quantization
    assert kf(L, c=None) == QUANT                     # scales without codes
    assert kf(L, mix=None) == NULL
    assert kf(L, m=0) == SIZE
    assert kf(L, m=9) == SIZE
    assert kf(L, nb=1000) == SIZE
    assert kf(L, m=3, nb=4096) == UNSUPPORTED         # 12288 > 8192
    assert kf(L, nb=8192, m=1) == UNSUPPORTED
    assert kf(L, m=1, nb=4096) == OK
    assert kf(L, m=5, nb=256, group=512) == QUANT     # group must divide nb
    for m in range(2, 9):
        assert kf(L, m=m, nb=512) == OK
    assert kf(L, ws=None) == NULL
    assert kf(L, wsb=B.bfly_coeff_bytes(1024) - 1) == WORKSPACE
    assert kf(L, ws=None, wsb=0, co=CO) == OK


def bw(L, x=X, g=X, y=None, dx=Y, dth=C, rows=16, n=4096, th=TH, ws=WS, wsb=None):
    if wsb is None:
        wsb = B.bfly_backward_workspace_bytes(max(rows, 0), n)
    return L.bfly_backward(x, g, y, dx, dth, rows, n, th, None, ws, wsb, None)


def test_backward_validation(L):
    assert bw(L, x=None) == NULL
    assert bw(L, dth=None) == NULL
    assert bw(L, ws=None) == NULL
    assert bw(L, th=None) == NULL
    assert bw(L, rows=-1, wsb=1 << 30) == SIZE
    assert bw(L, n=100, wsb=1 << 30) == SIZE
    assert bw(L, n=8192, wsb=1 << 30) == UNSUPPORTED
    assert bw(L, wsb=B.bfly_backward_workspace_bytes(16, 4096) - 1) == WORKSPACE
    assert bw(L, dx=ctypes.c_void_p(0x20008)) == ALIGN


def test_prepare_validation(L):
    assert L.bfly_prepare(None, 256, CO, 1 << 20, None) == NULL
    assert L.bfly_prepare(TH, 256, None, 1 << 20, None) == NULL
    assert L.bfly_prepare(TH, 255, CO, 1 << 20, None) == SIZE
    assert L.bfly_prepare(TH, 256, CO, 100, None) == WORKSPACE
    assert L.bfly_prepare(TH, 256, ctypes.c_void_p(0x90008), 1 << 20, None) == ALIGN


def test_prepare_hadamard_validation(L):
    assert L.bfly_prepare_hadamard(256, None, 1 << 20, None) == NULL
    assert L.bfly_prepare_hadamard(255, CO, 1 << 20, None) == SIZE
    assert L.bfly_prepare_hadamard(1, CO, 1 << 20, None) == SIZE
    assert L.bfly_prepare_hadamard(32, CO, 1 << 20, None) == UNSUPPORTED
    assert L.bfly_prepare_hadamard(256, CO, 100, None) == WORKSPACE
    assert L.bfly_prepare_hadamard(256, ctypes.c_void_p(0x90008), 1 << 20, None) == ALIGN


def qm(L, a=X, ad=1, c=C, s=S, z=Z, y=Y, yd=1, rows=0, n_out=11008, k=4096, bits=2, group=128,
       mode=1):
    return L.bfly_quant_matmul(a, ad, c, s, z, y, yd, rows, n_out, k, bits, group, mode, None)


def test_quant_matmul_validation(L):
    assert qm(L) == OK                                   # rows == 0: nothing to do
    assert qm(L, a=None, y=None) == OK
    assert qm(L, rows=-1) == SIZE
    assert qm(L, n_out=0) == SIZE
    assert qm(L, k=0) == SIZE
    assert qm(L, rows=5, a=None) == NULL
    assert qm(L, rows=5, y=None) == NULL
    assert qm(L, c=None) == NULL
    assert qm(L, s=None) == NULL
    assert qm(L, ad=0) == DTYPE                          # activations are bf16
    assert qm(L, yd=2) == DTYPE
    assert qm(L, bits=3) == QUANT
    assert qm(L, z=None) == QUANT                        # asymmetric needs zero points
    assert qm(L, mode=0) == QUANT                        # symmetric takes none
    assert qm(L, mode=0, z=None) == OK
    assert qm(L, group=32) == QUANT
    assert qm(L, group=512, k=4096 + 128) == QUANT       # group must divide k
    assert qm(L, n_out=11008 + 64) == UNSUPPORTED
    assert qm(L, k=4096 + 64, group=64) == OK
    assert qm(L, k=65536 + 128) == UNSUPPORTED
    assert qm(L, c=ctypes.c_void_p(0x30008)) == ALIGN
    assert qm(L, a=ctypes.c_void_p(0x10008)) == ALIGN
    assert qm(L, y=ctypes.c_void_p(0x20004)) == ALIGN
    assert qm(L, s=ctypes.c_void_p(0x40001)) == ALIGN


def kb(L, x=X, g=X, dx=Y, dth=C, rows=16, m=5, nb=1024, th=TH, co=None, mix=MIX, ws=WS,
       wsb=None):
    if wsb is None:
        wsb = B.bfly_kron_backward_workspace_bytes(max(rows, 0), m, nb)
    return L.bfly_kron_backward(x, g, dx, dth, rows, m, nb, th, co, mix, ws, wsb, None)


def test_kron_backward_validation(L):
    assert B.bfly_kron_backward_workspace_bytes(16, 5, 1024) > B.bfly_backward_workspace_bytes(80, 1024)
    assert B.bfly_kron_backward_workspace_bytes(16, 1, 1024) == 0
    assert B.bfly_kron_backward_workspace_bytes(16, 65, 256) == 0
    assert B.bfly_kron_backward_workspace_bytes(16, 5, 8192) == 0
    assert B.bfly_kron_backward_workspace_bytes(16, 32, 4096) == 0         # m * nb > 65536
    assert B.bfly_kron_backward_workspace_bytes(16, 43, 256) > B.bfly_backward_workspace_bytes(16 * 43, 256)
    assert kb(L, x=None) == NULL
    assert kb(L, mix=None) == NULL
    assert kb(L, dth=None) == NULL
    assert kb(L, th=None, co=None) == NULL
    assert kb(L, ws=None) == NULL
    assert kb(L, rows=-1, wsb=1 << 30) == SIZE
    assert kb(L, m=0, wsb=1 << 30) == SIZE
    assert kb(L, m=65, wsb=1 << 30) == SIZE
    assert kb(L, nb=1000, wsb=1 << 30) == SIZE
    assert kb(L, m=1, wsb=1 << 30) == UNSUPPORTED
    assert kb(L, m=32, nb=4096, wsb=1 << 30) == UNSUPPORTED  # m * nb > 65536
    assert kb(L, nb=128, wsb=1 << 30) == UNSUPPORTED
    # wide composites pass the size checks (and reach the workspace check,
    # the last before any HIP call)
    assert kb(L, m=43, nb=256, wsb=B.bfly_kron_backward_workspace_bytes(16, 43, 256) - 1) == WORKSPACE
    assert kb(L, m=9, nb=512, wsb=B.bfly_kron_backward_workspace_bytes(16, 9, 512) - 1) == WORKSPACE
    assert kb(L, wsb=B.bfly_kron_backward_workspace_bytes(16, 5, 1024) - 1) == WORKSPACE
    assert kb(L, dx=ctypes.c_void_p(0x20008)) == ALIGN
    assert kb(L, ws=ctypes.c_void_p(0x80008)) == ALIGN


def kw(L, x=X, y=Y, c=C, s=S, z=None, rows=16, m=43, nb=256, th=TH, co=None, mix=MIX, ws=WS,
       wsb=None, group=128, xd=1, yd=1):
    if wsb is None:
        wsb = B.bfly_kron_forward_wide_workspace_bytes(max(rows, 0), m, nb)
    return L.bfly_kron_forward_wide(x, xd, y, yd, c, s, z, rows, m, nb, th, co, mix, 4, group, 0,
                                    ws, wsb, None)


def test_kron_forward_wide_validation(L):
    tab = (B.bfly_coeff_bytes(256) + 255) // 256 * 256
    assert B.bfly_kron_forward_wide_workspace_bytes(16, 43, 256) == tab + 16 * 11008 * 4
    assert B.bfly_kron_forward_wide_workspace_bytes(16, 65, 256) == 0
    assert B.bfly_kron_forward_wide_workspace_bytes(16, 43, 128) == 0
    assert B.bfly_kron_forward_wide_workspace_bytes(16, 32, 4096) == 0    # m * nb > 65536
    assert kw(L, rows=0) == OK
    assert kw(L, x=None) == NULL
    assert kw(L, mix=None) == NULL
    assert kw(L, ws=None) == NULL
    assert kw(L, th=None, co=None) == NULL
    assert kw(L, c=None) == QUANT                      # scales without codes
    assert kw(L, xd=5) == DTYPE
    assert kw(L, m=1, wsb=1 << 30) == SIZE
    assert kw(L, m=65, wsb=1 << 30) == SIZE
    assert kw(L, nb=300, wsb=1 << 30) == SIZE
    assert kw(L, nb=128, wsb=1 << 30) == UNSUPPORTED
    assert kw(L, group=512) == QUANT                   # group must divide nb
    assert kw(L, wsb=tab + 16 * 11008 * 4 - 1) == WORKSPACE
    assert kw(L, ws=ctypes.c_void_p(0x80008)) == ALIGN


def test_calib_step_validation(L):
    cfg = B.bfly_calib_config(4, 128, 16, 0.1, 1e-3, 0.9, 0.999, 1e-8)
    wsb = B.bfly_calib_workspace_bytes(64, 4096)
    assert wsb > 64 * 4096 * 4 + B.bfly_backward_workspace_bytes(64, 4096)
    assert B.bfly_calib_workspace_bytes(0, 4096) == 0
    assert B.bfly_calib_workspace_bytes(64, 8192) == 0

    def cs(x=X, rows=64, n=4096, th=TH, m=C, v=S, step=1, c=cfg, loss=Z, ws=WS, wsb=wsb):
        return L.bfly_calib_step(x, rows, n, th, m, v, step, ctypes.byref(c) if c else None, loss,
                                 ws, wsb, None)
    assert cs(x=None) == NULL
    assert cs(c=None) == NULL
    assert cs(loss=None) == NULL
    assert cs(rows=0) == SIZE
    assert cs(step=0) == SIZE
    assert cs(n=100) == SIZE
    assert cs(n=8192) == UNSUPPORTED
    assert cs(c=B.bfly_calib_config(3, 128, 16, 0.1, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cs(c=B.bfly_calib_config(4, 96, 16, 0.1, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cs(c=B.bfly_calib_config(4, 128, 33, 0.1, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cs(wsb=wsb - 1) == WORKSPACE
    assert cs(ws=ctypes.c_void_p(0x80008)) == ALIGN


def test_calib_step_weight_validation(L):
    cfg = B.bfly_calib_weight_config(2, 128, 1, 16, 0.05, 1e-3, 0.9, 0.999, 1e-8)
    wsb = B.bfly_calib_step_weight_workspace_bytes(64, 256, 4096)
    assert wsb > 64 * 4096 * 4 * 2 + 256 * 4096 * 4 + 64 * 256 * 4
    assert B.bfly_calib_step_weight_workspace_bytes(0, 256, 4096) == 0
    assert B.bfly_calib_step_weight_workspace_bytes(64, 250, 4096) == 0     # out % 16
    assert B.bfly_calib_step_weight_workspace_bytes(64, 256, 8192) == 0
    assert B.bfly_calib_step_weight_workspace_bytes(64, 65536 + 16, 1024) == 0

    def cw(x=X, rows=64, w=Y, wd=1, out=256, n=4096, th=TH, m=C, v=S, step=1, c=cfg, loss=Z,
           ws=WS, wsb=wsb):
        return L.bfly_calib_step_weight(x, rows, w, wd, out, n, th, m, v, step,
                                        ctypes.byref(c) if c else None, loss, ws, wsb, None)
    assert cw(x=None) == NULL
    assert cw(w=None) == NULL
    assert cw(c=None) == NULL
    assert cw(ws=None) == NULL
    assert cw(wd=7) == DTYPE
    assert cw(rows=0) == SIZE
    assert cw(step=0) == SIZE
    assert cw(n=100) == SIZE
    assert cw(n=8192) == UNSUPPORTED
    assert cw(out=100) == UNSUPPORTED                 # not a multiple of 16
    assert cw(c=B.bfly_calib_weight_config(3, 128, 1, 16, 0.05, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cw(c=B.bfly_calib_weight_config(2, 96, 1, 16, 0.05, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cw(c=B.bfly_calib_weight_config(2, 128, 2, 16, 0.05, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cw(c=B.bfly_calib_weight_config(2, 128, 1, 12, 0.05, 1e-3, 0.9, 0.999, 1e-8)) == QUANT
    assert cw(wsb=wsb - 1) == WORKSPACE
    assert cw(ws=ctypes.c_void_p(0x80008)) == ALIGN
    assert cw(w=ctypes.c_void_p(0x20004)) == ALIGN
