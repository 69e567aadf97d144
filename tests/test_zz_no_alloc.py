"""bfly_forward_quant_noalloc (the table in the library's fixed scratch, no
allocation) against bfly_forward_quant with a caller workspace: the same
outputs bit for bit, on two calls in a row, the second with a smaller input
(n = 4096, then n = 1024 with fewer rows: the scratch keeps the first call's
larger table and the second must not depend on it), and against the oracle.
Both entry points are called through the C ABI."""
import numpy as np
import pytest

import oracle
import learnable_butterfly_rotation_amd as B
from learnable_butterfly_rotation_amd import inputs

from parity import check_bf16, check_quant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.element_size() == 2 \
        else t.cpu().numpy()


def _outputs(rows, n, bits, group, mode):
    y = torch.full((rows, n), 7.0, dtype=torch.bfloat16, device="cuda")
    codes = torch.full((rows, n * bits // 8), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, n // group), 3.0, dtype=torch.float16, device="cuda")
    zeros = torch.full((rows, n // group), 3.0, dtype=torch.float16, device="cuda") if mode else None
    return y, codes, scales, zeros


@pytest.mark.parametrize("first,second", [((4096, 300, 4, 128, 0), (1024, 77, 2, 64, 1)),
                                          ((2048, 129, 2, 128, 1), (256, 5, 4, 32, 0))])
def test_noalloc_matches_workspace_call(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = B.lib()
    rng = np.random.default_rng(4242 + first[0])
    for n, rows, bits, group, mode in (first, second):
        th = inputs.angles(rng, n)
        x = inputs.f32_to_bf16_bits((rng.standard_normal((rows, n)) * 2).astype(np.float32))
        xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        thd = torch.from_numpy(th).cuda()
        ws = torch.empty(B.bfly_coeff_bytes(n), dtype=torch.uint8, device="cuda")
        sh = torch.cuda.current_stream().cuda_stream
        ref = _outputs(rows, n, bits, group, mode)
        got = _outputs(rows, n, bits, group, mode)
        ptr = lambda t: None if t is None else t.data_ptr()
        st = L.bfly_forward_quant(xd.data_ptr(), B.BFLY_BF16, ref[0].data_ptr(), B.BFLY_BF16,
                                  ref[1].data_ptr(), ref[2].data_ptr(), ptr(ref[3]), rows, n,
                                  thd.data_ptr(), None, bits, group, mode, ws.data_ptr(),
                                  ws.numel(), sh)
        assert st == 0, st
        st = L.bfly_forward_quant_noalloc(xd.data_ptr(), B.BFLY_BF16, got[0].data_ptr(),
                                          B.BFLY_BF16, got[1].data_ptr(), got[2].data_ptr(),
                                          ptr(got[3]), rows, n, thd.data_ptr(), bits, group, mode,
                                          sh)
        assert st == 0, st
        for a, b in zip(ref, got):
            if a is not None:
                assert np.array_equal(_bits(a), _bits(b))
        y64 = oracle.forward(x, th)
        xl2 = np.linalg.norm(inputs.bf16_bits_to_f32(x).reshape(rows, n).astype(np.float64), axis=1)
        r = check_bf16(_bits(got[0]), y64, xl2, n)
        assert r["ok"], r
        r = check_quant(y64, _bits(got[1]), _bits(got[2]),
                        _bits(got[3]) if got[3] is not None else None, bits, group, mode)
        assert r["ok"], r


def test_noalloc_rejects_sizes_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = B.lib()
    # n = 8192 is beyond the scratch; nothing is launched
    st = L.bfly_forward_quant_noalloc(0x10000, 1, 0x20000, 1, 0x30000, 0x40000, None, 4, 8192,
                                      0x60000, 4, 128, 0, None)
    assert st == 7, st   # BFLY_ERR_UNSUPPORTED
