"""GPU parity for the fused RMS normalisation + MXFP8 quantiser (jfa_rmsnorm_quantize_mxfp8)
against the oracle's fp64 ``rmsnorm`` followed by its ``mxfp8_quantize``.

The codes are integers decided by floating point. The kernel forms y in fp32: the sum of
squares takes at most 8 + 6 roundings of positive terms, then come the square root, the
division and two products. So |y_fp32 / y - 1| <= 2^-18, with room to spare. A code or a
scale may therefore differ from the fp64 decision only where y, or a block's amax, lies within
that bound of a rounding boundary. The test accepts exactly the decisions that the oracle takes
on y(1 - 2^-18) or y(1 + 2^-18), and asks that such cases are rare.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu
DELTA = 2.0 ** -18


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


def _check(x, w, n, eps, codes, scales):
    y = oracle.rmsnorm(x.float(), None if w is None else w.cpu(), n=n, eps=eps)
    ref = [oracle.mxfp8_quantize(y * f) for f in (1.0, 1.0 - DELTA, 1.0 + DELTA)]
    c = codes.cpu().numpy()
    s = scales.cpu().numpy()
    ok_s = np.zeros(s.shape, bool)
    ok_c = np.zeros(c.shape, bool)
    for rc, rs in ref:
        ok_s |= s == rs
        ok_c |= c == rc
    off_c = int(np.count_nonzero(c != ref[0][0]))
    off_s = int(np.count_nonzero(s != ref[0][1]))
    say(f"  codes off the fp64 decision: {off_c} of {c.size}; scales: {off_s} of {s.size}")
    assert ok_s.all() and ok_c.all()
    assert off_c <= max(2, c.size // 10000) and off_s <= max(1, s.size // 10000)
    # and the decoded values are y to E4M3's precision: half a step (2^-4 relative) in the
    # normal range below the saturation value 448, exactly +-448 above it
    table = np.array([oracle.e4m3_decode(i) for i in range(256)])
    unit = np.exp2(np.repeat(s.reshape(s.shape[0], -1), 32, axis=1).reshape(c.shape)
                   .astype(np.float64) - 127)
    deq = table[c] * unit
    ys = np.abs(y) / unit
    normal = (ys >= 2.0 ** -6) & (ys < 448.0)
    assert np.all(np.abs(deq - y)[normal] <= 2.0 ** -4 * np.abs(y)[normal] * (1 + 4 * DELTA))
    sat = ys >= 448.0 * (1 + DELTA)
    assert np.all(np.abs(deq[sat]) == 448.0 * unit[sat])


@pytest.mark.parametrize("n", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("gain", [False, True])
def test_norm_quant_parity(n, gain):
    import jagged_attention_amd as jfa
    g = torch.Generator().manual_seed(100 + n)
    groups = 3001                                    # not a multiple of a workgroup's groups
    x = (torch.randn(groups, n, generator=g) * torch.exp(torch.randn(groups, 1, generator=g)))
    x[5] = 0.0                                       # an all-zero group: y = 0, scale code 127
    x[7, :] = 3.0                                    # a constant group: y = 3 / sqrt(9 + eps)
    x = x.to(torch.bfloat16)
    w = (1.0 + 0.5 * torch.randn(n, generator=g)).float() if gain else None
    say(f"[norm+quant] n={n} gain={gain}")
    xd = x.cuda()
    wd = None if w is None else w.cuda()
    codes, scales = jfa.rmsnorm_quantize_mxfp8(xd.view(-1, n), wd, n=n, eps=1e-6)
    torch.cuda.synchronize()
    assert int(scales[5].min()) == 127 and int(codes[5].max()) == 0
    _check(x, w, n, 1e-6, codes, scales)


def test_norm_quant_per_head_layout():
    """Attention inputs [rows, H, d]: one group per (row, head), n = d."""
    import jagged_attention_amd as jfa
    g = torch.Generator().manual_seed(9)
    x = torch.randn(777, 4, 128, generator=g).to(torch.bfloat16)
    say("[norm+quant] per head [777, 4, 128]")
    codes, scales = jfa.rmsnorm_quantize_mxfp8(x.cuda(), None, n=128, eps=1e-5)
    torch.cuda.synchronize()
    assert codes.shape == (777, 4, 128) and scales.shape == (777, 4, 4)
    _check(x.reshape(-1, 128), None, 128, 1e-5, codes.reshape(-1, 128), scales.reshape(-1, 4))


def test_norm_quant_rejects_bad_sizes():
    import jagged_attention_amd as jfa
    x = torch.zeros(4, 96, dtype=torch.bfloat16).cuda()
    c = torch.empty(4, 96, dtype=torch.uint8).cuda()
    s = torch.empty(4, 3, dtype=torch.uint8).cuda()
    with pytest.raises(jfa.JfaError):
        jfa.jfa_rmsnorm_quantize_mxfp8(x, None, 4, 96, 1e-6, c, s)
    with pytest.raises(jfa.JfaError):
        jfa.jfa_rmsnorm_quantize_mxfp8(x, None, 4, 32, -1.0, c, s)
