"""GPU side of reading R15: the attention kernel's own P conversion (p4_e4m3:
one fused multiply-add onto the 2^-11 grid, v_exp_f32, round-to-nearest-even
E4M3 conversion) gives the exactly rounded E4M3 code of 2^x at every grid point
a low-bit tile can produce, so P is bit-identical to the oracle's.

ThriftAttention (abstract): low-bit and FP16 blocks merge through one online
softmax; the pages fix no exponent, so the kernel and the oracle share the
grid-snapped one of R15, and this test checks the GPU half of that contract.
"""

import ctypes

import numpy as np
import pytest

from gpu_helpers import gpu_or_skip, load_test_kernels
from oracle import formats as F
from oracle.attention import softmax_scale_log2

pytestmark = pytest.mark.gpu


def _gpu_codes(s, c, off):
    """E4M3 codes from p4_e4m3 for scores s (groups of 4 share c and off)."""
    import torch

    lib = load_test_kernels()
    n4 = s.size // 4
    ts = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).cuda()
    tc = torch.from_numpy(np.ascontiguousarray(c, dtype=np.float32)).cuda()
    to = torch.from_numpy(np.ascontiguousarray(off, dtype=np.float32)).cuda()
    out = torch.empty(n4, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.mxqt_p_codes(ts.data_ptr(), tc.data_ptr(), to.data_ptr(), n4, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32).view(np.uint8).reshape(-1)  # byte i = score i


def test_every_grid_point_matches_the_exact_code():
    """Every x on the 2^-11 grid in [-12, 8.5] (c = 1, reference 8, so the
    fused multiply-add returns 6144 + x and the kernel evaluates 2^x): the
    code equals the exactly rounded one.  Below -10 every code is 0; the
    kernel's exponent never exceeds 8 + 2^-11 for references below 2^12, and
    8.5 covers references up to 2^14."""
    gpu_or_skip()
    xs = np.arange(-12 * 2048, int(8.5 * 2048) + 1, dtype=np.int64).astype(np.float32) / np.float32(2048.0)
    pad = (-xs.size) % 4
    xs = np.concatenate([xs, np.full(pad, -12.0, np.float32)])
    n4 = xs.size // 4
    got = _gpu_codes(xs, np.ones(n4, np.float32), np.full(n4, F.P_GRID_MAGIC, np.float32))
    want = F.p_e4m3_code(xs.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} grid points differ, first x = {xs[bad[:5]]}"


@pytest.mark.parametrize("seed", [0, 1])
def test_random_scores_references_and_scales(seed):
    """The whole step on random inputs: scores s, the logit scale c of head_dim
    64 / 128 or a random one, integer references m at or above the row's
    snapped maximum; codes equal the oracle's p_e4m3_code(p_exponent_grid)."""
    gpu_or_skip()
    rng = np.random.default_rng(seed)
    n4 = 1 << 18
    s = (rng.standard_normal(4 * n4) * rng.choice([1.0, 10.0, 80.0], size=4 * n4)).astype(np.float32)
    cs = np.array([softmax_scale_log2(64), softmax_scale_log2(128)], np.float32)
    c = np.where(rng.random(n4) < 0.5, cs[rng.integers(0, 2, n4)],
                 rng.uniform(0.01, 0.5, n4).astype(np.float32)).astype(np.float32)
    s4 = s.reshape(n4, 4)
    top = np.ceil((s4.max(axis=1).astype(np.float64) * c).astype(np.float32))  # ceil(fl32(max * c))
    m = (top + rng.integers(0, 24, n4)).astype(np.float32)
    off = ((F.P_GRID_MAGIC + np.float32(F.P_EXP_OFFSET)) - m).astype(np.float32)
    got = _gpu_codes(s, c, off)
    xq = F.p_exponent_grid(s4, c[:, None], m[:, None]).reshape(-1)
    want = F.p_e4m3_code(xq.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} of {got.size} codes differ"
