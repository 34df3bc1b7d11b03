"""GPU side of readings R2-R5: the quantisers' element conversions give the
exactly rounded code of every value a block-scaled bf16 element can take.
  - E2M1 (Q and K): e2m1_pack8, gfx950's packed FP4 conversion, unit scale;
  - E4M3 (V): e4m3_pack4, a clamp to +-448 and the packed FP8 conversion.

ThriftAttention (abstract): Q and K are quantised to 4-bit and V to 8-bit
block-scaled floats; an element x of a block with shared exponent e becomes
the code of x * 2^-e, a value with at most 8 significant bits, so every such
value is itself bf16-representable and the 65536 bf16 bit patterns cover them
all.
"""

import ctypes

import numpy as np
import pytest

from gpu_helpers import gpu_or_skip, load_test_kernels
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _finite_bf16_values(multiple):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_bits_to_f32(bits)
    v = v[np.isfinite(v)]
    pad = (-v.size) % multiple
    return np.concatenate([v, np.zeros(pad, np.float32)]).astype(np.float32)


def test_every_bf16_value_matches_the_exact_code():
    """All finite bf16 values (both signs, zeros and subnormals included), as
    fp32 inputs: nibble i of word j is the code of value 8 j + i, equal to
    oracle.formats.e2m1_round_code (nearest, ties to even, saturating at 6,
    sign copied)."""
    gpu_or_skip()
    import torch

    v = _finite_bf16_values(8)
    n8 = v.size // 8
    lib = load_test_kernels()
    tv = torch.from_numpy(v).cuda()
    out = torch.empty(n8, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.mxqt_e2m1_codes(tv.data_ptr(), n8, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    words = out.cpu().numpy().view(np.uint32)
    got = ((words[:, None] >> (4 * np.arange(8, dtype=np.uint32))[None, :]) & 0xF).astype(np.uint8).reshape(-1)
    want = F.e2m1_round_code(v.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} values differ, e.g. v={v[bad[:6]]} got={got[bad[:6]]} want={want[bad[:6]]}"


def test_every_bf16_value_matches_the_exact_e4m3_code():
    """All finite bf16 values as fp32 inputs: byte i of word j is the code of
    value 4 j + i, equal to oracle.formats.e4m3_round_code (nearest, ties to
    even, saturating at 448, subnormals k * 2^-9, sign copied)."""
    gpu_or_skip()
    import torch

    v = _finite_bf16_values(4)
    n4 = v.size // 4
    lib = load_test_kernels()
    tv = torch.from_numpy(v).cuda()
    out = torch.empty(n4, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.mxqt_e4m3_codes(tv.data_ptr(), n4, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).view(np.uint8).reshape(-1)  # byte i = value i (little endian)
    want = F.e4m3_round_code(v.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} values differ, e.g. v={v[bad[:6]]} got={got[bad[:6]]} want={want[bad[:6]]}"
