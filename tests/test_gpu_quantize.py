"""GPU parity: mxq_quantize codes and scales are bit-exact against the oracle."""

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip, random_bf16, u8, u16
import mxq_inputs
from oracle import formats as F

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 2, 256, 64, 256),
    (2, 3, 384, 128, 301),      # ragged n_valid, several tiles
    (1, 1, 128, 32, 1),         # single valid row
]


def _zero_pad(x32, n_valid):
    x32 = x32.copy()
    x32[..., n_valid:, :] = 0
    return x32


@pytest.mark.parametrize("shape", SHAPES)
def test_mxfp4_bit_exact(shape):
    mxq = gpu_or_skip()
    B, H, N, D, nv = shape
    bits = random_bf16((B, H, N, D), seed=N + D, scale=3.0)
    codes, scales, _ = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_MXFP4_E2M1, mxq.MXQ_AXIS_D, nv)
    rc, rs = F.quantize_mxfp4(_zero_pad(F.bf16_bits_to_f32(bits), nv))
    assert np.array_equal(u8(codes), F.pack_nibbles(rc))
    assert np.array_equal(u8(scales), rs)


@pytest.mark.parametrize("shape", SHAPES[:2])
def test_mxfp8_keys_bit_exact(shape):
    mxq = gpu_or_skip()
    B, H, N, D, nv = shape
    bits = random_bf16((B, H, N, D), seed=7 + N, scale=2.0)
    codes, scales, _ = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_MXFP8_E4M3, mxq.MXQ_AXIS_N, nv)
    rc, rs = F.quantize_mxfp8_keys(_zero_pad(F.bf16_bits_to_f32(bits), nv))
    assert np.array_equal(u8(codes), rc)
    assert np.array_equal(u8(scales), rs)


@pytest.mark.parametrize("axis", [0, 1])
def test_fp16_copy_bit_exact(axis):
    mxq = gpu_or_skip()
    bits = random_bf16((2, 2, 256, 128), seed=11, scale=100.0)
    out, _, _ = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_FP16, axis, 250)
    ref = _zero_pad(F.bf16_bits_to_f32(bits), 250).astype(np.float16)
    if axis == 1:
        ref = np.ascontiguousarray(np.swapaxes(ref, -1, -2))
    assert np.array_equal(u16(out), ref.view(np.uint16))


# V^T layouts along N: the LDS-transpose path (D <= 256, blocks of 64 keys, or
# 32 when N is not a multiple of 64) and the per-tile path (D > 256).
VT_SHAPES = [
    (2, 3, 96, 64, 77),         # fp16 only: N % 64 != 0
    (1, 2, 192, 256, 192),      # widest head dim of the transpose path
    (1, 1, 128, 288, 100),      # per-tile path
    (4, 6, 256, 64, 200),       # many (b, h) pairs, ragged
]


@pytest.mark.parametrize("shape", VT_SHAPES)
def test_vt_layouts_bit_exact(shape):
    mxq = gpu_or_skip()
    B, H, N, D, nv = shape
    bits = random_bf16((B, H, N, D), seed=3 * N + D, scale=5.0)
    x32 = _zero_pad(F.bf16_bits_to_f32(bits), nv)
    out, _, _ = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_FP16, mxq.MXQ_AXIS_N, nv)
    ref = np.ascontiguousarray(np.swapaxes(x32.astype(np.float16), -1, -2))
    assert np.array_equal(u16(out), ref.view(np.uint16))
    if N % 128 == 0:
        codes, scales, _ = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_MXFP8_E4M3, mxq.MXQ_AXIS_N, nv)
        rc, rs = F.quantize_mxfp8_keys(x32)
        assert np.array_equal(u8(codes), rc)
        assert np.array_equal(u8(scales), rs)


def test_int4_g32_bit_exact():
    mxq = gpu_or_skip()
    bits = random_bf16((2, 2, 320, 128), seed=13, scale=1.5)
    bits[0, 0, 5, :32] = bits[0, 0, 5, 0]  # constant group -> zero scale
    codes, sc, zr = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_INT4_ASYM_G32, mxq.MXQ_AXIS_D, 300)
    rc, rs, rz = F.quantize_int4_g32(_zero_pad(F.bf16_bits_to_f32(bits), 300))
    assert np.array_equal(u8(codes), F.pack_nibbles(rc))
    assert np.array_equal(u16(sc), rs.view(np.uint16))
    assert np.array_equal(u16(zr), rz.view(np.uint16))


def test_full_size_llama8b_operands_bit_exact():
    """Q, K (MXFP4) and V (MXFP8) of the Llama-8B-shaped workload at full size."""
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b")
    for name, fmt, axis in (("q", mxq.MXQ_MXFP4_E2M1, 0), ("k", mxq.MXQ_MXFP4_E2M1, 0),
                            ("v", mxq.MXQ_MXFP8_E4M3, 1)):
        codes, scales, _ = mxq.mxq_quantize(bf16_dev(cfg[name]), fmt, axis, cfg["n_valid"])
        x32 = F.bf16_bits_to_f32(cfg[name])
        if fmt == mxq.MXQ_MXFP4_E2M1:
            rc, rs = F.quantize_mxfp4(x32)
            rc = F.pack_nibbles(rc)
        else:
            rc, rs = F.quantize_mxfp8_keys(x32)
        assert np.array_equal(u8(codes), rc), name
        assert np.array_equal(u8(scales), rs), name


def test_error_paths_return_status():
    mxq = gpu_or_skip()
    import torch

    x = torch.zeros((1, 1, 64, 48), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mxq.MxqError) as ei:
        mxq.mxq_quantize(x, mxq.MXQ_MXFP4_E2M1, mxq.MXQ_AXIS_D)
    assert ei.value.status == mxq.MXQ_EUNSUPPORTED
    y = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mxq.MxqError) as ei:
        mxq.mxq_quantize(y, mxq.MXQ_MXFP4_E2M1, mxq.MXQ_AXIS_N)
    assert ei.value.status == mxq.MXQ_EUNSUPPORTED


@pytest.mark.parametrize("shape", [(1, 2, 256, 128, 256), (2, 3, 384, 64, 301), (1, 1, 128, 32, 77),
                                   (1, 2, 128, 256, 128)])
def test_mxfp4_hadamard_bit_exact(shape):
    """MXFP4 of Walsh-Hadamard-rotated rows (with special values mixed in)."""
    mxq = gpu_or_skip()
    B, H, N, D, nv = shape
    bits = random_bf16((B, H, N, D), seed=5 * N + D, scale=3.0)
    bits[..., 3] = F.f32_to_bf16_bits(np.float32(40.0))  # an outlier channel
    codes, scales, _ = mxq.mxq_quantize(bf16_dev(bits), mxq.MXQ_MXFP4_E2M1_HADAMARD, mxq.MXQ_AXIS_D, nv)
    rc, rs = F.quantize_mxfp4(F.hadamard_rotate(_zero_pad(F.bf16_bits_to_f32(bits), nv)))
    assert np.array_equal(u8(codes), F.pack_nibbles(rc))
    assert np.array_equal(u8(scales), rs)


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 1, 384, 128, 301), (2, 2, 2, 256, 64, 256)])
def test_prefill_operands_equal_the_separate_calls(shape, rotate):
    """mxq_prefill_operands (Q and K in one launch, V's MXFP8 and fp16 copies
    from one read) writes what the per-tensor mxq_quantize calls write."""
    mxq = gpu_or_skip()
    B, Hq, Hkv, N, D, nv = shape
    q = bf16_dev(random_bf16((B, Hq, N, D), seed=N + 1, scale=2.0))
    k = bf16_dev(random_bf16((B, Hkv, N, D), seed=N + 2, scale=2.0))
    v = bf16_dev(random_bf16((B, Hkv, N, D), seed=N + 3, scale=2.0))
    ops = mxq.prepare_prefill(q, k, v, nv, rotate=rotate)
    f4 = mxq.MXQ_MXFP4_E2M1_HADAMARD if rotate else mxq.MXQ_MXFP4_E2M1
    for got, ref in ((ops.q_codes, mxq.mxq_quantize(q, f4, 0, nv)[0]), (ops.q_scales, mxq.mxq_quantize(q, f4, 0, nv)[1]),
                     (ops.k_codes, mxq.mxq_quantize(k, f4, 0, nv)[0]), (ops.k_scales, mxq.mxq_quantize(k, f4, 0, nv)[1]),
                     (ops.v_codes, mxq.mxq_quantize(v, mxq.MXQ_MXFP8_E4M3, 1, nv)[0]),
                     (ops.v_scales, mxq.mxq_quantize(v, mxq.MXQ_MXFP8_E4M3, 1, nv)[1])):
        assert np.array_equal(u8(got), u8(ref))
    assert np.array_equal(u16(ops.v_f16t), u16(mxq.mxq_quantize(v, mxq.MXQ_FP16, 1, nv)[0]))
    low = mxq.prepare_prefill(q, k, v, nv, mode=mxq.MXQ_ALL_LOWBIT)
    assert low.v_f16t is None and np.array_equal(u8(low.v_codes), u8(ops.v_codes))
    hi = mxq.prepare_prefill(q, k, v, nv, mode=mxq.MXQ_ALL_FP16)
    assert hi.q_codes is None and np.array_equal(u16(hi.v_f16t), u16(ops.v_f16t))
