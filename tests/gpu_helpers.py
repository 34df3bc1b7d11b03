"""Shared helpers for the GPU parity tests (not a test module)."""

import ctypes
import os

import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def gpu_or_skip():
    if torch is None or not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_mixed_precision_mxq_amd as mxq

    mxq.load_library()  # raises if the library is missing: no silent fallback
    return mxq


def bf16_dev(bits: np.ndarray):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on cuda:0 (bit copy)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def u8(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def u16(t) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u32(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def random_bf16(shape, seed, scale=1.0, specials=True):
    """N(0,1)*scale bf16 bits, with some special values mixed in: zeros,
    negative zeros, subnormals, large and tiny magnitudes, exact E2M1 grid
    points and exact midpoints."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    if specials:
        flat = x.reshape(-1)
        n = flat.size
        idx = rng.choice(n, size=max(1, n // 50), replace=False)
        pool = np.array([0.0, -0.0, 1e-40, -3e-39, 6.0, 5.0, -2.5, 0.75, 1.25, 3.5, 448.0, 464.0,
                         1e30, -7e-20, 0.25, -0.25, 1.75], dtype=np.float32)
        flat[idx] = pool[rng.integers(0, len(pool), size=len(idx))]
    b = x.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def load_test_kernels():
    """The test-only kernel library (tests/hip/libmxq_testkernels.so, built by
    __graft_entry__.build() or tests/hip/build_test_kernels.py)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libmxq_testkernels.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run python tests/hip/build_test_kernels.py")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.mxqt_p_codes.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp]
    lib.mxqt_p_codes.restype = ctypes.c_int
    lib.mxqt_e2m1_codes.argtypes = [vp, ctypes.c_int, vp, vp]
    lib.mxqt_e2m1_codes.restype = ctypes.c_int
    lib.mxqt_e4m3_codes.argtypes = [vp, ctypes.c_int, vp, vp]
    lib.mxqt_e4m3_codes.restype = ctypes.c_int
    lib.mxqt_fill_lds.argtypes = [ctypes.c_uint32, ctypes.c_int, vp, vp]
    lib.mxqt_fill_lds.restype = ctypes.c_int
    return lib


def poison_lds(word):
    """Fill the LDS of every CU with a 32-bit pattern, on torch's current
    stream, so that the next kernel starts on stale LDS contents."""
    lib = load_test_kernels()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert lib.mxqt_fill_lds(ctypes.c_uint32(word), 4 * n_cu, ctypes.c_void_p(sink.data_ptr()), st) == 0
