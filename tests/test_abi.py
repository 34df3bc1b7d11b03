"""C ABI checks that need no GPU: the library loads, exports every function
include/mxq.h declares, sizes workspaces, and rejects bad arguments on the
host before anything is launched."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")
LIB = os.path.join(ROOT, "bit_mixed_precision_mxq_amd", "libmxq.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*((?:mxq|attn)_\w+)\s*\(", text, flags=re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmxq.so is not built (run __graft_entry__.build())")
    import bit_mixed_precision_mxq_amd as mxq

    return mxq, mxq.load_library()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert {"mxq_quantize", "attn_select_blocks", "attn_mixed_fwd", "attn_quantkv_decode"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    missing = declared - exported
    assert not missing, missing
    mxq, so = lib
    for name in declared:
        assert hasattr(so, name)
    assert set(mxq.EXPORTED) == declared


def test_status_strings_and_version(lib):
    mxq, so = lib
    assert so.mxq_status_string(0) == b"MXQ_OK"
    assert b"EINVAL" in so.mxq_status_string(1)
    assert b"gfx950" in so.mxq_version()


def test_workspace_sizes(lib):
    mxq, so = lib
    s = mxq.AttnShape(1, 32, 8, 8192, 8192, 128, 128, 64, 1)
    n = so.attn_select_blocks_workspace(ctypes.byref(s))
    assert n == (1 * 32 * 64 + 1 * 8 * 128) * 128 * 4
    # INT4 splits plus one for the fp16 sink and recent tokens; the default is
    # one split per 4096 cached tokens
    assert so.attn_quantkv_decode_workspace(64, 32, 128, 16, 32768) == 64 * 32 * 17 * 130 * 4
    assert so.attn_quantkv_decode_workspace(64, 32, 128, 0, 32768) == 64 * 32 * 9 * 130 * 4


def test_host_validation_rejects_before_launch(lib):
    mxq, so = lib
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    st = so.mxq_quantize(None, 1, 1, 64, 64, 64, mxq.MXQ_MXFP4_E2M1, mxq.MXQ_AXIS_D, fake, fake, None, None)
    assert st == mxq.MXQ_EINVAL and b"null" in so.mxq_last_error()
    st = so.mxq_quantize(fake, 1, 1, 64, 48, 64, mxq.MXQ_MXFP4_E2M1, mxq.MXQ_AXIS_D, fake, fake, None, None)
    assert st == mxq.MXQ_EUNSUPPORTED
    st = so.mxq_quantize(fake, 1, 1, 64, 64, 65, mxq.MXQ_MXFP4_E2M1, mxq.MXQ_AXIS_D, fake, fake, None, None)
    assert st == mxq.MXQ_EINVAL
    st = so.mxq_quantize(fake, 1, 1, 64, 64, 64, mxq.MXQ_MXFP8_E4M3, mxq.MXQ_AXIS_D, fake, fake, None, None)
    assert st == mxq.MXQ_EUNSUPPORTED
    bad_d = mxq.AttnShape(1, 2, 2, 256, 256, 96, 64, 64, 0)
    p = mxq.SelectParams(1, 0, 1, 0, 0)
    st = so.attn_select_blocks(fake, fake, ctypes.byref(bad_d), ctypes.byref(p), fake, 1 << 20, fake, None, None, None)
    assert st == mxq.MXQ_EUNSUPPORTED
    gqa = mxq.AttnShape(1, 3, 2, 256, 256, 64, 64, 64, 0)
    st = so.attn_select_blocks(fake, fake, ctypes.byref(gqa), ctypes.byref(p), fake, 1 << 20, fake, None, None, None)
    assert st == mxq.MXQ_EINVAL
    ok = mxq.AttnShape(1, 2, 2, 256, 256, 64, 64, 64, 0)
    st = so.attn_select_blocks(fake, fake, ctypes.byref(ok), ctypes.byref(p), fake, 16, fake, None, None, None)
    assert st == mxq.MXQ_EINVAL and b"workspace" in so.mxq_last_error()
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, None, None, 0, ctypes.byref(ok),
                           0.0, mxq.MXQ_MIXED, fake, 0, None, None)
    assert st == mxq.MXQ_EINVAL and b"mask" in so.mxq_last_error()
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, fake, None, 0, ctypes.byref(ok),
                           0.0, mxq.MXQ_ALL_FP16, fake, 0, None, None)
    assert st == mxq.MXQ_EINVAL
    # vertical lines: at most 16, and they need the bf16/fp16 operands
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, fake, fake, fake, None, fake, fake, 17, ctypes.byref(ok),
                           0.0, mxq.MXQ_MIXED, fake, 0, None, None)
    assert st == mxq.MXQ_EINVAL and b"n_lines" in so.mxq_last_error()
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, None, fake, 4, ctypes.byref(ok),
                           0.0, mxq.MXQ_ALL_LOWBIT, fake, 0, None, None)
    assert st == mxq.MXQ_EINVAL and b"lines" in so.mxq_last_error()
    # MIXED needs fp16 V^T, or bf16 V when no tile is promoted
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, fake, fake, None, None, fake, None, 0, ctypes.byref(ok),
                           0.0, mxq.MXQ_MIXED, fake, 0, None, None)
    assert st == mxq.MXQ_EINVAL and b"bf16 V" in so.mxq_last_error()
    # one workgroup per kv group: G = Hq / Hkv in {2, 4} and N > 256
    gh = mxq.MXQ_ALL_LOWBIT | mxq.MXQ_GROUP_HEADS
    long_g1 = mxq.AttnShape(1, 2, 2, 512, 512, 64, 64, 64, 0)
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, None, None, 0,
                           ctypes.byref(long_g1), 0.0, gh, fake, 0, None, None)
    assert st == mxq.MXQ_EUNSUPPORTED and b"GROUP_HEADS" in so.mxq_last_error()
    short_g2 = mxq.AttnShape(1, 4, 2, 256, 256, 64, 64, 64, 0)
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, None, None, 0,
                           ctypes.byref(short_g2), 0.0, gh, fake, 0, None, None)
    assert st == mxq.MXQ_EUNSUPPORTED and b"GROUP_HEADS" in so.mxq_last_error()
    st = so.attn_mixed_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, None, None, 0,
                           ctypes.byref(ok), 0.0, 3 | mxq.MXQ_GROUP_HEADS, fake, 0, None, None)
    assert st == mxq.MXQ_EINVAL and b"mode" in so.mxq_last_error()
    lp = mxq.LineParams(17, 1, 0)
    st = so.attn_select_lines(fake, fake, ctypes.byref(ok), ctypes.byref(lp), fake, 1 << 20, fake, None, None)
    assert st == mxq.MXQ_EINVAL and b"n_lines" in so.mxq_last_error()
    lp = mxq.LineParams(8, 1, 2)
    st = so.attn_select_lines(fake, fake, ctypes.byref(ok), ctypes.byref(lp), fake, 1 << 20, fake, None, None)
    assert st == mxq.MXQ_EINVAL
    lp = mxq.LineParams(8, 1, 1)
    st = so.attn_select_lines(fake, fake, ctypes.byref(ok), ctypes.byref(lp), fake, 16, fake, None, None)
    assert st == mxq.MXQ_EINVAL and b"workspace" in so.mxq_last_error()
    assert so.attn_select_lines_workspace(ctypes.byref(ok)) == (1 * 2 * 4 * 64 + 1 * 2 * 256) * 4
    kv = mxq.KVCache()
    st = so.attn_quantkv_decode(fake, ctypes.byref(kv), 1, 8, 2, 128, 64, 0.0, 0, fake, 1 << 20, fake, None)
    assert st == mxq.MXQ_EINVAL
    st = so.attn_quantkv_decode(fake, ctypes.byref(kv), 1, 8, 2, 64, 64, 0.0, 0, fake, 1 << 20, fake, None)
    assert st == mxq.MXQ_EUNSUPPORTED
    # cache append: validation before any launch
    st = so.attn_quantkv_append(fake, fake, None, 1, 2, 128, None)
    assert st == mxq.MXQ_EINVAL
    rw = mxq.KVCacheRW(fake, fake, fake, fake, fake, fake, None, None, fake, fake, fake, 64, 4, 8)
    st = so.attn_quantkv_append(fake, fake, ctypes.byref(rw), 1, 2, 128, None)
    assert st == mxq.MXQ_EINVAL and b"sink" in so.mxq_last_error()
    rw = mxq.KVCacheRW(fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, 64, 4, 8)
    st = so.attn_quantkv_append(fake, fake, ctypes.byref(rw), 1, 2, 48, None)
    assert st == mxq.MXQ_EUNSUPPORTED
    rw = mxq.KVCacheRW(fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, None, 64, 4, 8)
    st = so.attn_quantkv_append(fake, fake, ctypes.byref(rw), 1, 2, 128, None)
    assert st == mxq.MXQ_EINVAL and b"seq_len" in so.mxq_last_error()
    # decode with vertical lines: at most 16, arrays required
    kvl = mxq.KVCache(fake, fake, fake, fake, fake, fake, None, None, None, None, fake, 64, 0, 0, fake, fake, fake, 17)
    st = so.attn_quantkv_decode(fake, ctypes.byref(kvl), 1, 8, 2, 128, 64, 0.0, 0, fake, 1 << 20, fake, None)
    assert st == mxq.MXQ_EINVAL and b"n_lines" in so.mxq_last_error()
    kvl = mxq.KVCache(fake, fake, fake, fake, fake, fake, None, None, None, None, fake, 64, 0, 0, fake, None, fake, 4)
    st = so.attn_quantkv_decode(fake, ctypes.byref(kvl), 1, 8, 2, 128, 64, 0.0, 0, fake, 1 << 20, fake, None)
    assert st == mxq.MXQ_EINVAL and b"lines" in so.mxq_last_error()


def test_fused_means_entry_points_validate_before_launch(lib):
    mxq, so = lib
    ok = mxq.AttnShape(1, 2, 2, 256, 256, 64, 64, 64, 0)
    fake = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    st = so.mxq_prefill_operands_means(fake, fake, fake, ctypes.byref(ok), fake, fake, fake, fake, None, None, None,
                                       None, fake, None)
    assert st == mxq.MXQ_EINVAL and b"mean" in so.mxq_last_error()
    bad_bq = mxq.AttnShape(1, 2, 2, 256, 256, 64, 32, 64, 0)
    st = so.mxq_prefill_operands_means(fake, fake, fake, ctypes.byref(bad_bq), fake, fake, fake, fake, None, None,
                                       None, fake, fake, None)
    assert st == mxq.MXQ_EUNSUPPORTED
    sp = mxq.SelectParams(-1, 5, 100, 1, 1)
    st = so.attn_select_blocks_means(fake, None, ctypes.byref(ok), ctypes.byref(sp), fake, None, None, None)
    assert st == mxq.MXQ_EINVAL and b"k_means" in so.mxq_last_error()
    bad = mxq.SelectParams(-1, 5, 0, 1, 1)
    st = so.attn_select_blocks_means(fake, fake, ctypes.byref(ok), ctypes.byref(bad), fake, None, None, None)
    assert st == mxq.MXQ_EINVAL
