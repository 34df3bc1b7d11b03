"""Python binding of libmxq (mixed-precision block-scaled attention on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmxq.so, called through its C ABI (include/mxq.h).  torch provides device
memory and the current HIP stream.  There is no CPU fallback: if the library
is missing or no GPU is present, these functions raise.

Entry points (same names as the C ABI):
  mxq_quantize(x, fmt, axis, n_valid)         -> codes, scales[, zeros]
  attn_select_blocks(q, k, shape, params)     -> mask, n_fp16, scores
  attn_select_lines(q, k, shape, n_lines, ..) -> lines, scores
  attn_mixed_fwd(ops, mask, shape, ...)       -> out, lse
  attn_quantkv_decode(q, cache, ...)          -> out
  attn_quantkv_decode_noalloc(q, cache, ...)  -> out (no workspace: a fixed per-GPU array)
  attn_quantkv_append(cache, k_new, v_new)    -> None (updates the cache in place)
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxq.so")

MXQ_OK, MXQ_EINVAL, MXQ_EUNSUPPORTED, MXQ_EHIP = 0, 1, 2, 3
MXQ_MXFP4_E2M1, MXQ_MXFP8_E4M3, MXQ_INT4_ASYM_G32, MXQ_FP16, MXQ_MXFP4_E2M1_HADAMARD = 1, 2, 3, 4, 5
MXQ_AXIS_D, MXQ_AXIS_N = 0, 1
MXQ_MIXED, MXQ_ALL_LOWBIT, MXQ_ALL_FP16 = 0, 1, 2
MXQ_GROUP_HEADS = 16  # mode flag: one workgroup serves the G query heads of a kv group
MXQ_OUT_F32, MXQ_OUT_BF16 = 0, 1

EXPORTED = [
    "mxq_quantize", "mxq_prefill_operands", "mxq_prefill_operands_means", "attn_select_blocks_workspace",
    "attn_select_blocks", "attn_select_blocks_means", "attn_select_lines_workspace",
    "attn_select_lines", "attn_mixed_fwd",
    "attn_quantkv_decode_workspace", "attn_quantkv_decode", "attn_quantkv_decode_noalloc", "attn_quantkv_append",
    "mxq_kv_lines_from_prefill",
    "mxq_status_string",
    "mxq_last_error", "mxq_version",
]


class MxqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "Hq", "Hkv", "N", "n_valid", "D", "Bq", "Bk", "causal")]


class SelectParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("topk", "ratio_num", "ratio_den", "sink_tiles", "local_tiles",
                                              "group_shared", "heuristic")]


class LineParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_lines", "sink_tokens", "group_shared")]


_KV_FIELDS = [
    ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
    ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
    ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
    ("k_sink", ctypes.c_void_p), ("v_sink", ctypes.c_void_p),
    ("k_recent", ctypes.c_void_p), ("v_recent", ctypes.c_void_p),
    ("seq_len", ctypes.c_void_p),
    ("L_cap", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
]


class KVCache(ctypes.Structure):  # mxq_kv_cache
    _fields_ = _KV_FIELDS + [
        ("lines", ctypes.c_void_p), ("k_lines", ctypes.c_void_p), ("v_lines", ctypes.c_void_p),
        ("n_lines", ctypes.c_int32),
    ]


class KVCacheRW(ctypes.Structure):  # mxq_kv_cache_rw
    _fields_ = _KV_FIELDS


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmxq.so and declare its signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m bit_mixed_precision_mxq_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mxq_quantize.argtypes = [vp, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.mxq_quantize.restype = i32
    lib.mxq_prefill_operands.argtypes = [vp, vp, vp, ctypes.POINTER(AttnShape), i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mxq_prefill_operands.restype = i32
    lib.mxq_prefill_operands_means.argtypes = [vp, vp, vp, ctypes.POINTER(AttnShape), vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp]
    lib.mxq_prefill_operands_means.restype = i32
    lib.attn_select_blocks_means.argtypes = [vp, vp, ctypes.POINTER(AttnShape), ctypes.POINTER(SelectParams), vp, vp,
                                             vp, vp]
    lib.attn_select_blocks_means.restype = i32
    lib.attn_select_blocks_workspace.argtypes = [ctypes.POINTER(AttnShape)]
    lib.attn_select_blocks_workspace.restype = sz
    lib.attn_select_blocks.argtypes = [vp, vp, ctypes.POINTER(AttnShape), ctypes.POINTER(SelectParams),
                                       vp, sz, vp, vp, vp, vp]
    lib.attn_select_blocks.restype = i32
    lib.attn_select_lines_workspace.argtypes = [ctypes.POINTER(AttnShape)]
    lib.attn_select_lines_workspace.restype = sz
    lib.attn_select_lines.argtypes = [vp, vp, ctypes.POINTER(AttnShape), ctypes.POINTER(LineParams),
                                      vp, sz, vp, vp, vp]
    lib.attn_select_lines.restype = i32
    lib.attn_mixed_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, ctypes.POINTER(AttnShape),
                                   ctypes.c_float, i32, vp, i32, vp, vp]
    lib.attn_mixed_fwd.restype = i32
    lib.attn_quantkv_decode_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_quantkv_decode_workspace.restype = sz
    lib.attn_quantkv_decode.argtypes = [vp, ctypes.POINTER(KVCache), i32, i32, i32, i32, i32,
                                        ctypes.c_float, i32, vp, sz, vp, vp]
    lib.attn_quantkv_decode.restype = i32
    lib.attn_quantkv_decode_noalloc.argtypes = [vp, ctypes.POINTER(KVCache), i32, i32, i32, i32, i32,
                                                ctypes.c_float, i32, vp, vp]
    lib.attn_quantkv_decode_noalloc.restype = i32
    lib.mxq_kv_lines_from_prefill.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.mxq_kv_lines_from_prefill.restype = i32
    lib.attn_quantkv_append.argtypes = [vp, vp, ctypes.POINTER(KVCacheRW), i32, i32, i32, vp]
    lib.attn_quantkv_append.restype = i32
    lib.mxq_status_string.argtypes = [i32]
    lib.mxq_status_string.restype = ctypes.c_char_p
    lib.mxq_last_error.argtypes = []
    lib.mxq_last_error.restype = ctypes.c_char_p
    lib.mxq_version.argtypes = []
    lib.mxq_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != MXQ_OK:
        lib = load_library()
        raise MxqError(status, lib.mxq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


# ------------------------------------------------------------------ quantize
def mxq_quantize(x: torch.Tensor, fmt: int, axis: int, n_valid: int | None = None):
    """x: bf16 [B,H,N,D] on the GPU.  Returns (codes, scales, zeros) with the
    layouts of include/mxq.h (scales/zeros None where the format has none)."""
    _need_gpu(x)
    assert x.dtype == torch.bfloat16 and x.dim() == 4
    B, H, N, D = x.shape
    nv = N if n_valid is None else int(n_valid)
    dev = x.device
    zeros = None
    if fmt in (MXQ_MXFP4_E2M1, MXQ_MXFP4_E2M1_HADAMARD):
        codes = torch.empty((B, H, N, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, N, D // 32), dtype=torch.uint8, device=dev)
    elif fmt == MXQ_MXFP8_E4M3:
        codes = torch.empty((B, H, D, N), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, D, N // 32), dtype=torch.uint8, device=dev)
    elif fmt == MXQ_FP16:
        shape = (B, H, N, D) if axis == MXQ_AXIS_D else (B, H, D, N)
        codes = torch.empty(shape, dtype=torch.float16, device=dev)
        scales = None
    elif fmt == MXQ_INT4_ASYM_G32:
        codes = torch.empty((B, H, N, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, N, D // 32), dtype=torch.float16, device=dev)
        zeros = torch.empty((B, H, N, D // 32), dtype=torch.float16, device=dev)
    else:
        raise ValueError("unknown format")
    lib = load_library()
    _check(lib.mxq_quantize(_ptr(x), B, H, N, D, nv, fmt, axis, _ptr(codes), _ptr(scales), _ptr(zeros), _stream()))
    return codes, scales, zeros


# ------------------------------------------------------------------ select
@dataclass
class Shape:
    B: int
    Hq: int
    Hkv: int
    N: int
    n_valid: int
    D: int
    Bq: int
    Bk: int
    causal: bool

    def c(self) -> AttnShape:
        return AttnShape(self.B, self.Hq, self.Hkv, self.N, self.n_valid, self.D, self.Bq, self.Bk, int(self.causal))


def select_workspace(shape: Shape, device) -> torch.Tensor:
    n = load_library().attn_select_blocks_workspace(ctypes.byref(shape.c()))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attn_select_blocks(q, k, shape: Shape, topk=-1, ratio=(5, 100), sink_tiles=0, local_tiles=0,
                       want_scores=False, workspace=None, mask=None, n_fp16=None, group_shared=False,
                       heuristic=0):
    """Returns (mask u32-as-int32 [B,Hq,n_qt,words], n_fp16 [B,Hq,n_qt], scores or None);
    mask and n_fp16 may be passed in to be reused."""
    _need_gpu(q, k)
    n_qt, n_kt = shape.N // shape.Bq, shape.N // shape.Bk
    words = (n_kt + 31) // 32
    dev = q.device
    if mask is None:
        mask = torch.empty((shape.B, shape.Hq, n_qt, words), dtype=torch.int32, device=dev)
    nfp = n_fp16 if n_fp16 is not None else torch.empty((shape.B, shape.Hq, n_qt), dtype=torch.int32, device=dev)
    _need_gpu(mask, nfp)
    assert mask.numel() == shape.B * shape.Hq * n_qt * words and nfp.numel() == shape.B * shape.Hq * n_qt
    scores = torch.empty((shape.B, shape.Hq, n_qt, n_kt), dtype=torch.float32, device=dev) if want_scores else None
    ws = workspace if workspace is not None else select_workspace(shape, dev)
    sp = SelectParams(int(topk), int(ratio[0]), int(ratio[1]), int(sink_tiles), int(local_tiles),
                      int(bool(group_shared)), int(heuristic))
    cs = shape.c()
    _check(load_library().attn_select_blocks(_ptr(q), _ptr(k), ctypes.byref(cs), ctypes.byref(sp), _ptr(ws),
                                             ws.numel(), _ptr(mask), _ptr(nfp), _ptr(scores), _stream()))
    return mask, nfp, scores


def attn_select_blocks_means(q_means, k_means, shape: Shape, topk=-1, ratio=(5, 100), sink_tiles=0, local_tiles=0,
                             want_scores=False, mask=None, n_fp16=None, group_shared=False):
    """attn_select_blocks on tile means from prepare_prefill_means (same result)."""
    _need_gpu(q_means, k_means)
    n_qt, n_kt = shape.N // shape.Bq, shape.N // shape.Bk
    words = (n_kt + 31) // 32
    dev = q_means.device
    assert q_means.dtype == k_means.dtype == torch.float32
    assert q_means.numel() == shape.B * shape.Hq * n_qt * shape.D and k_means.numel() == shape.B * shape.Hkv * n_kt * shape.D
    if mask is None:
        mask = torch.empty((shape.B, shape.Hq, n_qt, words), dtype=torch.int32, device=dev)
    nfp = n_fp16 if n_fp16 is not None else torch.empty((shape.B, shape.Hq, n_qt), dtype=torch.int32, device=dev)
    scores = torch.empty((shape.B, shape.Hq, n_qt, n_kt), dtype=torch.float32, device=dev) if want_scores else None
    sp = SelectParams(int(topk), int(ratio[0]), int(ratio[1]), int(sink_tiles), int(local_tiles),
                      int(bool(group_shared)))
    cs = shape.c()
    _check(load_library().attn_select_blocks_means(_ptr(q_means), _ptr(k_means), ctypes.byref(cs), ctypes.byref(sp),
                                                   _ptr(mask), _ptr(nfp), _ptr(scores), _stream()))
    return mask, nfp, scores


def lines_workspace(shape: Shape, device) -> torch.Tensor:
    n = load_library().attn_select_lines_workspace(ctypes.byref(shape.c()))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attn_select_lines(q, k, shape: Shape, n_lines, sink_tokens=1, group_shared=False, want_scores=False,
                      workspace=None, lines=None):
    """Vertical-line keys per query head.  Returns (lines int32 [B,Hq,n_lines]
    ascending and -1 padded, scores f32 [B,Hq,N] or None); lines may be passed
    in to be reused."""
    _need_gpu(q, k)
    dev = q.device
    if lines is None:
        lines = torch.empty((shape.B, shape.Hq, n_lines), dtype=torch.int32, device=dev)
    _need_gpu(lines)
    assert lines.dtype == torch.int32 and lines.numel() == shape.B * shape.Hq * n_lines
    scores = torch.empty((shape.B, shape.Hq, shape.N), dtype=torch.float32, device=dev) if want_scores else None
    ws = workspace if workspace is not None else lines_workspace(shape, dev)
    lp = LineParams(int(n_lines), int(sink_tokens), int(bool(group_shared)))
    cs = shape.c()
    _check(load_library().attn_select_lines(_ptr(q), _ptr(k), ctypes.byref(cs), ctypes.byref(lp), _ptr(ws),
                                            ws.numel(), _ptr(lines), _ptr(scores), _stream()))
    return lines, scores


# ------------------------------------------------------------------ attention
@dataclass
class PrefillOperands:
    q_codes: torch.Tensor | None = None
    q_scales: torch.Tensor | None = None
    k_codes: torch.Tensor | None = None
    k_scales: torch.Tensor | None = None
    v_codes: torch.Tensor | None = None
    v_scales: torch.Tensor | None = None
    q_bf16: torch.Tensor | None = None
    k_bf16: torch.Tensor | None = None
    v_f16t: torch.Tensor | None = None
    v_bf16: torch.Tensor | None = None   # read for line keys only when v_f16t is None


def prepare_prefill(q, k, v, n_valid, mode=MXQ_MIXED, lines=False, rotate=False, promoted=True) -> PrefillOperands:
    """Quantise Q/K (MXFP4, optionally of the Walsh-Hadamard-rotated rows),
    V (MXFP8 along keys) and make the fp16 V^T copy (needed by FP16 tiles and
    by vertical lines), all on the GPU in two launches (mxq_prefill_operands).
    promoted=False (MIXED mode whose mask promotes no tile) skips the fp16
    copy: the attention then takes the line keys' V from bf16 V."""
    _need_gpu(q, k, v)
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16 and q.dim() == k.dim() == v.dim() == 4
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == v.shape == (B, Hkv, N, D)
    dev = q.device
    ops = PrefillOperands(q_bf16=q, k_bf16=k, v_bf16=v)
    if mode != MXQ_ALL_FP16:
        ops.q_codes = torch.empty((B, Hq, N, D // 2), dtype=torch.uint8, device=dev)
        ops.q_scales = torch.empty((B, Hq, N, D // 32), dtype=torch.uint8, device=dev)
        ops.k_codes = torch.empty((B, Hkv, N, D // 2), dtype=torch.uint8, device=dev)
        ops.k_scales = torch.empty((B, Hkv, N, D // 32), dtype=torch.uint8, device=dev)
        ops.v_codes = torch.empty((B, Hkv, D, N), dtype=torch.uint8, device=dev)
        ops.v_scales = torch.empty((B, Hkv, D, N // 32), dtype=torch.uint8, device=dev)
    if mode == MXQ_ALL_FP16 or (mode == MXQ_MIXED and promoted) or (lines and mode != MXQ_MIXED):
        ops.v_f16t = torch.empty((B, Hkv, D, N), dtype=torch.float16, device=dev)
    cs = Shape(B, Hq, Hkv, N, int(n_valid), D, 64, 64, False).c()
    _check(load_library().mxq_prefill_operands(
        _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs), int(bool(rotate)), _ptr(ops.q_codes), _ptr(ops.q_scales),
        _ptr(ops.k_codes), _ptr(ops.k_scales), _ptr(ops.v_codes), _ptr(ops.v_scales), _ptr(ops.v_f16t), _stream()))
    return ops


def prepare_prefill_means(q, k, v, shape: Shape, out=None, means=None):
    """prepare_prefill (no rotation) plus the tile means attn_select_blocks
    scores with, from one read of Q and K (mxq_prefill_operands_means).
    Returns (ops, q_means f32 [B,Hq,N/Bq,D], k_means f32 [B,Hkv,D,N/Bk]);
    out (PrefillOperands) and means (a pair) may be passed in to be reused."""
    _need_gpu(q, k, v)
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16 and q.dim() == k.dim() == v.dim() == 4
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    ops = out if out is not None else PrefillOperands(q_bf16=q, k_bf16=k, v_bf16=v)
    ops.q_bf16, ops.k_bf16, ops.v_bf16 = q, k, v
    if ops.q_codes is None:
        ops.q_codes = torch.empty((B, Hq, N, D // 2), dtype=torch.uint8, device=dev)
        ops.q_scales = torch.empty((B, Hq, N, D // 32), dtype=torch.uint8, device=dev)
        ops.k_codes = torch.empty((B, Hkv, N, D // 2), dtype=torch.uint8, device=dev)
        ops.k_scales = torch.empty((B, Hkv, N, D // 32), dtype=torch.uint8, device=dev)
        ops.v_codes = torch.empty((B, Hkv, D, N), dtype=torch.uint8, device=dev)
        ops.v_scales = torch.empty((B, Hkv, D, N // 32), dtype=torch.uint8, device=dev)
        ops.v_f16t = torch.empty((B, Hkv, D, N), dtype=torch.float16, device=dev)
    if means is None:
        means = (torch.empty((B, Hq, N // shape.Bq, D), dtype=torch.float32, device=dev),
                 torch.empty((B, Hkv, D, N // shape.Bk), dtype=torch.float32, device=dev))
    cs = shape.c()
    _check(load_library().mxq_prefill_operands_means(
        _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs), _ptr(ops.q_codes), _ptr(ops.q_scales), _ptr(ops.k_codes),
        _ptr(ops.k_scales), _ptr(ops.v_codes), _ptr(ops.v_scales), _ptr(ops.v_f16t), _ptr(means[0]), _ptr(means[1]),
        _stream()))
    return ops, means[0], means[1]


def attn_mixed_fwd(ops: PrefillOperands, mask, shape: Shape, softmax_scale=0.0, mode=MXQ_MIXED,
                   out_dtype=MXQ_OUT_F32, want_lse=True, out=None, lse=None, lines=None, group_heads=False):
    """lines: int32 [B,Hq,n_lines] vertical-line keys (attn_select_lines) or None.
    group_heads: one workgroup serves the G query heads of each kv group, and
    the mask row and line list of the group's first head apply to all G (as
    written by selection with group_shared)."""
    if lines is not None:
        _need_gpu(lines)
        assert lines.dtype == torch.int32 and lines.dim() == 3
    dev = (ops.q_bf16 if ops.q_bf16 is not None else ops.q_codes).device
    if out is None:
        out = torch.empty((shape.B, shape.Hq, shape.N, shape.D),
                          dtype=torch.float32 if out_dtype == MXQ_OUT_F32 else torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((shape.B, shape.Hq, shape.N), dtype=torch.float32, device=dev)
    cs = shape.c()
    _check(load_library().attn_mixed_fwd(
        _ptr(ops.q_codes), _ptr(ops.q_scales), _ptr(ops.k_codes), _ptr(ops.k_scales), _ptr(ops.v_codes),
        _ptr(ops.v_scales), _ptr(ops.q_bf16), _ptr(ops.k_bf16), _ptr(ops.v_f16t), _ptr(ops.v_bf16), _ptr(mask),
        _ptr(lines), 0 if lines is None else int(lines.shape[-1]), ctypes.byref(cs), float(softmax_scale),
        int(mode) | (MXQ_GROUP_HEADS if group_heads else 0), _ptr(out), int(out_dtype), _ptr(lse), _stream()))
    return out, lse


class PrefillPipeline:
    """One prefill step.  When tiles are chosen by score (and Q/K are not
    rotated), one chain on the caller's stream: the quantiser also writes the
    tile means, selection scores them, then attention.  Otherwise a small DAG
    on two HIP streams (default priority): selection (and line selection) reads
    only bf16 Q and K and runs on a second stream while Q, K and V are
    quantised on the caller's stream, and the attention waits for both.
    Workspaces and outputs are allocated once."""

    def __init__(self, shape: Shape, topk=-1, ratio=(5, 100), sink_tiles=0, local_tiles=0, n_lines=0,
                 sink_tokens=0, rotate=False, out_dtype=MXQ_OUT_BF16, device="cuda:0", fused_means=True,
                 group_shared=False, group_heads=False, v_beside=True):
        self.shape, self.topk, self.ratio = shape, topk, ratio
        self.group_shared = bool(group_shared)
        # one workgroup per kv group in the attention (needs the shared masks)
        self.group_heads = bool(group_heads)
        assert not self.group_heads or self.group_shared, "group_heads needs group_shared selection"
        self.sink_tiles, self.local_tiles = sink_tiles, local_tiles
        self.n_lines, self.sink_tokens, self.rotate, self.out_dtype = n_lines, sink_tokens, rotate, out_dtype
        dev = torch.device(device)
        n_qt, n_kt = shape.N // shape.Bq, shape.N // shape.Bk
        self.ws = select_workspace(shape, dev)
        self.mask = torch.empty((shape.B, shape.Hq, n_qt, (n_kt + 31) // 32), dtype=torch.int32, device=dev)
        self.nfp = torch.empty((shape.B, shape.Hq, n_qt), dtype=torch.int32, device=dev)
        self.lws = lines_workspace(shape, dev) if n_lines else None
        self.lines = torch.empty((shape.B, shape.Hq, n_lines), dtype=torch.int32, device=dev) if n_lines else None
        odt = torch.float32 if out_dtype == MXQ_OUT_F32 else torch.bfloat16
        self.out = torch.empty((shape.B, shape.Hq, shape.N, shape.D), dtype=odt, device=dev)
        self.lse = torch.empty((shape.B, shape.Hq, shape.N), dtype=torch.float32, device=dev)
        self.aux = torch.cuda.Stream(device=dev)
        self.ev_in, self.ev_sel = torch.cuda.Event(), torch.cuda.Event()
        # when tiles are chosen by score and Q/K are not rotated, the quantiser
        # also writes the tile means and the step runs as one chain on the
        # caller's stream (no cross-stream waits); a zero budget needs no
        # scores, and its selection runs beside the quantisers instead
        scored = topk > 0 or (topk < 0 and ratio[0] > 0)
        self.fused = bool(fused_means) and not rotate and scored
        self.ops = PrefillOperands() if self.fused else None
        self.means = ((torch.empty((shape.B, shape.Hq, n_qt, shape.D), dtype=torch.float32, device=dev),
                       torch.empty((shape.B, shape.Hkv, shape.D, n_kt), dtype=torch.float32, device=dev))
                      if self.fused else None)
        # a zero budget with no forced tile promotes nothing: no fp16 copy of
        # V, and (v_beside) V's MXFP8 quantiser runs on the second stream
        # after selection while Q and K are quantised on the caller's stream
        self.promoted = sink_tiles > 0 or local_tiles > 0 or scored
        self.v_beside = bool(v_beside) and not self.fused and not self.promoted
        if self.v_beside:
            B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
            u8 = dict(dtype=torch.uint8, device=dev)
            self.ops = PrefillOperands(
                q_codes=torch.empty((B, Hq, N, D // 2), **u8), q_scales=torch.empty((B, Hq, N, D // 32), **u8),
                k_codes=torch.empty((B, Hkv, N, D // 2), **u8), k_scales=torch.empty((B, Hkv, N, D // 32), **u8),
                v_codes=torch.empty((B, Hkv, D, N), **u8), v_scales=torch.empty((B, Hkv, D, N // 32), **u8))

    def __call__(self, q, k, v, events=None):
        """Returns (out, lse).  events=(e0, e1) are recorded around the
        attention kernel on the caller's stream."""
        main = torch.cuda.current_stream()
        if self.fused:
            ops, qm, km = prepare_prefill_means(q, k, v, self.shape, out=self.ops, means=self.means)
            attn_select_blocks_means(qm, km, self.shape, topk=self.topk, ratio=self.ratio, sink_tiles=self.sink_tiles,
                                     local_tiles=self.local_tiles, mask=self.mask, n_fp16=self.nfp,
                                     group_shared=self.group_shared)
            if self.n_lines:
                attn_select_lines(q, k, self.shape, self.n_lines, self.sink_tokens, workspace=self.lws,
                                  lines=self.lines, group_shared=self.group_heads)
            if events is not None:
                events[0].record(main)
            attn_mixed_fwd(ops, self.mask, self.shape, out_dtype=self.out_dtype, out=self.out, lse=self.lse,
                           lines=self.lines, group_heads=self.group_heads)
            if events is not None:
                events[1].record(main)
            return self.out, self.lse
        self.ev_in.record(main)
        with torch.cuda.stream(self.aux):
            self.aux.wait_event(self.ev_in)
            attn_select_blocks(q, k, self.shape, topk=self.topk, ratio=self.ratio, sink_tiles=self.sink_tiles,
                               local_tiles=self.local_tiles, workspace=self.ws, mask=self.mask, n_fp16=self.nfp,
                               group_shared=self.group_shared)
            if self.n_lines:
                attn_select_lines(q, k, self.shape, self.n_lines, self.sink_tokens, workspace=self.lws,
                                  lines=self.lines, group_shared=self.group_heads)
            self.ev_sel.record(self.aux)
        if self.v_beside:
            lib, sh, ops = load_library(), self.shape, self.ops
            ops.q_bf16, ops.k_bf16, ops.v_bf16 = q, k, v
            fmt = MXQ_MXFP4_E2M1_HADAMARD if self.rotate else MXQ_MXFP4_E2M1
            with torch.cuda.stream(self.aux):
                _check(lib.mxq_quantize(_ptr(v), sh.B, sh.Hkv, sh.N, sh.D, sh.n_valid, MXQ_MXFP8_E4M3, MXQ_AXIS_N,
                                        _ptr(ops.v_codes), _ptr(ops.v_scales), None, _stream()))
                self.ev_sel.record(self.aux)
            for x, H, codes, scales in ((q, sh.Hq, ops.q_codes, ops.q_scales), (k, sh.Hkv, ops.k_codes, ops.k_scales)):
                _check(lib.mxq_quantize(_ptr(x), sh.B, H, sh.N, sh.D, sh.n_valid, fmt, MXQ_AXIS_D, _ptr(codes),
                                        _ptr(scales), None, _stream()))
        else:
            ops = prepare_prefill(q, k, v, self.shape.n_valid, lines=bool(self.n_lines), rotate=self.rotate,
                                  promoted=self.promoted)
        main.wait_event(self.ev_sel)
        if events is not None:
            events[0].record(main)
        attn_mixed_fwd(ops, self.mask, self.shape, out_dtype=self.out_dtype, out=self.out, lse=self.lse,
                       lines=self.lines, group_heads=self.group_heads)
        if events is not None:
            events[1].record(main)
        return self.out, self.lse


# ------------------------------------------------------------------ decode
@dataclass
class QuantKVCache:
    k_codes: torch.Tensor
    v_codes: torch.Tensor
    k_scale: torch.Tensor
    k_zero: torch.Tensor
    v_scale: torch.Tensor
    v_zero: torch.Tensor
    k_sink: torch.Tensor | None
    v_sink: torch.Tensor | None
    k_recent: torch.Tensor | None
    v_recent: torch.Tensor | None
    seq_len: torch.Tensor
    n_sink: int
    n_recent: int
    lines: torch.Tensor | None = None     # int32 [B,Hkv,n_lines] vertical-line tokens
    k_lines: torch.Tensor | None = None   # fp16 [B,Hkv,n_lines,D]
    v_lines: torch.Tensor | None = None

    def _common(self):
        return (_ptr(self.k_codes), _ptr(self.v_codes), _ptr(self.k_scale), _ptr(self.k_zero),
                _ptr(self.v_scale), _ptr(self.v_zero), _ptr(self.k_sink), _ptr(self.v_sink),
                _ptr(self.k_recent), _ptr(self.v_recent), _ptr(self.seq_len),
                int(self.k_codes.shape[2]), int(self.n_sink), int(self.n_recent))

    def c(self) -> KVCache:
        n_lines = 0 if self.lines is None else int(self.lines.shape[-1])
        return KVCache(*self._common(), _ptr(self.lines), _ptr(self.k_lines), _ptr(self.v_lines), n_lines)

    def rw(self) -> KVCacheRW:
        return KVCacheRW(*self._common())


def build_quant_kv_cache(k, v, seq_len, n_sink, n_recent, k_recent=None, v_recent=None, lines=None,
                         k_line_rows=None, v_line_rows=None) -> QuantKVCache:
    """k, v: bf16 [B,Hkv,L,D] on the GPU; seq_len int32 [B] on the GPU.  The
    INT4 arrays cover all L positions; the sink copy is tokens 0..n_sink-1 and
    the recent copy (bf16 [B,Hkv,n_recent,D], given by the caller, who knows
    each sequence's last tokens) is converted to fp16.  Optional vertical-line
    tokens: lines int32 [B,Hkv,n] on the GPU and their bf16 rows
    [B,Hkv,n,D] (gathered by the caller), kept in fp16."""
    kc, ks, kz = mxq_quantize(k, MXQ_INT4_ASYM_G32, MXQ_AXIS_D)
    vc, vs, vz = mxq_quantize(v, MXQ_INT4_ASYM_G32, MXQ_AXIS_D)
    k_sink = v_sink = k_rec = v_rec = None
    if n_sink > 0:
        k_sink, _, _ = mxq_quantize(k[:, :, :n_sink].contiguous(), MXQ_FP16, MXQ_AXIS_D)
        v_sink, _, _ = mxq_quantize(v[:, :, :n_sink].contiguous(), MXQ_FP16, MXQ_AXIS_D)
    if n_recent > 0:
        k_rec, _, _ = mxq_quantize(k_recent.contiguous(), MXQ_FP16, MXQ_AXIS_D)
        v_rec, _, _ = mxq_quantize(v_recent.contiguous(), MXQ_FP16, MXQ_AXIS_D)
    k_ln = v_ln = None
    if lines is not None:
        _need_gpu(lines)
        k_ln, _, _ = mxq_quantize(k_line_rows.contiguous(), MXQ_FP16, MXQ_AXIS_D)
        v_ln, _, _ = mxq_quantize(v_line_rows.contiguous(), MXQ_FP16, MXQ_AXIS_D)
    return QuantKVCache(kc, vc, ks, kz, vs, vz, k_sink, v_sink, k_rec, v_rec, seq_len, n_sink, n_recent,
                        lines, k_ln, v_ln)


def kv_lines_from_prefill(lines_hq, k, v):
    """Decode line tokens from the prefill's group-shared vertical lines:
    lines_hq int32 [B,Hq,n] (attn_select_lines with group_shared=True), k, v
    the prompt's bf16 [B,Hkv,L,D].  Returns (lines int32 [B,Hkv,n], k_lines,
    v_lines fp16 [B,Hkv,n,D]) for QuantKVCache."""
    _need_gpu(lines_hq, k, v)
    B, Hq, n = lines_hq.shape
    _, Hkv, L, D = k.shape
    dev = k.device
    lines = torch.empty((B, Hkv, n), dtype=torch.int32, device=dev)
    kl = torch.empty((B, Hkv, n, D), dtype=torch.float16, device=dev)
    vl = torch.empty_like(kl)
    _check(load_library().mxq_kv_lines_from_prefill(_ptr(lines_hq), Hq, _ptr(k), _ptr(v), B, Hkv, L, D, n,
                                                    _ptr(lines), _ptr(kl), _ptr(vl), _stream()))
    return lines, kl, vl


def decode_workspace(B, Hq, D, num_splits, max_seq_len, device) -> torch.Tensor:
    n = load_library().attn_quantkv_decode_workspace(B, Hq, D, num_splits, max_seq_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attn_quantkv_decode(q, cache: QuantKVCache, Hkv, max_seq_len, softmax_scale=0.0, num_splits=0,
                        workspace=None, out=None):
    """q: bf16 [B,Hq,D] on the GPU.  Returns out f32 [B,Hq,D]."""
    _need_gpu(q)
    B, Hq, D = q.shape
    ws = workspace if workspace is not None else decode_workspace(B, Hq, D, num_splits, max_seq_len, q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    kv = cache.c()
    _check(load_library().attn_quantkv_decode(_ptr(q), ctypes.byref(kv), B, Hq, Hkv, D, int(max_seq_len),
                                              float(softmax_scale), int(num_splits), _ptr(ws), ws.numel(),
                                              _ptr(out), _stream()))
    return out


DECODE_SCRATCH_BYTES = 16 << 20  # MXQ_DECODE_SCRATCH_BYTES


def attn_quantkv_decode_noalloc(q, cache: QuantKVCache, Hkv, max_seq_len, softmax_scale=0.0, num_splits=0, out=None):
    """attn_quantkv_decode with the split partials in the library's fixed
    per-GPU array: no workspace, nothing allocated by the library (out must be
    passed in for a call that allocates nothing at all).  Calls that overlap on
    one GPU race on that array."""
    _need_gpu(q)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    kv = cache.c()
    _check(load_library().attn_quantkv_decode_noalloc(_ptr(q), ctypes.byref(kv), B, Hq, Hkv, D, int(max_seq_len),
                                                      float(softmax_scale), int(num_splits), _ptr(out), _stream()))
    return out


def attn_quantkv_append(cache: QuantKVCache, k_new, v_new):
    """Append one token per sequence (k_new, v_new: bf16 [B,Hkv,D] on the GPU):
    it enters the fp16 recent window, the token leaving the window is quantised
    to INT4, and seq_len grows by one -- all on the GPU, in place."""
    _need_gpu(k_new, v_new)
    assert k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16 and k_new.shape == v_new.shape
    B, Hkv, D = k_new.shape
    kv = cache.rw()
    _check(load_library().attn_quantkv_append(_ptr(k_new), _ptr(v_new), ctypes.byref(kv), B, Hkv, D, _stream()))
