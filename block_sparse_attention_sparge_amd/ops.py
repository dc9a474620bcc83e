"""Thin ctypes binding of libsparge.so (the C ABI in include/sparge.h).

Each function here only marshals torch tensors into the C ABI: it checks
devices, dtypes and layouts, allocates the outputs with torch (PyTorch is the
device-memory and stream provider), passes raw pointers, element strides and
the current HIP stream, and raises SpargeError on a non-zero status.  All
arithmetic runs in the library's HIP kernels; if the library cannot be loaded
every entry point raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparge.so")

SPARGE_OK, SPARGE_ERR_INVALID, SPARGE_ERR_UNSUPPORTED, SPARGE_ERR_HIP = 0, 1, 2, 3
SPARGE_F16, SPARGE_BF16, SPARGE_F32 = 0, 1, 2
SPARGE_FLAG_SMOOTH_K, SPARGE_FLAG_CAUSAL, SPARGE_FLAG_ATTN_SINK, SPARGE_FLAG_QUANT_FP8 = 1, 2, 4, 8
ABI_VERSION = 7
NOALLOC_SCRATCH_BYTES = 32 << 20
MAX_HEADS = 128
MAX_KBLOCKS = 1024

EXPORTED_SYMBOLS = (
    "sparge_abi_version", "sparge_last_error", "sparge_build_block_map",
    "sparge_build_block_map_workspace", "sparse_fmha_fwd", "sparse_fmha_fwd_qk_int8", "attn_combine",
    "sparge_validate_lut", "sparge_build_block_map_noalloc", "sparse_fmha_fwd_qk_fp8",
)


class SpargeError(RuntimeError):
    """A non-zero status from the library (status code in .status)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"sparge status {status}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()

_i = ctypes.c_int
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_f = ctypes.c_float
_u = ctypes.c_uint
_sz = ctypes.c_size_t
_I64x3 = ctypes.c_int64 * 3


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsparge.so once and declare its signatures; raises if missing."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise SpargeError(SPARGE_ERR_HIP, f"{p} not found: build it with "
                              "`python -m block_sparse_attention_sparge_amd.build`")
        lib = ctypes.CDLL(p)
        lib.sparge_abi_version.restype = _i
        lib.sparge_abi_version.argtypes = []
        if lib.sparge_abi_version() != ABI_VERSION:
            raise SpargeError(SPARGE_ERR_HIP, f"{p} has ABI version {lib.sparge_abi_version()}, this "
                              f"binding needs {ABI_VERSION}: rebuild it")
        lib.sparge_last_error.restype = ctypes.c_char_p
        lib.sparge_last_error.argtypes = []
        lib.sparge_build_block_map_workspace.restype = _sz
        lib.sparge_build_block_map_workspace.argtypes = [_i] * 7
        lib.sparge_build_block_map.restype = _i
        lib.sparge_build_block_map.argtypes = [
            _p, _p, _i, _i, _i, _i, _i, _i, _i, _I64x3, _I64x3, _i, _i,
            _p, _p, _p, _f, _u, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
        lib.sparge_build_block_map_noalloc.restype = _i
        lib.sparge_build_block_map_noalloc.argtypes = [
            _p, _p, _i, _i, _i, _i, _i, _i, _i, _I64x3, _I64x3, _i, _i,
            _p, _p, _p, _f, _u, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]
        lib.sparse_fmha_fwd.restype = _i
        lib.sparse_fmha_fwd.argtypes = [
            _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
            _I64x3, _I64x3, _I64x3, _I64x3, _i, _i, _p, _p, _i, _i, _f, _u, _f, _i, _i64, _p]
        lib.sparse_fmha_fwd_qk_int8.restype = _i
        lib.sparse_fmha_fwd_qk_int8.argtypes = [
            _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
            _I64x3, _I64x3, _I64x3, _I64x3, _p, _p, _i, _i, _f, _u, _i, _i64, _p]
        lib.sparse_fmha_fwd_qk_fp8.restype = _i
        lib.sparse_fmha_fwd_qk_fp8.argtypes = lib.sparse_fmha_fwd_qk_int8.argtypes
        lib.attn_combine.restype = _i
        lib.attn_combine.argtypes = [_p, _i, _p, _i, _i, _i, _i, _i, _i64, _p, _i, _p, _p]
        lib.sparge_validate_lut.restype = _i
        lib.sparge_validate_lut.argtypes = [_p, _p, _i64, _i, _i, _p, _p]
        if path is None:
            _lib = lib
        return lib


def _check(status: int):
    if status != SPARGE_OK:
        msg = load_library().sparge_last_error().decode(errors="replace")
        raise SpargeError(status, msg)


def _dt(t: torch.dtype) -> int:
    if t == torch.float16:
        return SPARGE_F16
    if t == torch.bfloat16:
        return SPARGE_BF16
    if t == torch.float32:
        return SPARGE_F32
    raise SpargeError(SPARGE_ERR_UNSUPPORTED, f"dtype {t} not supported")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(x: torch.Tensor):
    if x.dim() != 4:
        raise SpargeError(SPARGE_ERR_INVALID, f"expected a [b, h, s, d] tensor, got {tuple(x.shape)}")
    if x.stride(3) != 1:
        raise SpargeError(SPARGE_ERR_INVALID, "the last dimension must be contiguous")
    return _I64x3(x.stride(0), x.stride(1), x.stride(2))


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise SpargeError(SPARGE_ERR_INVALID, "tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise SpargeError(SPARGE_ERR_INVALID, "tensors are on different devices")
    return dev


def _f32_array(vals: Optional[Sequence[float]], n: int, name: str):
    if vals is None:
        return None
    if isinstance(vals, (int, float)):
        vals = [float(vals)] * n
    vals = list(vals)
    if len(vals) != n:
        raise SpargeError(SPARGE_ERR_INVALID, f"{name} needs {n} entries, got {len(vals)}")
    return (ctypes.c_float * n)(*vals)


def _flags(smooth_k: bool = False, causal: bool = False, attention_sink: bool = False,
           quant_fp8: bool = False) -> int:
    return ((SPARGE_FLAG_SMOOTH_K if smooth_k else 0) | (SPARGE_FLAG_CAUSAL if causal else 0) |
            (SPARGE_FLAG_ATTN_SINK if attention_sink else 0) | (SPARGE_FLAG_QUANT_FP8 if quant_fp8 else 0))


def _check_lut_rows(lut, count, b, nq):
    """A block LUT holds one row per (b, LUT head, Q-tile); the kernels read
    nq of them per head, so a shorter LUT is refused here."""
    if lut.dim() != 4 or lut.shape[0] != b or lut.shape[2] != nq:
        raise SpargeError(SPARGE_ERR_INVALID, f"lut must be [b={b}, heads, nq={nq}, L] (got {tuple(lut.shape)})")
    if count is not None and tuple(count.shape) != tuple(lut.shape[:3]):
        raise SpargeError(SPARGE_ERR_INVALID, f"count must be {tuple(lut.shape[:3])} (got {tuple(count.shape)})")


def _check_attn_shapes(q, k, v, o, lse, num_splits):
    """q [b, h_q, s_q, d]; k, v [b, h_kv, s_k, d]; o [(S,) b, h_q, s_q, d] and lse
    [(S,) b, h_q, s_q] contiguous fp32, the split axis S present when num_splits
    > 1.  The C ABI takes a single b, s_k and d for all of them, so any other
    shape would send the kernels past the end of a buffer."""
    b, h_q, s_q, d = q.shape
    if k.dim() != 4 or v.dim() != 4:
        raise SpargeError(SPARGE_ERR_INVALID, "k and v must be [b, h_kv, s_k, d]")
    if k.shape[0] != b or k.shape[3] != d:
        raise SpargeError(SPARGE_ERR_INVALID, f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in b or d")
    if tuple(v.shape) != tuple(k.shape):
        raise SpargeError(SPARGE_ERR_INVALID, f"v {tuple(v.shape)} must have the shape of k {tuple(k.shape)}")
    lead = () if num_splits == 1 else (int(num_splits),)
    if o is not None and tuple(o.shape) != lead + (b, h_q, s_q, d):
        raise SpargeError(SPARGE_ERR_INVALID, f"o must be {lead + (b, h_q, s_q, d)} (got {tuple(o.shape)})")
    if lse is not None:
        if tuple(lse.shape) != lead + (b, h_q, s_q):
            raise SpargeError(SPARGE_ERR_INVALID, f"lse must be {lead + (b, h_q, s_q)} (got {tuple(lse.shape)})")
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise SpargeError(SPARGE_ERR_INVALID, "lse must be contiguous float32")


def block_map_workspace_bytes(b: int, h: int, s_q: int, s_k: int, d: int, blk_q: int = 64,
                              blk_k: int = 64) -> int:
    return int(load_library().sparge_build_block_map_workspace(b, h, s_q, s_k, d, blk_q, blk_k))


def build_block_map(q: torch.Tensor, k: torch.Tensor, topk, simthreshd1, cdfthreshd=None,
                    softmax_scale: float = 0.0, blk_q: int = 64, blk_k: int = 64,
                    return_debug: bool = False, workspace: Optional[torch.Tensor] = None,
                    out: Optional[dict] = None, smooth_k: bool = False, causal: bool = False,
                    attention_sink: bool = False, quantize_int8: bool = False,
                    quantize_fp8: bool = False) -> dict:
    """Stage 1 (sparge_build_block_map).  q [b, h, s_q, d], k [b, h_kv, s_k, d]
    with h a multiple of h_kv (query head j reads K head j // (h / h_kv)).

    nq = ceil(s_q / 64), nk = ceil(s_k / 64): a partial last block pools its
    own tokens.  Returns a dict with 'lut' int32 [b, h, nq, nk], 'count' int32 [b, h, nq],
    and with return_debug also 'bitmap', 'prob', 'sim_q', 'sim_k', 'q_mean',
    'k_mean'.  `out` may hold preallocated tensors under the same keys (plus
    'workspace').  smooth_k / causal / attention_sink set SPARGE_FLAG_SMOOTH_K /
    SPARGE_FLAG_CAUSAL / SPARGE_FLAG_ATTN_SINK.  quantize_int8 also returns the
    per-block int8 codes 'q_i8' [b, h, s_q, d], 'k_i8' [b, h_kv, s_k, d] and their
    scales 'q_i8_scale' [b, h, nq], 'k_i8_scale' [b, h_kv, nk]; 'k_mean' is
    [b, h_kv, nk, d] and 'sim_k' [b, h, nk] (the K gate as each query head
    sees it).  quantize_fp8 returns fp8 e4m3 codes instead (uint8 bytes) under
    'q_fp8', 'k_fp8' with 'q_fp8_scale', 'k_fp8_scale' (SPARGE_FLAG_QUANT_FP8).
    """
    return _block_map(q, k, topk, simthreshd1, cdfthreshd, softmax_scale, blk_q, blk_k, return_debug,
                      workspace, out, smooth_k, causal, attention_sink, quantize_int8, noalloc=False,
                      quantize_fp8=quantize_fp8)


def build_block_map_noalloc(q: torch.Tensor, k: torch.Tensor, topk, simthreshd1, cdfthreshd=None,
                            softmax_scale: float = 0.0, blk_q: int = 64, blk_k: int = 64,
                            return_debug: bool = False, out: Optional[dict] = None,
                            smooth_k: bool = False, causal: bool = False,
                            attention_sink: bool = False, quantize_int8: bool = False,
                            quantize_fp8: bool = False) -> dict:
    """build_block_map through sparge_build_block_map_noalloc: the library's
    static per-GPU scratch (NOALLOC_SCRATCH_BYTES) replaces the workspace.
    Outputs not given in `out` are still allocated here by torch; pass them
    all in `out` for a call that allocates nothing (e.g. under graph capture).
    Calls whose work overlaps on one GPU share the scratch and race."""
    return _block_map(q, k, topk, simthreshd1, cdfthreshd, softmax_scale, blk_q, blk_k, return_debug,
                      None, out, smooth_k, causal, attention_sink, quantize_int8, noalloc=True,
                      quantize_fp8=quantize_fp8)


def _block_map(q, k, topk, simthreshd1, cdfthreshd, softmax_scale, blk_q, blk_k, return_debug,
               workspace, out, smooth_k, causal, attention_sink, quantize_int8, noalloc,
               quantize_fp8=False) -> dict:
    """The implementation of build_block_map and build_block_map_noalloc."""
    lib = load_library()
    dev = _on_gpu(q, k)
    b, h, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    if k.shape[0] != b or k.shape[3] != d or h_kv == 0 or h % h_kv:
        raise SpargeError(SPARGE_ERR_INVALID, "q and k shapes disagree")
    if q.dtype != k.dtype:
        raise SpargeError(SPARGE_ERR_INVALID, "q and k dtypes disagree")
    nq, nk = -(-s_q // blk_q) if blk_q else 0, -(-s_k // blk_k) if blk_k else 0   # partial last blocks count
    out = dict(out or {})

    def get(key, shape, dtype):
        t = out.get(key)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
            out[key] = t
        return t

    lut = get("lut", (b, h, nq, nk), torch.int32)
    count = get("count", (b, h, nq), torch.int32)
    dbg = {}
    if return_debug:
        dbg = dict(bitmap=get("bitmap", (b, h, nq, nk), torch.uint8),
                   prob=get("prob", (b, h, nq, nk), torch.float32),
                   sim_q=get("sim_q", (b, h, nq), torch.uint8),
                   sim_k=get("sim_k", (b, h, nk), torch.uint8),
                   q_mean=get("q_mean", (b, h, nq, d), torch.float32),
                   k_mean=get("k_mean", (b, h_kv, nk, d), torch.float32))
    qz = {}
    if quantize_int8 and quantize_fp8:
        raise SpargeError(SPARGE_ERR_INVALID, "quantize_int8 and quantize_fp8 exclude each other")
    if quantize_int8:
        qz = dict(q_i8=get("q_i8", (b, h, s_q, d), torch.int8),
                  q_i8_scale=get("q_i8_scale", (b, h, nq), torch.float32),
                  k_i8=get("k_i8", (b, h_kv, s_k, d), torch.int8),
                  k_i8_scale=get("k_i8_scale", (b, h_kv, nk), torch.float32))
    if quantize_fp8:
        qz = dict(q_fp8=get("q_fp8", (b, h, s_q, d), torch.uint8),
                  q_fp8_scale=get("q_fp8_scale", (b, h, nq), torch.float32),
                  k_fp8=get("k_fp8", (b, h_kv, s_k, d), torch.uint8),
                  k_fp8_scale=get("k_fp8_scale", (b, h_kv, nk), torch.float32))
    for key in ("q_i8", "k_i8", "q_fp8", "k_fp8"):
        if key in qz and not qz[key].is_contiguous():
            raise SpargeError(SPARGE_ERR_INVALID, f"{key} must be contiguous")
    codes = ("q_fp8", "q_fp8_scale", "k_fp8", "k_fp8_scale") if quantize_fp8 else \
        ("q_i8", "q_i8_scale", "k_i8", "k_i8_scale")
    args = (_ptr(q), _ptr(k), _dt(q.dtype), b, h, h_kv, s_q, s_k, d, _strides(q), _strides(k), blk_q, blk_k,
            _f32_array(topk, h, "topk"), _f32_array(cdfthreshd, h, "cdfthreshd"),
            _f32_array(simthreshd1, h, "simthreshd1"), float(softmax_scale),
            _flags(smooth_k=smooth_k, causal=causal, attention_sink=attention_sink, quant_fp8=quantize_fp8),
            _ptr(lut), _ptr(count), _ptr(dbg.get("bitmap")), _ptr(dbg.get("prob")),
            _ptr(dbg.get("sim_q")), _ptr(dbg.get("sim_k")), _ptr(dbg.get("q_mean")),
            _ptr(dbg.get("k_mean")), *(_ptr(qz.get(key)) for key in codes))
    if noalloc:
        _check(lib.sparge_build_block_map_noalloc(*args, _stream(dev)))
        res = dict(lut=lut, count=count)
        res.update(dbg)
        res.update(qz)
        return res
    ws_bytes = lib.sparge_build_block_map_workspace(b, h, s_q, s_k, d, blk_q, blk_k)
    if workspace is None:
        workspace = out.get("workspace")
    if workspace is None:
        workspace = torch.empty(max(int(ws_bytes), 256), dtype=torch.uint8, device=dev)
        out["workspace"] = workspace
    _check(lib.sparge_build_block_map(*args, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(dev)))
    res = dict(lut=lut, count=count, workspace=workspace)
    res.update(dbg)
    res.update(qz)
    return res


def sparse_fmha_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    lut: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                    blk_q: int = 64, blk_k: int = 64, softmax_scale: float = 0.0,
                    num_splits: int = 1, out_dtype: Optional[torch.dtype] = None,
                    o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    return_lse: bool = True, causal: bool = False, pv_threshold: float = 0.0):
    """Stage 2 (sparse_fmha_fwd).  q [b, h_q, s_q, d]; k, v [b, h_kv, s_k, d].

    Block mode (64, 64): lut [b, h_lut, nq, L] (+ count [b, h_lut, nq]),
    nq = ceil(s_q / 64); lut None = dense.  Lengths need not be multiples of
    64.  Token mode (1, 1): lut [b, h_kv, L] token positions.
    With num_splits > 1 the outputs are partials o [S, b, h_q, s_q, d] and
    lse [S, b, h_q, s_q] (fp32 unless out_dtype says otherwise).  causal sets
    SPARGE_FLAG_CAUSAL (block mode, s_q = s_k).  pv_threshold > 0 lets the
    kernel skip the P.V product of a listed block for a whole Q-tile when
    every row of the tile scores more than that far below its running
    maximum (block mode, num_splits = 1).  Returns (o, lse).
    """
    lib = load_library()
    dev = _on_gpu(q, k, v, lut, count, o, lse)
    if q.dim() != 4:
        raise SpargeError(SPARGE_ERR_INVALID, f"q must be [b, h_q, s_q, d], got {tuple(q.shape)}")
    b, h_q, s_q, d = q.shape
    h_kv, s_k = k.shape[1], k.shape[2]
    if not (q.dtype == k.dtype == v.dtype):
        raise SpargeError(SPARGE_ERR_INVALID, "q, k, v dtypes disagree")
    _check_attn_shapes(q, k, v, o, lse, num_splits)
    if out_dtype is None:
        out_dtype = q.dtype if num_splits == 1 else torch.float32
    split_stride = 0
    if o is None:
        if num_splits == 1:
            o = torch.empty((b, h_q, s_q, d), dtype=out_dtype, device=dev)
        else:
            o = torch.empty((num_splits, b, h_q, s_q, d), dtype=out_dtype, device=dev)
    o4 = o if o.dim() == 4 else o[0]
    if num_splits > 1:
        split_stride = o.stride(0)
    if lse is None and (return_lse or num_splits > 1):
        shape = (b, h_q, s_q) if num_splits == 1 else (num_splits, b, h_q, s_q)
        lse = torch.empty(shape, dtype=torch.float32, device=dev)
    lut_row_len, lut_heads = 0, h_q
    if lut is not None:
        if lut.dtype != torch.int32 or not lut.is_contiguous():
            raise SpargeError(SPARGE_ERR_INVALID, "lut must be contiguous int32")
        lut_row_len = lut.shape[-1]
        lut_heads = lut.shape[1]
    if count is not None and (count.dtype != torch.int32 or not count.is_contiguous()):
        raise SpargeError(SPARGE_ERR_INVALID, "count must be contiguous int32")
    if blk_q == 64 and lut is not None:
        _check_lut_rows(lut, count, b, -(-s_q // 64))
    if blk_q == 1 and lut is not None and (lut.dim() != 3 or tuple(lut.shape[:2]) != (b, h_kv)):
        raise SpargeError(SPARGE_ERR_INVALID, f"token lists must be [b={b}, h_kv={h_kv}, L] (got {tuple(lut.shape)})")
    st = lib.sparse_fmha_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dt(q.dtype), _dt(o.dtype),
        b, h_q, h_kv, s_q, s_k, d, _strides(q), _strides(k), _strides(v), _strides(o4),
        blk_q, blk_k, _ptr(lut), _ptr(count), lut_row_len, lut_heads, float(softmax_scale),
        _flags(causal=causal), float(pv_threshold), int(num_splits), int(split_stride),
        _stream(dev))
    _check(st)
    return o, lse


def sparse_fmha_fwd_qk_int8(q_i8: torch.Tensor, q_scale: torch.Tensor, k_i8: torch.Tensor,
                            k_scale: torch.Tensor, v: torch.Tensor,
                            lut: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                            softmax_scale: float = 0.0, num_splits: int = 1,
                            out_dtype: Optional[torch.dtype] = None, o: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                            causal: bool = False, _fp8: bool = False):
    """Stage 2 on int8 Q/K codes (sparse_fmha_fwd_qk_int8), block mode.

    q_i8 [b, h_q, s_q, d] int8 with q_scale [b, h_q, ceil(s_q/64)]; k_i8 [b, h_kv,
    s_k, d] int8 with k_scale [b, h_kv, ceil(s_k/64)] (as build_block_map(...,
    quantize_int8=True) returns them); v [b, h_kv, s_k, d] fp16/bf16.  The LUT,
    splits and outputs are as in sparse_fmha_fwd.  Returns (o, lse).
    """
    lib = load_library()
    dev = _on_gpu(q_i8, q_scale, k_i8, k_scale, v, lut, count, o, lse)
    if q_i8.dim() != 4:
        raise SpargeError(SPARGE_ERR_INVALID, f"q_i8 must be [b, h_q, s_q, d], got {tuple(q_i8.shape)}")
    b, h_q, s_q, d = q_i8.shape
    h_kv, s_k = k_i8.shape[1], k_i8.shape[2]
    code_dt = torch.uint8 if _fp8 else torch.int8
    if q_i8.dtype != code_dt or k_i8.dtype != code_dt:
        raise SpargeError(SPARGE_ERR_INVALID, f"the Q and K codes must be {code_dt}")
    _check_attn_shapes(q_i8, k_i8, v, o, lse, num_splits)
    for name, t, shape in (("q_scale", q_scale, (b, h_q, -(-s_q // 64))), ("k_scale", k_scale, (b, h_kv, -(-s_k // 64)))):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise SpargeError(SPARGE_ERR_INVALID, f"{name} must be contiguous float32 {shape}")
    if out_dtype is None:
        out_dtype = v.dtype if num_splits == 1 else torch.float32
    split_stride = 0
    if o is None:
        shape = (b, h_q, s_q, d) if num_splits == 1 else (num_splits, b, h_q, s_q, d)
        o = torch.empty(shape, dtype=out_dtype, device=dev)
    o4 = o if o.dim() == 4 else o[0]
    if num_splits > 1:
        split_stride = o.stride(0)
    if lse is None and (return_lse or num_splits > 1):
        shape = (b, h_q, s_q) if num_splits == 1 else (num_splits, b, h_q, s_q)
        lse = torch.empty(shape, dtype=torch.float32, device=dev)
    lut_row_len, lut_heads = 0, h_q
    if lut is not None:
        if lut.dtype != torch.int32 or not lut.is_contiguous():
            raise SpargeError(SPARGE_ERR_INVALID, "lut must be contiguous int32")
        lut_row_len, lut_heads = lut.shape[-1], lut.shape[1]
        _check_lut_rows(lut, count, b, -(-s_q // 64))
    if count is not None and (count.dtype != torch.int32 or not count.is_contiguous()):
        raise SpargeError(SPARGE_ERR_INVALID, "count must be contiguous int32")
    entry = lib.sparse_fmha_fwd_qk_fp8 if _fp8 else lib.sparse_fmha_fwd_qk_int8
    st = entry(
        _ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(v), _ptr(o), _ptr(lse),
        _dt(v.dtype), _dt(o.dtype), b, h_q, h_kv, s_q, s_k, d, _strides(q_i8), _strides(k_i8),
        _strides(v), _strides(o4), _ptr(lut), _ptr(count), lut_row_len, lut_heads,
        float(softmax_scale), _flags(causal=causal), int(num_splits), int(split_stride), _stream(dev))
    _check(st)
    return o, lse


def sparse_fmha_fwd_qk_fp8(q_fp8: torch.Tensor, q_scale: torch.Tensor, k_fp8: torch.Tensor,
                           k_scale: torch.Tensor, v: torch.Tensor,
                           lut: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None, **kw):
    """Stage 2 on fp8 (e4m3) Q/K codes (sparse_fmha_fwd_qk_fp8), block mode:
    q_fp8 / k_fp8 uint8 e4m3 bytes with their per-block scales, as
    build_block_map(..., quantize_fp8=True) returns them.  Other arguments as
    sparse_fmha_fwd_qk_int8.  Returns (o, lse)."""
    return sparse_fmha_fwd_qk_int8(q_fp8, q_scale, k_fp8, k_scale, v, lut, count, _fp8=True, **kw)


def dense_fmha_fwd(q, k, v, softmax_scale: float = 0.0, **kw):
    """The dense baseline: sparse_fmha_fwd with no LUT (every block)."""
    return sparse_fmha_fwd(q, k, v, None, None, 64, 64, softmax_scale, **kw)


def attn_combine(o_parts: torch.Tensor, lse_parts: torch.Tensor,
                 out_dtype: Optional[torch.dtype] = None, o: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Merge n partials: o_parts [n, b, h, s, d] (each part contiguous), lse_parts
    [n, b, h, s] fp32.  Returns (o [b, h, s, d], lse [b, h, s])."""
    lib = load_library()
    dev = _on_gpu(o_parts, lse_parts, o, lse)
    n, b, h, s, d = o_parts.shape
    if lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise SpargeError(SPARGE_ERR_INVALID, "lse_parts must be contiguous fp32")
    if tuple(lse_parts.shape) != (n, b, h, s):
        raise SpargeError(SPARGE_ERR_INVALID, "lse_parts shape mismatch")
    if not o_parts[0].is_contiguous() or (n > 1 and not o_parts[1].is_contiguous()):
        raise SpargeError(SPARGE_ERR_INVALID, "each part must be contiguous")
    part_stride = o_parts.stride(0) if n > 1 else b * h * s * d
    if out_dtype is None:
        out_dtype = o_parts.dtype
    if o is not None and (tuple(o.shape) != (b, h, s, d) or not o.is_contiguous()):
        raise SpargeError(SPARGE_ERR_INVALID, f"o must be contiguous {(b, h, s, d)} (got {tuple(o.shape)})")
    if lse is not None and (tuple(lse.shape) != (b, h, s) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise SpargeError(SPARGE_ERR_INVALID, f"lse must be contiguous float32 {(b, h, s)}")
    if o is None:
        o = torch.empty((b, h, s, d), dtype=out_dtype, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((b, h, s), dtype=torch.float32, device=dev)
    st = lib.attn_combine(_ptr(o_parts), _dt(o_parts.dtype), _ptr(lse_parts), n, b, h, s, d,
                          int(part_stride), _ptr(o), _dt(o.dtype), _ptr(lse), _stream(dev))
    _check(st)
    return o, lse


def validate_lut(lut: torch.Tensor, count: Optional[torch.Tensor], n_blocks: int) -> int:
    """Number of malformed LUT rows (debug check, runs on the device)."""
    lib = load_library()
    dev = _on_gpu(lut, count)
    row_len = lut.shape[-1]
    rows = lut.numel() // row_len
    bad = torch.empty(1, dtype=torch.int32, device=dev)
    st = lib.sparge_validate_lut(_ptr(lut), _ptr(count), rows, row_len, int(n_blocks), _ptr(bad),
                                 _stream(dev))
    _check(st)
    return int(bad.item())


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
