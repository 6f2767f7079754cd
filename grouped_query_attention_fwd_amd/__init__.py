"""Grouped-query attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libgqa.so (include/gqa.h).  It only
marshals arguments: torch tensors become device pointers and the current HIP
stream is passed through; every step of the computation runs in the HIP
kernels.  There is no CPU fallback: if the library is missing or the tensors
are not on a GPU the call raises.

    decode(q, k, v, mask=None, out=None, out_dtype=None, workspace=None)
        q [B,H,1,D], k/v [B,H_kv,M,D], mask [B,1,M] bool/uint8 or None
    prefill(q, k, v, mask=None, causal=False, out=None, out_dtype=None)
        q [B,H,N,D], k/v [B,H_kv,M,D], mask [B,N,M] bool/uint8 or None
    prefill_band(q, k, v, mask=None, q_offset=0, window_left=-1, window_right=-1,
                 out=None, out_dtype=None)
        key j visible to query i iff i+q_offset-window_left <= j <= i+q_offset+window_right
        (a negative window leaves that side open)
    decode_paged(q, k_pool, v_pool, block_table, kv_len, out=None, out_dtype=None,
                 workspace=None)
        q [B,H,1,D], pools [num_blocks,H_kv,block_size,D], block_table
        [B,max_blocks] int32, kv_len [B] int32
    decode_noalloc(q, k, v, mask=None, out=None, out_dtype=None)
        decode with no workspace and no allocation inside the library (a fixed
        per-GPU scratch area of DECODE_NOALLOC_SCRATCH_BYTES; calls that may
        overlap on one GPU race on it)
    decode_workspace_size(B, H, H_kv, M, D) -> bytes
    decode_paged_workspace_size(B, H, H_kv, max_blocks, block_size, D) -> bytes
    status_string(code) -> str

Query head h reads KV head h // (H // H_kv) (repeat-interleave grouping),
scores are scaled by 1/sqrt(D), a mask entry that is False/0 hides the key
from every head, and causal means key j is visible to query i iff j <= i.
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["decode", "decode_noalloc", "decode_paged", "prefill", "prefill_band", "decode_op", "decode_paged_op",
           "prefill_op", "prefill_band_op",
           "decode_workspace_size", "decode_paged_workspace_size", "status_string",
           "library_path", "GQAError", "load_library", "DECODE_COUNTER_BYTES",
           "DECODE_NOALLOC_SCRATCH_BYTES"]

# Bytes of arrival counters at the start of a decode workspace; they must be
# zero before the first call, and every call leaves them zero.
DECODE_COUNTER_BYTES = 16384
# Size of the fixed per-GPU scratch area of decode_noalloc.
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgqa.so")
_lib = None

GQA_F32, GQA_BF16, GQA_F16 = 0, 1, 2
_STATUS_VALUE_ERRORS = {1, 2, 3, 4, 5, 6, 7, 9, 10}


class GQAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"gqa status {code}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library(path=None):
    """Load libgqa.so once; raise if it has not been built.  `path` loads
    another build of the same library instead (the benchmark's timing build),
    and only before the first load."""
    global _lib
    if _lib is not None:
        if path is not None and path != _lib._name:
            raise RuntimeError(f"{_lib._name} is already loaded")
        return _lib
    path = _LIB_PATH if path is None else path
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not built: {path} is missing "
            "(build it with `python -m grouped_query_attention_fwd_amd._build`)")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.gqa_decode.restype = i
    lib.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.gqa_decode_noalloc.restype = i
    lib.gqa_prefill.argtypes = [vp, vp, vp, vp, i, vp, i, i, i, i, i, i, i, i, vp]
    lib.gqa_prefill.restype = i
    lib.gqa_prefill_band.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, vp]
    lib.gqa_prefill_band.restype = i
    lib.gqa_decode_workspace_size.argtypes = [i, i, i, i, i]
    lib.gqa_decode_workspace_size.restype = sz
    lib.gqa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, sz,
                                     vp]
    lib.gqa_decode_paged.restype = i
    lib.gqa_decode_paged_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.gqa_decode_paged_workspace_size.restype = sz
    lib.gqa_status_string.argtypes = [i]
    lib.gqa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().gqa_status_string(int(code)).decode()


def _check(code: int):
    if code != 0:
        msg = status_string(code)
        if code in _STATUS_VALUE_ERRORS:
            raise ValueError(f"gqa status {code}: {msg}")
        raise GQAError(code, msg)


def decode_workspace_size(B, H, H_kv, M, D) -> int:
    return int(load_library().gqa_decode_workspace_size(B, H, H_kv, M, D))


def decode_paged_workspace_size(B, H, H_kv, max_blocks, block_size, D) -> int:
    return int(load_library().gqa_decode_paged_workspace_size(B, H, H_kv, max_blocks,
                                                              block_size, D))


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t == torch.float32:
        return GQA_F32
    if t == torch.bfloat16:
        return GQA_BF16
    if t == torch.float16:
        return GQA_F16
    raise ValueError(f"unsupported dtype {t} (float32, bfloat16 or float16)")


def _check_tensors(q, k, v, mask, same_batch=True):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU (no CPU path)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have the same dtype")
    if k.shape != v.shape or k.shape[3] != q.shape[3] or (same_batch and k.shape[0] != q.shape[0]):
        raise ValueError("k and v must have the same shape, with q's D (and B, unpaged)")
    if mask is not None:
        if not mask.is_cuda or mask.device != q.device:
            raise ValueError("mask must be on the same GPU as q")
        if not mask.is_contiguous():
            raise ValueError("mask must be contiguous")
        if mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be bool or uint8")


def _mask_ptr(mask):
    if mask is None:
        return None
    # bool and uint8 share the one-byte layout; nonzero = visible
    return mask.data_ptr()


def _out(q, out, out_dtype, shape):
    torch = _torch()
    od = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(shape, dtype=od, device=q.device)
    else:
        if tuple(out.shape) != tuple(shape) or out.dtype != od or not out.is_contiguous() \
                or out.device != q.device:
            raise ValueError("out has the wrong shape, dtype, device or layout")
    return out


# Decode workspaces kept per (device, stream) for the one-shot calls,
# zero-filled when allocated.  Every decode call leaves the counter area zero
# again, so calls queued on one stream can share one buffer; calls on
# different streams get different buffers.  A buffer only grows (a larger,
# zeroed one replaces it).
_STREAM_WS = {}
_STREAM_WS_MAX = 16


def _stream_workspace(device, need):
    torch = _torch()
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _STREAM_WS.get(key)
    if ws is None or ws.numel() < need:
        with torch.cuda.device(device):
            ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _STREAM_WS.pop(key, None)
        if len(_STREAM_WS) >= _STREAM_WS_MAX:
            _STREAM_WS.pop(next(iter(_STREAM_WS)))
        _STREAM_WS[key] = ws
    return ws


def _workspace(q, need, workspace, shared):
    if workspace is not None or need == 0:
        return workspace
    if shared:
        return _stream_workspace(q.device, need)
    return _torch().zeros(need, dtype=_torch().uint8, device=q.device)


def _prepare_decode(q, k, v, mask, out, out_dtype, workspace, shared=False):
    torch = _torch()
    _check_tensors(q, k, v, mask)
    B, H, N, D = q.shape
    _, H_kv, M, _ = k.shape
    if N != 1:
        raise ValueError("decode takes one query position (q [B,H,1,D])")
    if mask is not None and tuple(mask.shape) != (B, 1, M):
        raise ValueError("decode mask must be [B,1,M]")
    out = _out(q, out, out_dtype, (B, H, 1, D))
    lib = load_library()
    need = int(lib.gqa_decode_workspace_size(B, H, H_kv, M, D))
    workspace = _workspace(q, need, workspace, shared)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), _mask_ptr(mask), out.data_ptr(),
            B, H, H_kv, M, D, _dtype_code(q.dtype), _dtype_code(out.dtype), ws_ptr, ws_bytes)
    return lib, args, out, workspace


def _prepare_decode_paged(q, k_pool, v_pool, block_table, kv_len, out, out_dtype, workspace,
                          shared=False):
    torch = _torch()
    _check_tensors(q, k_pool, v_pool, None, same_batch=False)
    B, H, N, D = q.shape
    num_blocks, H_kv, block_size, _ = k_pool.shape
    if N != 1:
        raise ValueError("decode takes one query position (q [B,H,1,D])")
    for name, t in (("block_table", block_table), ("kv_len", kv_len)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a tensor on the same GPU as q")
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    if tuple(kv_len.shape) != (B,):
        raise ValueError("kv_len must be [B]")
    max_blocks = block_table.shape[1]
    out = _out(q, out, out_dtype, (B, H, 1, D))
    lib = load_library()
    need = int(lib.gqa_decode_paged_workspace_size(B, H, H_kv, max_blocks, block_size, D))
    workspace = _workspace(q, need, workspace, shared)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
            kv_len.data_ptr(), out.data_ptr(), B, H, H_kv, max_blocks, block_size, num_blocks,
            D, _dtype_code(q.dtype), _dtype_code(out.dtype), ws_ptr, ws_bytes)
    return lib, args, out, workspace


def _prepare_prefill(q, k, v, mask, causal, out, out_dtype):
    _check_tensors(q, k, v, mask)
    B, H, N, D = q.shape
    _, H_kv, M, _ = k.shape
    if mask is not None and tuple(mask.shape) != (B, N, M):
        raise ValueError("prefill mask must be [B,N,M]")
    out = _out(q, out, out_dtype, (B, H, N, D))
    lib = load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), _mask_ptr(mask), 1 if causal else 0,
            out.data_ptr(), B, H, H_kv, N, M, D, _dtype_code(q.dtype), _dtype_code(out.dtype))
    return lib, args, out


def _prepare_prefill_band(q, k, v, mask, q_offset, window_left, window_right, out, out_dtype):
    _check_tensors(q, k, v, mask)
    B, H, N, D = q.shape
    _, H_kv, M, _ = k.shape
    if mask is not None and tuple(mask.shape) != (B, N, M):
        raise ValueError("prefill mask must be [B,N,M]")
    out = _out(q, out, out_dtype, (B, H, N, D))
    lib = load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), _mask_ptr(mask), out.data_ptr(),
            B, H, H_kv, N, M, D, int(q_offset), int(window_left), int(window_right),
            _dtype_code(q.dtype), _dtype_code(out.dtype))
    return lib, args, out


class _PreparedOp:
    """A validated, marshalled call: calling it only passes the current
    stream and enqueues the kernels.  The tensors it was built from must stay
    alive and unchanged in shape while it is used."""

    def __init__(self, fn, args, out, keep):
        self._fn, self._args, self.out, self._keep = fn, args, out, keep
        torch = _torch()
        self._device = out.device
        self._stream_of = torch.cuda.current_stream

    def __call__(self, stream=None):
        s = stream if stream is not None else self._stream_of(self._device)
        _check(self._fn(*self._args, s.cuda_stream))
        return self.out


def decode_op(q, k, v, mask=None, out=None, out_dtype=None, workspace=None):
    """Prepared decode call for tight loops (e.g. a serving step or HIP
    graph capture): validation and marshalling happen once here."""
    lib, args, out, ws = _prepare_decode(q, k, v, mask, out, out_dtype, workspace)
    return _PreparedOp(lib.gqa_decode, args, out, (q, k, v, mask, ws))


def decode_paged_op(q, k_pool, v_pool, block_table, kv_len, out=None, out_dtype=None,
                    workspace=None):
    """Prepared paged decode call; see decode_op.  The table and lengths are
    read by the kernel at every call, so they may change between calls."""
    lib, args, out, ws = _prepare_decode_paged(q, k_pool, v_pool, block_table, kv_len, out,
                                               out_dtype, workspace)
    return _PreparedOp(lib.gqa_decode_paged, args, out,
                       (q, k_pool, v_pool, block_table, kv_len, ws))


def prefill_op(q, k, v, mask=None, causal=False, out=None, out_dtype=None):
    """Prepared prefill call; see decode_op."""
    lib, args, out = _prepare_prefill(q, k, v, mask, causal, out, out_dtype)
    return _PreparedOp(lib.gqa_prefill, args, out, (q, k, v, mask))


def prefill_band_op(q, k, v, mask=None, q_offset=0, window_left=-1, window_right=-1, out=None,
                    out_dtype=None):
    """Prepared banded prefill call; see decode_op."""
    lib, args, out = _prepare_prefill_band(q, k, v, mask, q_offset, window_left, window_right,
                                           out, out_dtype)
    return _PreparedOp(lib.gqa_prefill_band, args, out, (q, k, v, mask))


def decode(q, k, v, mask=None, out=None, out_dtype=None, workspace=None):
    """One decode step; see the module docstring.  workspace: optional
    uint8 device tensor of at least decode_workspace_size(...) bytes whose
    first DECODE_COUNTER_BYTES bytes are zero before its first use (every
    call leaves them so).  When omitted, a buffer kept for the current
    stream is used."""
    torch = _torch()
    lib, args, out, _ws = _prepare_decode(q, k, v, mask, out, out_dtype, workspace, shared=True)
    with torch.cuda.device(q.device):
        _check(lib.gqa_decode(*args, torch.cuda.current_stream(q.device).cuda_stream))
    return out


def decode_noalloc(q, k, v, mask=None, out=None, out_dtype=None):
    """decode() through gqa_decode_noalloc: no workspace, and the library
    allocates nothing (its key-split scratch is a fixed area of
    DECODE_NOALLOC_SCRATCH_BYTES per GPU; larger problems raise ValueError).
    Calls that may overlap on one GPU race on that area.  `out` may be given
    to avoid the one allocation this binding would otherwise make."""
    torch = _torch()
    _check_tensors(q, k, v, mask)
    B, H, N, D = q.shape
    _, H_kv, M, _ = k.shape
    if N != 1:
        raise ValueError("decode takes one query position (q [B,H,1,D])")
    if mask is not None and tuple(mask.shape) != (B, 1, M):
        raise ValueError("decode mask must be [B,1,M]")
    out = _out(q, out, out_dtype, (B, H, 1, D))
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.gqa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _mask_ptr(mask),
                                      out.data_ptr(), B, H, H_kv, M, D, _dtype_code(q.dtype),
                                      _dtype_code(out.dtype),
                                      torch.cuda.current_stream(q.device).cuda_stream))
    return out


def decode_paged(q, k_pool, v_pool, block_table, kv_len, out=None, out_dtype=None,
                 workspace=None):
    """One decode step over a paged KV cache: key t of sequence b is row
    t % block_size of pool block block_table[b, t // block_size], and only
    keys t < kv_len[b] exist.  Workspace as for decode()."""
    torch = _torch()
    lib, args, out, _ws = _prepare_decode_paged(q, k_pool, v_pool, block_table, kv_len, out,
                                                out_dtype, workspace, shared=True)
    with torch.cuda.device(q.device):
        _check(lib.gqa_decode_paged(*args, torch.cuda.current_stream(q.device).cuda_stream))
    return out


def prefill(q, k, v, mask=None, causal=False, out=None, out_dtype=None):
    """Prefill forward; see the module docstring."""
    torch = _torch()
    lib, args, out = _prepare_prefill(q, k, v, mask, causal, out, out_dtype)
    with torch.cuda.device(q.device):
        _check(lib.gqa_prefill(*args, torch.cuda.current_stream(q.device).cuda_stream))
    return out


def prefill_band(q, k, v, mask=None, q_offset=0, window_left=-1, window_right=-1, out=None,
                 out_dtype=None):
    """Prefill with each query's keys limited to a band around its position
    i + q_offset: window_left keys before it and window_right keys after it
    (negative = unbounded).  Causal is window_right=0; q_offset=M-N places
    the queries at the end of the keys; window_left=W-1, window_right=0 is a
    sliding window of W keys."""
    torch = _torch()
    lib, args, out = _prepare_prefill_band(q, k, v, mask, q_offset, window_left, window_right,
                                           out, out_dtype)
    with torch.cuda.device(q.device):
        _check(lib.gqa_prefill_band(*args, torch.cuda.current_stream(q.device).cuda_stream))
    return out
