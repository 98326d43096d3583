"""Exact tiled attention for AMD MI355X (gfx950).

Python binding of libfa_mi355x.so, whose C ABI is declared in include/fa.h.
This module only marshals arguments: it checks tensor placement, shape and
dtype, allocates outputs with torch when the caller does not pass them, and
hands raw device pointers and the current HIP stream to the library. Every
step of the computation runs in the library's HIP kernels. There is no
fallback: if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "FAError", "forward", "decode_paged", "merge_partials", "decode_plan",
    "decode_max_splits", "decode_workspace_size", "lib", "LIB_PATH", "MAX_SPLITS", "PAGE_SIZE",
    "version",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_mi355x.so")
MAX_SPLITS = 64
PAGE_SIZE = 16

_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_LIB = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SIGNATURES = {
    "fa_forward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_forward_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                              _I, _F, _I, _I, _I, _P]),
    "fa_cascade_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "fa_cascade_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_cascade": (_I, [_P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                        _I, _I, _F, _I, _I, _I, _P, ctypes.c_size_t, _P]),
    "fa_decode_max_splits": (_I, [_I, _I, _I, _I, _I]),
    "fa_decode_plan": (_I, [_P, _I, _I, _I, _I, _I, _P]),
    "fa_decode_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                             _I, _I, _P, ctypes.c_size_t, _P]),
    "fa_decode_paged_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                _I, _I, _F, _I, _I, _P, ctypes.c_size_t, _P]),
    "fa_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                     _F, _I, _I, _F, _I, _I, _P]),
    "fa_decode_graph_create": (_I, [ctypes.POINTER(ctypes.c_void_p), _P, _P, _P, _P, _P, _P,
                                    _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _F, _I, _I, _P,
                                    ctypes.c_size_t]),
    "fa_decode_graph_launch": (_I, [_P, _P]),
    "fa_decode_graph_destroy": (None, [_P]),
    "fa_merge_partials": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_stream_read": (_I, [_P, ctypes.c_size_t, _P, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_version": (ctypes.c_char_p, []),
}


class FAError(RuntimeError):
    """A call into the library returned a status other than FA_OK."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded library with its argument and return types declared."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m exact_tiled_attention_11_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def version() -> str:
    return lib().fa_version().decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FAError(status, where)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return t.data_ptr()


def _code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {dtype}")
    return _DTYPE[dtype]


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def forward(q, k, v, causal: bool = False, scale: float | None = None, out_dtype=None,
            out=None, lse=None):
    """Exact attention forward. q [B,Nq,H,d], k/v [B,Nk,Hkv,d] -> (O [B,Nq,H,d], LSE [B,H,Nq])."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Nq,H,d] and k, v [B,Nk,Hkv,d]")
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v batch or head dim differ from q")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Nq, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, Nq, H, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out/lse shapes do not match")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().fa_forward(_dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                          _dev(out, "out", out_dtype), _dev(lse, "lse", torch.float32),
                          B, H, Hkv, Nq, Nk, d, scale, int(bool(causal)), _code(q.dtype),
                          _code(out_dtype), _stream(q.device))
    _check(st, "fa_forward")
    return out, lse


def forward_paged(q, qo_indptr, k_pool, v_pool, block_table, kv_lens, max_q_len: int,
                  causal: bool = False, scale: float | None = None, out_dtype=None, out=None,
                  lse=None):
    """Ragged queries over a paged cache. q [total_q,H,d]; qo_indptr [B+1] int32; pools
    [P,16,Hkv,d]; block_table [B,max_pages] int32; kv_lens [B] int32
    -> (O [total_q,H,d], LSE [total_q,H])."""
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [total_q,H,d] and pools [P,page,Hkv,d]")
    total_q, H, d = q.shape
    num_pages, page, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    B = kv_lens.shape[0]
    if tuple(qo_indptr.shape) != (B + 1,) or block_table.dim() != 2 or \
            block_table.shape[0] != B:
        raise ValueError("qo_indptr must be [B+1] and block_table [B, max_pages]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((total_q, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().fa_forward_paged(
        _dev(q, "q"), _dev(qo_indptr, "qo_indptr", torch.int32), _dev(k_pool, "k_pool", q.dtype),
        _dev(v_pool, "v_pool", q.dtype), _dev(block_table, "block_table", torch.int32),
        _dev(kv_lens, "kv_lens", torch.int32), _dev(out, "out", out_dtype),
        _dev(lse, "lse", torch.float32), B, H, Hkv, d, total_q, int(max_q_len), page,
        block_table.shape[1], num_pages, scale, int(bool(causal)), _code(q.dtype),
        _code(out_dtype), _stream(q.device))
    _check(st, "fa_forward_paged")
    return out, lse


def cascade(q, qo_indptr, k_pool, v_pool, prefix_pages, prefix_len: int, block_table, kv_lens,
            max_q_len: int, causal: bool = False, prefix_splits: int = 0,
            scale: float | None = None, out_dtype=None, out=None, lse=None, workspace=None):
    """Ragged queries over a paged cache whose sequences share one prefix
    (prefix_pages [ceil(prefix_len/16)] int32), the prefix attended once for all
    queries. Shapes as forward_paged -> (O [total_q,H,d], LSE [total_q,H])."""
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [total_q,H,d] and pools [P,page,Hkv,d]")
    total_q, H, d = q.shape
    num_pages, page, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    B = kv_lens.shape[0]
    if tuple(qo_indptr.shape) != (B + 1,) or block_table.dim() != 2 or \
            block_table.shape[0] != B:
        raise ValueError("qo_indptr must be [B+1] and block_table [B, max_pages]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((total_q, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    S = cascade_num_splits(prefix_len, total_q, H, Hkv, prefix_splits)
    if workspace is None and prefix_len > 0 and total_q > 0:
        workspace = torch.empty(cascade_workspace_size(total_q, H, d, S), dtype=torch.uint8,
                                device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    pp = _dev(prefix_pages, "prefix_pages", torch.int32) if prefix_pages is not None else None
    st = lib().fa_cascade(
        _dev(q, "q"), _dev(qo_indptr, "qo_indptr", torch.int32), _dev(k_pool, "k_pool", q.dtype),
        _dev(v_pool, "v_pool", q.dtype), pp, int(prefix_len), int(prefix_splits),
        _dev(block_table, "block_table", torch.int32), _dev(kv_lens, "kv_lens", torch.int32),
        _dev(out, "out", out_dtype), _dev(lse, "lse", torch.float32), B, H, Hkv, d, total_q,
        int(max_q_len), page, block_table.shape[1], num_pages, scale, int(bool(causal)),
        _code(q.dtype), _code(out_dtype), ws_ptr, ws_bytes, _stream(q.device))
    _check(st, "fa_cascade")
    return out, lse


def cascade_num_splits(prefix_len: int, total_q: int, H: int, Hkv: int,
                       prefix_splits: int = 0) -> int:
    return lib().fa_cascade_num_splits(prefix_len, total_q, H, Hkv, prefix_splits)


def cascade_workspace_size(total_q: int, H: int, d: int, num_splits: int) -> int:
    return int(lib().fa_cascade_workspace_size(total_q, H, d, num_splits))


def decode_max_splits(B: int, Hkv: int, max_pages_per_seq: int, window: int = 0,
                      num_splits: int = 0) -> int:
    """Partial slots per (sequence, head): the most key chunks any sequence can get."""
    return lib().fa_decode_max_splits(int(B), int(Hkv), int(max_pages_per_seq), int(window),
                                      int(num_splits))


def decode_plan(seq_lens, Hkv: int, max_pages_per_seq: int, window: int = 0,
                num_splits: int = 0):
    """The decode's split plan for a host list of sequence lengths: chunks per sequence."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    out = np.zeros(lens.shape[0], dtype=np.int32)
    st = lib().fa_decode_plan(lens.ctypes.data if lens.size else None, int(lens.shape[0]),
                              int(Hkv), int(max_pages_per_seq), int(window), int(num_splits),
                              out.ctypes.data if out.size else None)
    _check(st, "fa_decode_plan")
    return out


def decode_workspace_size(B: int, H: int, Hkv: int, d: int, max_pages_per_seq: int,
                          window: int = 0, num_splits: int = 0) -> int:
    return int(lib().fa_decode_workspace_size(int(B), int(H), int(Hkv), int(d),
                                              int(max_pages_per_seq), int(window),
                                              int(num_splits)))


def _decode(entry, q, k_pool, v_pool, block_table, seq_lens, scale, num_splits, out_dtype, out,
            lse, workspace, extra):
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [B,H,d] and pools [P,page,Hkv,d]")
    B, H, d = q.shape
    num_pages, page, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    window = extra[0] if extra else 0
    S = decode_max_splits(B, Hkv, block_table.shape[1], window, num_splits) if B > 0 else 1
    need = decode_workspace_size(B, H, Hkv, d, block_table.shape[1], window, num_splits) \
        if B > 0 else 0
    if workspace is None and S > 1 and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = getattr(lib(), entry)
    st = fn(_dev(q, "q"), _dev(k_pool, "k_pool", q.dtype), _dev(v_pool, "v_pool", q.dtype),
            _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
            _dev(out, "out", out_dtype), _dev(lse, "lse", torch.float32),
            B, H, Hkv, d, page, block_table.shape[1], num_pages, scale, int(num_splits), *extra,
            _code(q.dtype), _code(out_dtype), ws_ptr, ws_bytes, _stream(q.device))
    _check(st, entry)
    return out, lse


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float | None = None,
                 num_splits: int = 0, out_dtype=None, out=None, lse=None, workspace=None):
    """Paged decode. q [B,H,d]; pools [P,16,Hkv,d]; block_table [B,max_pages] int32;
    seq_lens [B] int32 -> (O [B,H,d], LSE [B,H])."""
    return _decode("fa_decode_paged", q, k_pool, v_pool, block_table, seq_lens, scale,
                   num_splits, out_dtype, out, lse, workspace, ())


def decode_paged_ex(q, k_pool, v_pool, block_table, seq_lens, window: int = 0,
                    softcap: float = 0.0, scale: float | None = None, num_splits: int = 0,
                    out_dtype=None, out=None, lse=None, workspace=None):
    """Paged decode with a sliding window (newest `window` tokens visible, 0 = all) and
    logit soft-capping (scaled scores x -> softcap*tanh(x/softcap), 0 = off)."""
    return _decode("fa_decode_paged_ex", q, k_pool, v_pool, block_table, seq_lens, scale,
                   num_splits, out_dtype, out, lse, workspace, (int(window), float(softcap)))


def decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, window: int = 0,
                         softcap: float = 0.0, scale: float | None = None, num_splits: int = 0,
                         out_dtype=None, out=None, lse=None):
    """decode_paged_ex whose partials live in the library's own per-device scratch
    buffer (fa_decode_paged_noalloc): no workspace. With `out` and `lse` given,
    nothing is allocated at all. Calls that overlap in time on one device race."""
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [B,H,d] and pools [P,page,Hkv,d]")
    B, H, d = q.shape
    num_pages, page, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        st = lib().fa_decode_paged_noalloc(
            _dev(q, "q"), _dev(k_pool, "k_pool", q.dtype), _dev(v_pool, "v_pool", q.dtype),
            _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
            _dev(out, "out", out_dtype), _dev(lse, "lse", torch.float32), B, H, Hkv, d, page,
            block_table.shape[1], num_pages, scale, int(num_splits), int(window), float(softcap),
            _code(q.dtype), _code(out_dtype), _stream(q.device))
    _check(st, "fa_decode_paged_noalloc")
    return out, lse


class DecodeGraph:
    """A paged decode step recorded once as a HIP graph (fa_decode_graph_*).

    The graph binds the tensors given at construction; write each step's inputs
    into them (q, the caches, block_table, seq_lens) and call `launch()`; the
    results land in `out` and `lse`. Keep every tensor alive and unmoved while
    the graph exists.
    """

    def __init__(self, q, k_pool, v_pool, block_table, seq_lens, window: int = 0,
                 softcap: float = 0.0, scale: float | None = None, num_splits: int = 0,
                 out_dtype=None, out=None, lse=None, workspace=None):
        if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
            raise ValueError("expected q [B,H,d] and pools [P,page,Hkv,d]")
        B, H, d = q.shape
        num_pages, page, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
        if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
            raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
        out_dtype = q.dtype if out_dtype is None else out_dtype
        self.out = out if out is not None else torch.empty((B, H, d), dtype=out_dtype,
                                                           device=q.device)
        self.lse = lse if lse is not None else torch.empty((B, H), dtype=torch.float32,
                                                           device=q.device)
        S = decode_max_splits(B, Hkv, block_table.shape[1], window, num_splits) if B > 0 else 1
        need = decode_workspace_size(B, H, Hkv, d, block_table.shape[1], window, num_splits) \
            if B > 0 else 0
        if workspace is None and S > 1 and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        self.workspace = workspace
        # the graph holds raw pointers: keep the tensors referenced
        self._keep = (q, k_pool, v_pool, block_table, seq_lens)
        self.device = q.device
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        handle = ctypes.c_void_p()
        st = lib().fa_decode_graph_create(
            ctypes.byref(handle), _dev(q, "q"), _dev(k_pool, "k_pool", q.dtype),
            _dev(v_pool, "v_pool", q.dtype), _dev(block_table, "block_table", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32), _dev(self.out, "out", out_dtype),
            _dev(self.lse, "lse", torch.float32), B, H, Hkv, d, page, block_table.shape[1],
            num_pages, scale, int(num_splits), int(window), float(softcap), _code(q.dtype),
            _code(out_dtype), ws_ptr, ws_bytes)
        _check(st, "fa_decode_graph_create")
        self._handle = handle

    def launch(self, stream=None):
        s = _stream(self.device) if stream is None else stream.cuda_stream
        _check(lib().fa_decode_graph_launch(self._handle, s), "fa_decode_graph_launch")
        return self.out, self.lse

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            lib().fa_decode_graph_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


def merge_partials(o_parts, lse_parts, num_parts=None, out_dtype=torch.float32, out=None,
                   lse=None):
    """Merge partials. o_parts [R,S,d] fp32, lse_parts [R,S] fp32, num_parts [R] int32
    or None -> (O [R,d] out_dtype, LSE [R] fp32)."""
    if o_parts.dim() != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("expected o_parts [R,S,d] and lse_parts [R,S]")
    R, S, d = o_parts.shape
    if out is None:
        out = torch.empty((R, d), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
    np_ptr = _dev(num_parts, "num_parts", torch.int32) if num_parts is not None else None
    st = lib().fa_merge_partials(_dev(o_parts, "o_parts", torch.float32),
                                 _dev(lse_parts, "lse_parts", torch.float32), np_ptr,
                                 _dev(out, "out", out_dtype), _dev(lse, "lse", torch.float32),
                                 R, S, d, _code(out_dtype), _stream(o_parts.device))
    _check(st, "fa_merge_partials")
    return out, lse


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Diagnostic: read every byte of the contiguous device tensor `buf` once
    (the achievable-bandwidth yardstick for memory-bound kernels); `sink` is
    a one-element int32 device tensor the kernel may write."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check(lib().fa_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                _dev(sink, "sink", torch.int32), _stream(buf.device)),
           "fa_stream_read")
