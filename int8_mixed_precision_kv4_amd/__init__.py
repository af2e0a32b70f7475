"""Python binding of libkv4 (include/kv4.h): KV4-RL hybrid decode attention on
MI355X.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; PyTorch only provides device memory and the current stream.  There is
no fallback: if libkv4.so has not been built, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkv4.so")
ABI_VERSION = 1
HEAD_DIM, PAGE, SINK, WINDOW, SIDE_ROWS, BLOCK_BYTES = 128, 16, 16, 128, 144, 2176

# Every extern "C" function of include/kv4.h.
EXPORTS = ("kv4_append", "kv4_prefill_quantize", "kv4_decode_workspace_bytes",
           "kv4_decode_attention", "kv4_decode_attention_debug", "kv4_strerror",
           "kv4bench_bf16_workspace_bytes", "kv4bench_bf16_paged_decode",
           "kv4bench_decode_attention_timed", "kv8_append", "kv8_prefill_quantize",
           "kv8_decode_workspace_bytes", "kv8_decode_attention", "kv8_decode_attention_debug",
           "kv4mx_append", "kv4mx_prefill_quantize", "kv4mx_decode_attention",
           "kv4_prefill_attention_workspace_bytes", "kv4_prefill_attention",
           "kv4_prefill_attention_debug", "kv4_append_decode_attention",
           "kv4_append_decode_attention_noalloc")
NOALLOC_SCRATCH_BYTES = 32 << 20  # KV4_NOALLOC_SCRATCH_BYTES
KV8_BLOCK_BYTES = 4160

_lib = None


class Kv4Error(RuntimeError):
    pass


class _Desc(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("sink", C.c_int32),
                ("window", C.c_int32), ("max_slots", C.c_int32), ("pages", C.c_void_p),
                ("side_codes", C.c_void_p), ("side_scales", C.c_void_p)]


class _Kv8Desc(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("pages", C.c_void_p)]


class _Debug(C.Structure):
    _fields_ = [("qcodes", C.c_void_p), ("qsum", C.c_void_p), ("qk", C.c_void_p),
                ("pcode", C.c_void_p), ("pv", C.c_void_p), ("max_ctx", C.c_int32),
                ("max_pages", C.c_int32)]


def lib():
    """Load libkv4.so (built by int8_mixed_precision_kv4_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Kv4Error(f"{LIB_PATH} is missing: build it with "
                           "`python int8_mixed_precision_kv4_amd/build.py`")
        L = C.CDLL(LIB_PATH)
        P, I, F, Z = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
        D = C.POINTER(_Desc)
        L.kv4_append.argtypes = [D, P, P, P, P, P, I, I, P]
        L.kv4_prefill_quantize.argtypes = [D, P, P, P, P, P, P, I, I, I, P]
        L.kv4_decode_workspace_bytes.argtypes = [D, I, I, I]
        L.kv4_decode_workspace_bytes.restype = Z
        L.kv4_decode_attention.argtypes = [D, P, P, P, P, I, I, I, I, F, P, P, P, Z, P]
        L.kv4_decode_attention_debug.argtypes = [D, P, P, P, P, I, I, I, I, F, P, P, P, Z,
                                                 C.POINTER(_Debug), P]
        L.kv4_strerror.argtypes = [C.c_int]
        L.kv4_strerror.restype = C.c_char_p
        L.kv4bench_bf16_workspace_bytes.argtypes = [I, I, I, I]
        L.kv4bench_bf16_workspace_bytes.restype = Z
        L.kv4bench_bf16_paged_decode.argtypes = [P, I, I, P, P, P, I, I, I, I, F, P, P, P, Z, P]
        L.kv4bench_decode_attention_timed.argtypes = [D, P, P, P, P, P, P, P, I, I, I, I, F, P, P,
                                                      P, Z, P, P, P]
        L.kv4_append_decode_attention.argtypes = [D, P, P, P, P, P, P, P, I, I, I, I, F, P, P, P, Z, P]
        L.kv4_append_decode_attention_noalloc.argtypes = [D, P, P, P, P, P, P, P, I, I, I, I, F, P, P, P]
        L.kv4_prefill_attention_workspace_bytes.argtypes = [D, I, I, I]
        L.kv4_prefill_attention_workspace_bytes.restype = Z
        L.kv4_prefill_attention.argtypes = [D, P, P, P, P, P, I, I, I, I, I, F, P, P, P, Z, P]
        L.kv4_prefill_attention_debug.argtypes = [D, P, P, P, P, P, I, I, I, I, I, F, P, P, P, Z,
                                                  C.POINTER(_Debug), P]
        L.kv4mx_append.argtypes = [D, P, P, P, P, P, I, I, P]
        L.kv4mx_prefill_quantize.argtypes = [D, P, P, P, P, P, P, I, I, I, P]
        L.kv4mx_decode_attention.argtypes = [D, P, P, P, P, I, I, I, I, F, P, P, P, Z, P]
        D8 = C.POINTER(_Kv8Desc)
        L.kv8_append.argtypes = [D8, P, P, P, P, I, I, P]
        L.kv8_prefill_quantize.argtypes = [D8, P, P, P, P, P, I, I, I, P]
        L.kv8_decode_workspace_bytes.argtypes = [D8, I, I, I]
        L.kv8_decode_workspace_bytes.restype = Z
        L.kv8_decode_attention.argtypes = [D8, P, P, P, I, I, I, I, F, P, P, P, Z, P]
        L.kv8_decode_attention_debug.argtypes = [D8, P, P, P, I, I, I, I, F, P, P, P, Z,
                                                 C.POINTER(_Debug), P]
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise Kv4Error(f"kv4 error {rc}: {lib().kv4_strerror(rc).decode()}")


def _ptr(t):
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous()):
        raise Kv4Error("device tensors must be contiguous CUDA tensors")
    return C.c_void_p(t.data_ptr())


def _want(t, dtype, what, rows=None, ndim=None, optional=False):
    """Host-side check of one argument before it reaches the library, which
    reads it on the device with the given element type: dtype, and (when
    given) the number of dimensions and at least `rows` leading rows."""
    if t is None:
        if optional:
            return
        raise Kv4Error(f"{what} is required")
    if t.dtype != dtype:
        raise Kv4Error(f"{what} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise Kv4Error(f"{what} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if rows is not None and (t.dim() == 0 or t.shape[0] < rows):
        raise Kv4Error(f"{what} needs at least {rows} rows, got shape {tuple(t.shape)}")


def _step_args(B, q=None, k=None, v=None, pos=None, slot=None, ctx_len=None, page_table=None):
    """Checks of the per-sequence arguments of an append / decode call."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            _want(t, torch.bfloat16, name, rows=B, ndim=3)
            if t.shape[0] != B or t.shape[2] != HEAD_DIM:
                raise Kv4Error(f"{name} must be [B={B}][heads][{HEAD_DIM}], got {tuple(t.shape)}")
    for name, t in (("pos", pos), ("ctx_len", ctx_len)):
        if t is not None:
            _want(t, torch.int32, name, ndim=1)
            if t.shape[0] != B:
                raise Kv4Error(f"{name} must hold B={B} entries, got {t.shape[0]}")
    _want(slot, torch.int32, "slot", rows=B, ndim=1, optional=True)
    _want(page_table, torch.int32, "page_table", rows=B, ndim=2)


def _chunk_args(nseq, T=None, k=None, v=None, q=None, cu_seqlens=None, start_pos=None, slot=None,
                page_table=None):
    """Checks of the arguments of a re-prefill call over nseq sequences."""
    for name, t in (("k", k), ("v", v), ("q", q)):
        if t is not None:
            _want(t, torch.bfloat16, name, ndim=3)
            if T is not None and t.shape[0] != T:
                raise Kv4Error(f"{name} must hold {T} tokens, got {t.shape[0]}")
    _want(cu_seqlens, torch.int32, "cu_seqlens", rows=nseq + 1, ndim=1)
    _want(start_pos, torch.int32, "start_pos", rows=nseq, ndim=1)
    _want(slot, torch.int32, "slot", rows=nseq, ndim=1, optional=True)
    _want(page_table, torch.int32, "page_table", rows=nseq, ndim=2)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class Kv4Cache:
    """One layer's cache: paged INT4 pool + INT8 side buffer (device tensors).
    sink / window: the protection budget s, w (the library checks s % 16 == 0
    and s + w <= 144)."""

    def __init__(self, pages: torch.Tensor, side_codes: torch.Tensor, side_scales: torch.Tensor,
                 sink: int = SINK, window: int = WINDOW):
        self.pages, self.side_codes, self.side_scales = pages, side_codes, side_scales
        self.sink, self.window = int(sink), int(window)
        self.num_pages, self.num_kv_heads = int(pages.shape[0]), int(pages.shape[1])
        self.max_slots = int(side_codes.shape[0])
        assert pages.shape[2] == BLOCK_BYTES and pages.dtype == torch.uint8
        assert tuple(side_codes.shape[1:]) == (self.num_kv_heads, SIDE_ROWS, 2, HEAD_DIM)
        assert tuple(side_scales.shape[1:]) == (self.num_kv_heads, SIDE_ROWS, 2)
        self._desc = _Desc(ABI_VERSION, self.num_pages, PAGE, self.num_kv_heads, HEAD_DIM,
                           self.sink, self.window, self.max_slots, pages.data_ptr(), side_codes.data_ptr(),
                           side_scales.data_ptr())

    @classmethod
    def zeros(cls, num_pages: int, num_kv_heads: int, max_slots: int, device="cuda",
              sink: int = SINK, window: int = WINDOW):
        return cls(torch.zeros((num_pages, num_kv_heads, BLOCK_BYTES), dtype=torch.uint8, device=device),
                   torch.zeros((max_slots, num_kv_heads, SIDE_ROWS, 2, HEAD_DIM), dtype=torch.int8,
                               device=device),
                   torch.zeros((max_slots, num_kv_heads, SIDE_ROWS, 2), dtype=torch.int16,
                               device=device), sink, window)

    def desc(self):
        return C.byref(self._desc)


def append(cache: Kv4Cache, k, v, pos, slot, page_table):
    """kv4_append: k, v bf16 [B][Hkv][128]; pos, slot int32 [B]; page_table int32 [B][W]."""
    _step_args(int(pos.shape[0]), k=k, v=v, pos=pos, slot=slot, page_table=page_table)
    _check(lib().kv4_append(cache.desc(), _ptr(k), _ptr(v), _ptr(pos), _ptr(slot),
                            _ptr(page_table), page_table.shape[1], pos.shape[0], _stream()))


def prefill_quantize(cache: Kv4Cache, k, v, cu_seqlens, start_pos, slot, page_table,
                     max_seqlen: int):
    """kv4_prefill_quantize: k, v bf16 [T][Hkv][128]; cu_seqlens int32 [nseq+1]."""
    _chunk_args(int(start_pos.shape[0]), k=k, v=v, cu_seqlens=cu_seqlens, start_pos=start_pos, slot=slot,
                page_table=page_table)
    _check(lib().kv4_prefill_quantize(cache.desc(), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                      _ptr(start_pos), _ptr(slot), _ptr(page_table),
                                      page_table.shape[1], start_pos.shape[0], int(max_seqlen),
                                      _stream()))


def decode_workspace_bytes(cache: Kv4Cache, B: int, Hq: int, max_ctx: int) -> int:
    return int(lib().kv4_decode_workspace_bytes(cache.desc(), B, Hq, max_ctx))


def decode_attention(cache: Kv4Cache, q, ctx_len, slot, page_table, max_ctx: int,
                     softmax_scale: float, out=None, lse=None, workspace=None):
    """kv4_decode_attention: q bf16 [B][Hq][128] -> (out fp32 [B][Hq][128], lse fp32 [B][Hq])."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, slot=slot, ctx_len=ctx_len, page_table=page_table)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(cache, B, Hq, max_ctx), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv4_decode_attention(cache.desc(), _ptr(q), _ptr(ctx_len), _ptr(slot),
                                      _ptr(page_table), page_table.shape[1], B, Hq, int(max_ctx),
                                      float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                      workspace.numel(), _stream()))
    return out, lse


def decode_attention_debug(cache: Kv4Cache, q, ctx_len, slot, page_table, max_ctx: int,
                           softmax_scale: float):
    """kv4_decode_attention_debug: also returns the integer intermediates
    (qcodes, qsum, qk, pcode, pv) as device tensors."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, slot=slot, ctx_len=ctx_len, page_table=page_table)
    W = int(page_table.shape[1])
    dev = q.device
    dbg = dict(qcodes=torch.zeros((B, Hq, HEAD_DIM), dtype=torch.int8, device=dev),
               qsum=torch.zeros((B, Hq), dtype=torch.int32, device=dev),
               qk=torch.zeros((B, Hq, W * PAGE), dtype=torch.int32, device=dev),
               pcode=torch.zeros((B, Hq, W * PAGE), dtype=torch.uint8, device=dev),
               pv=torch.zeros((B, Hq, W, HEAD_DIM), dtype=torch.int32, device=dev))
    d = _Debug(dbg["qcodes"].data_ptr(), dbg["qsum"].data_ptr(), dbg["qk"].data_ptr(),
               dbg["pcode"].data_ptr(), dbg["pv"].data_ptr(), W * PAGE, W)
    out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(decode_workspace_bytes(cache, B, Hq, max_ctx), dtype=torch.uint8, device=dev)
    _check(lib().kv4_decode_attention_debug(cache.desc(), _ptr(q), _ptr(ctx_len), _ptr(slot),
                                            _ptr(page_table), W, B, Hq, int(max_ctx),
                                            float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                            ws.numel(), C.byref(d), _stream()))
    return out, lse, dbg


def bf16_workspace_bytes(B: int, Hq: int, Hkv: int, max_ctx: int) -> int:
    return int(lib().kv4bench_bf16_workspace_bytes(B, Hq, Hkv, max_ctx))


def bf16_paged_decode(pages, q, ctx_len, page_table, max_ctx: int, softmax_scale: float,
                      out=None, lse=None, workspace=None):
    """kv4bench_bf16_paged_decode (comparator): pages bf16 [P][Hkv][2][16][128]
    with K token-major and V channel-major."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _want(pages, torch.bfloat16, "pages", ndim=5)
    _step_args(B, q=q, ctx_len=ctx_len, page_table=page_table)
    Hkv = int(pages.shape[1])
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(bf16_workspace_bytes(B, Hq, Hkv, max_ctx), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv4bench_bf16_paged_decode(_ptr(pages), int(pages.shape[0]), Hkv, _ptr(q),
                                            _ptr(ctx_len), _ptr(page_table), page_table.shape[1],
                                            B, Hq, int(max_ctx), float(softmax_scale), _ptr(out),
                                            _ptr(lse), _ptr(workspace), workspace.numel(),
                                            _stream()))
    return out, lse


def decode_attention_timed(cache: Kv4Cache, q, ctx_len, slot, page_table, max_ctx: int,
                           softmax_scale: float, out, lse, workspace, ev_begin, ev_end,
                           k=None, v=None, pos=None):
    """kv4bench_decode_attention_timed: as decode_attention (or, with k, v, pos,
    append_decode_attention), recording the two raw hipEvent_t handles
    (ctypes.c_void_p) around the main kernel."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, k=k, v=v, pos=pos, slot=slot, ctx_len=ctx_len, page_table=page_table)
    _check(lib().kv4bench_decode_attention_timed(
        cache.desc(), _ptr(k), _ptr(v), _ptr(pos), _ptr(q), _ptr(ctx_len), _ptr(slot),
        _ptr(page_table), page_table.shape[1], B, Hq, int(max_ctx), float(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), ev_begin, ev_end, _stream()))


def append_decode_attention(cache: Kv4Cache, k, v, pos, q, ctx_len, slot, page_table, max_ctx: int,
                            softmax_scale: float, out=None, lse=None, workspace=None):
    """kv4_append_decode_attention: append(k, v, pos) then decode_attention in one launch
    (pos = ctx_len - 1)."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, k=k, v=v, pos=pos, slot=slot, ctx_len=ctx_len, page_table=page_table)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(cache, B, Hq, max_ctx), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv4_append_decode_attention(
        cache.desc(), _ptr(k), _ptr(v), _ptr(pos), _ptr(q), _ptr(ctx_len), _ptr(slot),
        _ptr(page_table), page_table.shape[1], B, Hq, int(max_ctx), float(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse


def append_decode_attention_noalloc(cache: Kv4Cache, k, v, pos, q, ctx_len, slot, page_table,
                                    max_ctx: int, softmax_scale: float, out, lse):
    """kv4_append_decode_attention_noalloc: append_decode_attention with the
    workspace in the library's fixed per-device scratch; out fp32 [B][Hq][128]
    and lse fp32 [B][Hq] are the caller's (nothing is allocated here)."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, k=k, v=v, pos=pos, slot=slot, ctx_len=ctx_len, page_table=page_table)
    _want(out, torch.float32, "out", rows=B)
    _want(lse, torch.float32, "lse", rows=B)
    _check(lib().kv4_append_decode_attention_noalloc(
        cache.desc(), _ptr(k), _ptr(v), _ptr(pos), _ptr(q), _ptr(ctx_len), _ptr(slot),
        _ptr(page_table), page_table.shape[1], B, Hq, int(max_ctx), float(softmax_scale), _ptr(out),
        _ptr(lse), _stream()))
    return out, lse


# ------------------------------------------------------------ KV8 variant --

class Kv8Cache:
    """KV8-everywhere pool (the INT8 comparison variant): pages uint8
    [num_pages][Hkv][4160] = K codes [16][128] (rotated) | V codes [128][16] |
    s_k FP16 [16] | s_v FP16 [16]."""

    def __init__(self, pages: torch.Tensor):
        assert pages.dtype == torch.uint8 and pages.dim() == 3 and pages.shape[2] == KV8_BLOCK_BYTES
        self.pages = pages
        self.num_pages, self.num_kv_heads = int(pages.shape[0]), int(pages.shape[1])
        self._desc = _Kv8Desc(ABI_VERSION, self.num_pages, PAGE, self.num_kv_heads, HEAD_DIM,
                              pages.data_ptr())

    @classmethod
    def zeros(cls, num_pages: int, num_kv_heads: int, device="cuda"):
        return cls(torch.zeros((num_pages, num_kv_heads, KV8_BLOCK_BYTES), dtype=torch.uint8,
                               device=device))

    def desc(self):
        return C.byref(self._desc)


def kv8_append(cache: Kv8Cache, k, v, pos, page_table):
    """kv8_append: k, v bf16 [B][Hkv][128]; pos int32 [B]; page_table int32 [B][W]."""
    _step_args(int(pos.shape[0]), k=k, v=v, pos=pos, page_table=page_table)
    _check(lib().kv8_append(cache.desc(), _ptr(k), _ptr(v), _ptr(pos), _ptr(page_table),
                            page_table.shape[1], pos.shape[0], _stream()))


def kv8_prefill_quantize(cache: Kv8Cache, k, v, cu_seqlens, start_pos, page_table, max_seqlen: int):
    """kv8_prefill_quantize: k, v bf16 [T][Hkv][128]; cu_seqlens int32 [nseq+1]."""
    _chunk_args(int(start_pos.shape[0]), k=k, v=v, cu_seqlens=cu_seqlens, start_pos=start_pos,
                page_table=page_table)
    _check(lib().kv8_prefill_quantize(cache.desc(), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                      _ptr(start_pos), _ptr(page_table), page_table.shape[1],
                                      start_pos.shape[0], int(max_seqlen), _stream()))


def kv8_decode_workspace_bytes(cache: Kv8Cache, B: int, Hq: int, max_ctx: int) -> int:
    return int(lib().kv8_decode_workspace_bytes(cache.desc(), B, Hq, max_ctx))


def kv8_decode_attention(cache: Kv8Cache, q, ctx_len, page_table, max_ctx: int,
                         softmax_scale: float, out=None, lse=None, workspace=None):
    """kv8_decode_attention: q bf16 [B][Hq][128] -> (out fp32 [B][Hq][128], lse fp32 [B][Hq])."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, ctx_len=ctx_len, page_table=page_table)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(kv8_decode_workspace_bytes(cache, B, Hq, max_ctx), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv8_decode_attention(cache.desc(), _ptr(q), _ptr(ctx_len), _ptr(page_table),
                                      page_table.shape[1], B, Hq, int(max_ctx), float(softmax_scale),
                                      _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                      _stream()))
    return out, lse


def kv8_decode_attention_debug(cache: Kv8Cache, q, ctx_len, page_table, max_ctx: int,
                               softmax_scale: float):
    """kv8_decode_attention_debug: also returns qcodes, qsum and qk as device tensors."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, ctx_len=ctx_len, page_table=page_table)
    W = int(page_table.shape[1])
    dev = q.device
    dbg = dict(qcodes=torch.zeros((B, Hq, HEAD_DIM), dtype=torch.int8, device=dev),
               qsum=torch.zeros((B, Hq), dtype=torch.int32, device=dev),
               qk=torch.zeros((B, Hq, W * PAGE), dtype=torch.int32, device=dev))
    d = _Debug(dbg["qcodes"].data_ptr(), dbg["qsum"].data_ptr(), dbg["qk"].data_ptr(), None, None,
               W * PAGE, W)
    out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(kv8_decode_workspace_bytes(cache, B, Hq, max_ctx), dtype=torch.uint8, device=dev)
    _check(lib().kv8_decode_attention_debug(cache.desc(), _ptr(q), _ptr(ctx_len), _ptr(page_table),
                                            W, B, Hq, int(max_ctx), float(softmax_scale), _ptr(out),
                                            _ptr(lse), _ptr(ws), ws.numel(), C.byref(d), _stream()))
    return out, lse, dbg


# ---------------------------------------------------------- MXFP4 variant --
# The same Kv4Cache (descriptor, side buffer, budget); the page blocks hold the
# main region in OCP MXFP4.  A cache is written and read by one variant.

def mx_append(cache: Kv4Cache, k, v, pos, slot, page_table):
    """kv4mx_append: as append, main-region entry in MXFP4."""
    _step_args(int(pos.shape[0]), k=k, v=v, pos=pos, slot=slot, page_table=page_table)
    _check(lib().kv4mx_append(cache.desc(), _ptr(k), _ptr(v), _ptr(pos), _ptr(slot),
                              _ptr(page_table), page_table.shape[1], pos.shape[0], _stream()))


def mx_prefill_quantize(cache: Kv4Cache, k, v, cu_seqlens, start_pos, slot, page_table,
                        max_seqlen: int):
    _chunk_args(int(start_pos.shape[0]), k=k, v=v, cu_seqlens=cu_seqlens, start_pos=start_pos, slot=slot,
                page_table=page_table)
    _check(lib().kv4mx_prefill_quantize(cache.desc(), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                        _ptr(start_pos), _ptr(slot), _ptr(page_table),
                                        page_table.shape[1], start_pos.shape[0], int(max_seqlen),
                                        _stream()))


def mx_decode_attention(cache: Kv4Cache, q, ctx_len, slot, page_table, max_ctx: int,
                        softmax_scale: float, out=None, lse=None, workspace=None):
    """kv4mx_decode_attention: q bf16 [B][Hq][128] -> (out fp32 [B][Hq][128], lse fp32 [B][Hq])."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _step_args(B, q=q, slot=slot, ctx_len=ctx_len, page_table=page_table)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(cache, B, Hq, max_ctx), dtype=torch.uint8,
                                device=q.device)
    _check(lib().kv4mx_decode_attention(cache.desc(), _ptr(q), _ptr(ctx_len), _ptr(slot),
                                        _ptr(page_table), page_table.shape[1], B, Hq, int(max_ctx),
                                        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                        workspace.numel(), _stream()))
    return out, lse


# ------------------------------------------------- re-prefill attention --

def prefill_attention_workspace_bytes(cache: Kv4Cache, total_q: int, Hq: int, max_ctx: int) -> int:
    return int(lib().kv4_prefill_attention_workspace_bytes(cache.desc(), total_q, Hq, max_ctx))


def prefill_attention(cache: Kv4Cache, q, cu_seqlens, start_pos, slot, page_table, max_ctx: int,
                      softmax_scale: float, out=None, lse=None, workspace=None):
    """kv4_prefill_attention: q bf16 [T][Hq][128] of the chunks (cu_seqlens, start_pos as for
    prefill_quantize) -> (out fp32 [T][Hq][128], lse fp32 [T][Hq])."""
    T, Hq = int(q.shape[0]), int(q.shape[1])
    _chunk_args(int(start_pos.shape[0]), T=T, q=q, cu_seqlens=cu_seqlens, start_pos=start_pos, slot=slot,
                page_table=page_table)
    if out is None:
        out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(prefill_attention_workspace_bytes(cache, T, Hq, max_ctx),
                                dtype=torch.uint8, device=q.device)
    _check(lib().kv4_prefill_attention(cache.desc(), _ptr(q), _ptr(cu_seqlens), _ptr(start_pos),
                                       _ptr(slot), _ptr(page_table), page_table.shape[1],
                                       start_pos.shape[0], T, Hq, int(max_ctx), float(softmax_scale),
                                       _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                       _stream()))
    return out, lse


def prefill_attention_debug(cache: Kv4Cache, q, cu_seqlens, start_pos, slot, page_table,
                            max_ctx: int, softmax_scale: float):
    """kv4_prefill_attention_debug: also the integer intermediates, indexed by token."""
    T, Hq = int(q.shape[0]), int(q.shape[1])
    _chunk_args(int(start_pos.shape[0]), T=T, q=q, cu_seqlens=cu_seqlens, start_pos=start_pos, slot=slot,
                page_table=page_table)
    W = int(page_table.shape[1])
    dev = q.device
    dbg = dict(qcodes=torch.zeros((T, Hq, HEAD_DIM), dtype=torch.int8, device=dev),
               qsum=torch.zeros((T, Hq), dtype=torch.int32, device=dev),
               qk=torch.zeros((T, Hq, W * PAGE), dtype=torch.int32, device=dev),
               pcode=torch.zeros((T, Hq, W * PAGE), dtype=torch.uint8, device=dev),
               pv=torch.zeros((T, Hq, W, HEAD_DIM), dtype=torch.int32, device=dev))
    d = _Debug(dbg["qcodes"].data_ptr(), dbg["qsum"].data_ptr(), dbg["qk"].data_ptr(),
               dbg["pcode"].data_ptr(), dbg["pv"].data_ptr(), W * PAGE, W)
    out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(prefill_attention_workspace_bytes(cache, T, Hq, max_ctx), dtype=torch.uint8,
                     device=dev)
    _check(lib().kv4_prefill_attention_debug(cache.desc(), _ptr(q), _ptr(cu_seqlens), _ptr(start_pos),
                                             _ptr(slot), _ptr(page_table), W, start_pos.shape[0], T, Hq,
                                             int(max_ctx), float(softmax_scale), _ptr(out), _ptr(lse),
                                             _ptr(ws), ws.numel(), C.byref(d), _stream()))
    return out, lse, dbg
