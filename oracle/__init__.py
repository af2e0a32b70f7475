"""CPU oracle for the KV4-RL hybrid decode-attention path.

TEST INFRASTRUCTURE ONLY: a plain, slow statement of what the path computes,
used to check the HIP library.  Only tests/, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the library (the C source is oracle/kv4_oracle.c; the
FP64 / exact-rational brute force for tiny inputs is oracle/brute.py).

Every function here takes and returns numpy arrays; BF16 and FP16 values are
uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

HD, PAGE, SINK, WINDOW, SIDE_ROWS, BLOCK = 128, 16, 16, 128, 144, 2176

_lib = None


class _Cache(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("num_kv_heads", C.c_int32), ("max_slots", C.c_int32),
                ("pages", C.c_void_p), ("side_codes", C.c_void_p), ("side_scales", C.c_void_p),
                ("sink", C.c_int32), ("window", C.c_int32)]


class _Kv8Cache(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("num_kv_heads", C.c_int32), ("pages", C.c_void_p)]


class _Debug(C.Structure):
    _fields_ = [("qcodes", C.c_void_p), ("qsum", C.c_void_p), ("qk", C.c_void_p),
                ("pcode", C.c_void_p), ("pv", C.c_void_p), ("max_ctx", C.c_int32),
                ("max_pages", C.c_int32)]


def lib():
    global _lib
    if _lib is None:
        # KV4_ORACLE_LIB: another build of the same source (the sanitized one)
        path = os.environ.get("KV4_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        _lib = C.CDLL(path)
        _lib.kv4ref_f32_to_f16.restype = C.c_uint16
        _lib.kv4ref_f32_to_f16.argtypes = [C.c_float]
        _lib.kv4ref_f16_to_f32.restype = C.c_float
        _lib.kv4ref_f16_to_f32.argtypes = [C.c_uint16]
        _lib.kv4ref_exp2s.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        _lib.kv4ref_scale_log2.restype = C.c_float
        _lib.kv4ref_scale_log2.argtypes = [C.c_float]
        for name in ("kv4ref_convert_f16", "kv4ref_convert_bf16"):
            getattr(_lib, name).argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        _lib.kv4ref_fwht128.argtypes = [C.c_void_p, C.c_int64]
        _lib.kv4ref_quant_int4.argtypes = [C.c_void_p] * 4 + [C.c_int64]
        _lib.kv4ref_quant_int8.argtypes = [C.c_void_p] * 3 + [C.c_int64]
        _lib.kv4ref_quant_query.argtypes = [C.c_void_p] * 4 + [C.c_int64]
        _lib.kv4ref_exp2s_coeffs.argtypes = [C.c_void_p]
        _lib.kv4ref_append.argtypes = [C.POINTER(_Cache)] + [C.c_void_p] * 5 + [C.c_int32] * 2
        KC = C.POINTER(_Cache)
        _lib.kv4ref_prefill_attention.argtypes = ([KC] + [C.c_void_p] * 5 + [C.c_int32] * 3
                                                  + [C.c_float, C.c_int32, C.c_void_p, C.c_void_p,
                                                     C.POINTER(_Debug), C.c_int32])
        _lib.kv4ref_prefill_attention_sampled.argtypes = ([KC] + [C.c_void_p] * 5 + [C.c_int32] * 3
                                                          + [C.c_float, C.c_int32, C.c_void_p, C.c_void_p,
                                                             C.c_void_p, C.c_int32])
        _lib.mxref_append.argtypes = [KC] + [C.c_void_p] * 5 + [C.c_int32] * 2
        _lib.mxref_prefill.argtypes = [KC] + [C.c_void_p] * 6 + [C.c_int32] * 3
        _lib.mxref_decode.argtypes = ([KC] + [C.c_void_p] * 4 + [C.c_int32] * 3 + [C.c_float]
                                      + [C.c_void_p] * 2 + [C.c_int32])
        K8 = C.POINTER(_Kv8Cache)
        _lib.kv8ref_append.argtypes = [K8] + [C.c_void_p] * 4 + [C.c_int32] * 2
        _lib.kv8ref_prefill.argtypes = [K8] + [C.c_void_p] * 5 + [C.c_int32] * 3
        _lib.kv8ref_decode.argtypes = ([K8] + [C.c_void_p] * 3 + [C.c_int32] * 3 + [C.c_float]
                                       + [C.c_void_p] * 2 + [C.POINTER(_Debug), C.c_int32])
        _lib.kv4ref_prefill.argtypes = ([C.POINTER(_Cache)] + [C.c_void_p] * 6
                                        + [C.c_int32] * 3)
        _lib.kv4ref_decode.argtypes = ([C.POINTER(_Cache)] + [C.c_void_p] * 4
                                       + [C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_int32,
                                          C.c_void_p, C.c_void_p, C.POINTER(_Debug), C.c_int32])
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


# ---------------------------------------------------------------- scalars --

def f32_to_f16(x) -> np.ndarray:
    x = _c(x, np.float32)
    h = np.empty(x.shape, np.uint16)
    lib().kv4ref_convert_f16(_p(x), _p(h), x.size)
    return h


def f32_to_bf16(x) -> np.ndarray:
    x = _c(x, np.float32)
    h = np.empty(x.shape, np.uint16)
    lib().kv4ref_convert_bf16(_p(x), _p(h), x.size)
    return h


def f16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    return np.array([lib().kv4ref_f16_to_f32(int(v)) for v in h.ravel()],
                    dtype=np.float32).reshape(h.shape)


def bf16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def fwht(x) -> np.ndarray:
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    assert x.shape[-1] == HD
    lib().kv4ref_fwht128(_p(x), x.size // HD)
    return x


def quant_int4(x):
    x = _c(x, np.float32)
    n = x.size // HD
    codes = np.empty(x.shape, np.uint8)
    d = np.empty(x.shape[:-1], np.uint16)
    m = np.empty(x.shape[:-1], np.uint16)
    lib().kv4ref_quant_int4(_p(x), _p(codes), _p(d), _p(m), n)
    return codes, d, m


def quant_int8(x):
    x = _c(x, np.float32)
    codes = np.empty(x.shape, np.int8)
    s = np.empty(x.shape[:-1], np.uint16)
    lib().kv4ref_quant_int8(_p(x), _p(codes), _p(s), x.size // HD)
    return codes, s


def quant_query(x):
    x = _c(x, np.float32)
    codes = np.empty(x.shape, np.int8)
    s = np.empty(x.shape[:-1], np.float32)
    sm = np.empty(x.shape[:-1], np.int32)
    lib().kv4ref_quant_query(_p(x), _p(codes), _p(s), _p(sm), x.size // HD)
    return codes, s, sm


def exp2s(y) -> np.ndarray:
    y = _c(y, np.float32)
    e = np.empty(y.shape, np.float32)
    lib().kv4ref_exp2s(_p(y), _p(e), y.size)
    return e


def exp2s_coeffs() -> np.ndarray:
    c = np.empty(8, np.float32)
    lib().kv4ref_exp2s_coeffs(_p(c))
    return c


def scale_log2(softmax_scale: float) -> np.float32:
    return np.float32(lib().kv4ref_scale_log2(softmax_scale))


# ------------------------------------------------------------------ cache --

class Cache:
    """One layer's cache in host memory (oracle side); sink / window are the
    protection budget s, w (16 / 128 by default; s a multiple of 16,
    s + w <= 144)."""

    def __init__(self, num_pages: int, Hkv: int, max_slots: int, sink: int = SINK,
                 window: int = WINDOW):
        self.pages = np.zeros((num_pages, Hkv, BLOCK), np.uint8)
        self.side_codes = np.zeros((max_slots, Hkv, SIDE_ROWS, 2, HD), np.int8)
        self.side_scales = np.zeros((max_slots, Hkv, SIDE_ROWS, 2), np.uint16)
        self.num_pages, self.Hkv, self.max_slots = num_pages, Hkv, max_slots
        if sink < 0 or window < 0 or sink % PAGE or sink + window > SIDE_ROWS:
            raise ValueError(f"protection budget s={sink}, w={window}: need s % {PAGE} == 0 "
                             f"and s + w <= {SIDE_ROWS}")
        self.sink, self.window = sink, window

    def _struct(self):
        return _Cache(self.num_pages, self.Hkv, self.max_slots, _p(self.pages).value,
                      _p(self.side_codes).value, _p(self.side_scales).value, self.sink,
                      self.window)

    def copy(self) -> "Cache":
        c = Cache.__new__(Cache)
        c.pages, c.side_codes, c.side_scales = (self.pages.copy(), self.side_codes.copy(),
                                                self.side_scales.copy())
        c.num_pages, c.Hkv, c.max_slots = self.num_pages, self.Hkv, self.max_slots
        c.sink, c.window = self.sink, self.window
        return c


def append(cache: Cache, k, v, pos, slot, page_table):
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    pos, table = _c(pos, np.int32), _c(page_table, np.int32)
    slot = None if slot is None else _c(slot, np.int32)
    B = pos.shape[0]
    assert k.shape == (B, cache.Hkv, HD) and v.shape == k.shape
    st = cache._struct()
    rc = lib().kv4ref_append(C.byref(st), _p(k), _p(v), _p(pos),
                             None if slot is None else _p(slot), _p(table), table.shape[1], B)
    if rc != 0:
        raise ValueError(f"kv4ref_append failed ({rc}): invalid protection budget")


def prefill(cache: Cache, k, v, cu_seqlens, start_pos, slot, page_table, nthreads=None):
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    cu, start, table = (_c(cu_seqlens, np.int32), _c(start_pos, np.int32),
                        _c(page_table, np.int32))
    slot = None if slot is None else _c(slot, np.int32)
    nseq = start.shape[0]
    assert k.shape == (int(cu[-1]), cache.Hkv, HD)
    st = cache._struct()
    rc = lib().kv4ref_prefill(C.byref(st), _p(k), _p(v), _p(cu), _p(start),
                              None if slot is None else _p(slot), _p(table), table.shape[1],
                              nseq, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kv4ref_prefill failed ({rc}): invalid protection budget")


def decode(cache: Cache, q, ctx_len, slot, page_table, Hq: int, softmax_scale: float,
           pv_exact: bool = False, debug: bool = False, nthreads=None):
    """Returns (out [B][Hq][128] f64, lse [B][Hq] f64, dbg dict or None)."""
    q = _c(q, np.uint16)
    ctx, table = _c(ctx_len, np.int32), _c(page_table, np.int32)
    slot = None if slot is None else _c(slot, np.int32)
    B = ctx.shape[0]
    assert q.shape == (B, Hq, HD)
    out = np.zeros((B, Hq, HD), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    dbg = None
    dstruct = None
    if debug:
        max_ctx = int(table.shape[1]) * PAGE
        dbg = dict(qcodes=np.zeros((B, Hq, HD), np.int8), qsum=np.zeros((B, Hq), np.int32),
                   qk=np.zeros((B, Hq, max_ctx), np.int32),
                   pcode=np.zeros((B, Hq, max_ctx), np.uint8),
                   pv=np.zeros((B, Hq, table.shape[1], HD), np.int32))
        dstruct = _Debug(_p(dbg["qcodes"]).value, _p(dbg["qsum"]).value, _p(dbg["qk"]).value,
                         _p(dbg["pcode"]).value, _p(dbg["pv"]).value, max_ctx, table.shape[1])
    st = cache._struct()
    rc = lib().kv4ref_decode(C.byref(st), _p(q), _p(ctx), None if slot is None else _p(slot),
                             _p(table), table.shape[1], B, Hq, softmax_scale, int(pv_exact),
                             _p(out), _p(lse), C.byref(dstruct) if dstruct else None,
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kv4ref_decode failed ({rc}): invalid head counts or protection budget")
    return out, lse, dbg


# ------------------------------------------------------------ KV8 variant --

KV8_BLOCK, KV8_OFF_V, KV8_OFF_SK, KV8_OFF_SV = 4160, 2048, 4096, 4128


class Kv8Cache:
    """KV8-everywhere pool (the INT8 comparison variant) in host memory:
    [num_pages][Hkv][4160] = K codes int8 [16][128] (rotated keys) | V codes
    int8 [128][16] | s_k FP16 [16] | s_v FP16 [16]."""

    def __init__(self, num_pages: int, Hkv: int):
        self.pages = np.zeros((num_pages, Hkv, KV8_BLOCK), np.uint8)
        self.num_pages, self.Hkv = num_pages, Hkv

    def _struct(self):
        return _Kv8Cache(self.num_pages, self.Hkv, _p(self.pages).value)


def kv8_append(cache: Kv8Cache, k, v, pos, page_table):
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    pos, table = _c(pos, np.int32), _c(page_table, np.int32)
    B = pos.shape[0]
    assert k.shape == (B, cache.Hkv, HD) and v.shape == k.shape
    st = cache._struct()
    rc = lib().kv8ref_append(C.byref(st), _p(k), _p(v), _p(pos), _p(table), table.shape[1], B)
    if rc != 0:
        raise ValueError(f"kv8ref_append failed ({rc})")


def kv8_prefill(cache: Kv8Cache, k, v, cu_seqlens, start_pos, page_table, nthreads=None):
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    cu, start, table = (_c(cu_seqlens, np.int32), _c(start_pos, np.int32),
                        _c(page_table, np.int32))
    assert k.shape == (int(cu[-1]), cache.Hkv, HD)
    st = cache._struct()
    rc = lib().kv8ref_prefill(C.byref(st), _p(k), _p(v), _p(cu), _p(start), _p(table),
                              table.shape[1], start.shape[0], nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kv8ref_prefill failed ({rc})")


def kv8_decode(cache: Kv8Cache, q, ctx_len, page_table, Hq: int, softmax_scale: float,
               debug: bool = False, nthreads=None):
    """Every position through the protected path's arithmetic.  Returns
    (out [B][Hq][128] f64, lse [B][Hq] f64, dbg dict with qcodes, qsum, qk or None)."""
    q = _c(q, np.uint16)
    ctx, table = _c(ctx_len, np.int32), _c(page_table, np.int32)
    B = ctx.shape[0]
    assert q.shape == (B, Hq, HD)
    out = np.zeros((B, Hq, HD), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    dbg = dstruct = None
    if debug:
        max_ctx = int(table.shape[1]) * PAGE
        dbg = dict(qcodes=np.zeros((B, Hq, HD), np.int8), qsum=np.zeros((B, Hq), np.int32),
                   qk=np.zeros((B, Hq, max_ctx), np.int32))
        dstruct = _Debug(_p(dbg["qcodes"]).value, _p(dbg["qsum"]).value, _p(dbg["qk"]).value,
                         None, None, max_ctx, table.shape[1])
    st = cache._struct()
    rc = lib().kv8ref_decode(C.byref(st), _p(q), _p(ctx), _p(table), table.shape[1], B, Hq,
                             softmax_scale, _p(out), _p(lse), C.byref(dstruct) if dstruct else None,
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kv8ref_decode failed ({rc})")
    return out, lse, dbg


# ---------------------------------------------------------- MXFP4 variant --

MX_OFF_V, MX_OFF_KS, MX_OFF_VS = 1024, 2048, 2112


def mx_append(cache: Cache, k, v, pos, slot, page_table):
    """The MXFP4 variant's append: main-region block in OCP MXFP4, side rows as kv4 append."""
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    pos, table = _c(pos, np.int32), _c(page_table, np.int32)
    slot = None if slot is None else _c(slot, np.int32)
    B = pos.shape[0]
    assert k.shape == (B, cache.Hkv, HD) and v.shape == k.shape
    st = cache._struct()
    rc = lib().mxref_append(C.byref(st), _p(k), _p(v), _p(pos), None if slot is None else _p(slot),
                            _p(table), table.shape[1], B)
    if rc != 0:
        raise ValueError(f"mxref_append failed ({rc}): invalid protection budget")


def mx_prefill(cache: Cache, k, v, cu_seqlens, start_pos, slot, page_table, nthreads=None):
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    cu, start, table = (_c(cu_seqlens, np.int32), _c(start_pos, np.int32), _c(page_table, np.int32))
    slot = None if slot is None else _c(slot, np.int32)
    assert k.shape == (int(cu[-1]), cache.Hkv, HD)
    st = cache._struct()
    rc = lib().mxref_prefill(C.byref(st), _p(k), _p(v), _p(cu), _p(start),
                             None if slot is None else _p(slot), _p(table), table.shape[1],
                             start.shape[0], nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"mxref_prefill failed ({rc}): invalid protection budget")


def mx_decode(cache: Cache, q, ctx_len, slot, page_table, Hq: int, softmax_scale: float,
              nthreads=None):
    """Returns (out [B][Hq][128] f64, lse [B][Hq] f64) of the MXFP4 variant."""
    q = _c(q, np.uint16)
    ctx, table = _c(ctx_len, np.int32), _c(page_table, np.int32)
    slot = None if slot is None else _c(slot, np.int32)
    B = ctx.shape[0]
    assert q.shape == (B, Hq, HD)
    out = np.zeros((B, Hq, HD), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    st = cache._struct()
    rc = lib().mxref_decode(C.byref(st), _p(q), _p(ctx), None if slot is None else _p(slot),
                            _p(table), table.shape[1], B, Hq, softmax_scale, _p(out), _p(lse),
                            nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"mxref_decode failed ({rc})")
    return out, lse


# ------------------------------------------------- re-prefill attention --

def prefill_attention(cache: Cache, q, cu_seqlens, start_pos, slot, page_table, Hq: int,
                      softmax_scale: float, pv_exact: bool = False, debug: bool = False,
                      nthreads=None):
    """Chunk attention after the chunk's K/V were written: token i of sequence s
    attends [0, start[s] + i] with the protected set of the cache ending at
    start[s] + n_s.  q [T][Hq][128]; returns (out [T][Hq][128], lse [T][Hq], dbg)."""
    q = _c(q, np.uint16)
    cu, start, table = (_c(cu_seqlens, np.int32), _c(start_pos, np.int32), _c(page_table, np.int32))
    slot = None if slot is None else _c(slot, np.int32)
    T = int(cu[-1])
    assert q.shape == (T, Hq, HD)
    out = np.zeros((T, Hq, HD), np.float64)
    lse = np.zeros((T, Hq), np.float64)
    dbg = dstruct = None
    if debug:
        max_ctx = int(table.shape[1]) * PAGE
        dbg = dict(qcodes=np.zeros((T, Hq, HD), np.int8), qsum=np.zeros((T, Hq), np.int32),
                   qk=np.zeros((T, Hq, max_ctx), np.int32), pcode=np.zeros((T, Hq, max_ctx), np.uint8),
                   pv=np.zeros((T, Hq, table.shape[1], HD), np.int32))
        dstruct = _Debug(_p(dbg["qcodes"]).value, _p(dbg["qsum"]).value, _p(dbg["qk"]).value,
                         _p(dbg["pcode"]).value, _p(dbg["pv"]).value, max_ctx, table.shape[1])
    st = cache._struct()
    rc = lib().kv4ref_prefill_attention(C.byref(st), _p(q), _p(cu), _p(start),
                                        None if slot is None else _p(slot), _p(table), table.shape[1],
                                        start.shape[0], Hq, softmax_scale, int(pv_exact), _p(out),
                                        _p(lse), C.byref(dstruct) if dstruct else None,
                                        nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kv4ref_prefill_attention failed ({rc})")
    return out, lse, dbg


def prefill_attention_sampled(cache: Cache, q, cu_seqlens, start_pos, slot, page_table, Hq: int,
                              softmax_scale: float, tokens, heads, nthreads=None):
    """prefill_attention for the listed (token, q-head) pairs only; returns
    out [n][128], lse [n] (FP64)."""
    q = _c(q, np.uint16)
    cu, start, table = (_c(cu_seqlens, np.int32), _c(start_pos, np.int32), _c(page_table, np.int32))
    slot = None if slot is None else _c(slot, np.int32)
    th = _c(np.asarray(tokens, np.int64) * Hq + np.asarray(heads, np.int64), np.int64)
    n = th.shape[0]
    assert q.shape == (int(cu[-1]), Hq, HD)
    out = np.zeros((n, HD), np.float64)
    lse = np.zeros(n, np.float64)
    st = cache._struct()
    rc = lib().kv4ref_prefill_attention_sampled(C.byref(st), _p(q), _p(cu), _p(start),
                                                None if slot is None else _p(slot), _p(table),
                                                table.shape[1], start.shape[0], Hq, softmax_scale, n, _p(th),
                                                _p(out), _p(lse), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"kv4ref_prefill_attention_sampled failed ({rc})")
    return out, lse
