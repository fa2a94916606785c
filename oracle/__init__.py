"""CPU oracle (test infrastructure only).

Thin ctypes wrapper over ``tq_oracle.c``: plain, slow, obviously correct
reimplementations of the quantized paged-KV decode path, written from the
pages (triton_turboquant_decode.py, int4_per_token_head.py,
kpool_compress.py). Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.

The shared object is compiled from source with gcc on first use (or by
``build()``); nothing here touches a GPU.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtq_oracle.so")
_lock = threading.Lock()
_lib = None

# Format codes of the combined TurboQuant slot (oracle-side numbering).
KEY_FP8, KEY_MSE3, KEY_MSE4 = 1, 2, 3
VAL_U3, VAL_U4, VAL_FP8 = 1, 2, 3
DT_F32, DT_F16, DT_BF16 = 0, 1, 2


# Compiler flags of the oracle: no contraction, so each fp32 operation in
# the source rounds exactly once as written.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fPIC", "-shared"]


def compile_source(src: str, out: str, extra=()) -> str:
    """Compile one oracle source file into a shared object at `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile tq_oracle.c into libtq_oracle.so with gcc (no contraction)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _p(a, ctype):
    return None if a is None else a.ctypes.data_as(C.POINTER(ctype))


def _load(path):
    """Load an oracle shared object and declare its signatures."""
    L = C.CDLL(path)
    i32, i64, f32, f64, u8, u16 = (C.c_int32, C.c_int64, C.c_float,
                                   C.c_double, C.c_uint8, C.c_uint16)
    P = C.POINTER
    L.orc_f32_to_bf16.restype = u16; L.orc_f32_to_bf16.argtypes = [f32]
    L.orc_bf16_to_f32.restype = f32; L.orc_bf16_to_f32.argtypes = [u16]
    L.orc_f32_to_f16.restype = u16; L.orc_f32_to_f16.argtypes = [f32]
    L.orc_f16_to_f32.restype = f32; L.orc_f16_to_f32.argtypes = [u16]
    L.orc_f32_to_e4m3.restype = u8; L.orc_f32_to_e4m3.argtypes = [f32]
    L.orc_e4m3_to_f32.restype = f32; L.orc_e4m3_to_f32.argtypes = [u8]
    L.orc_fwht_f32.argtypes = [P(f32), i32]
    L.orc_fwht_f64.argtypes = [P(f64), i32]
    L.orc_int4_quantize_row.argtypes = [P(f32), i32, P(u8), P(f32)]
    L.orc_int4_dequant_row.argtypes = [P(u8), f32, i32, P(f64)]
    L.orc_reshape_and_cache_int4.restype = i32
    L.orc_reshape_and_cache_int4.argtypes = [
        C.c_void_p, C.c_void_p, i32, i64, i32, i32, P(i64), P(f32),
        P(u8), P(u8), P(f32), P(f32), i64, i32]
    L.orc_int4_decode.restype = i32
    L.orc_int4_decode.argtypes = [
        P(f32), P(u8), P(u8), P(f32), P(f32), P(i32), i32, P(i32),
        P(f32), i32, i32, i32, i32, i32, i32, f64, P(i32), i32,
        P(f64), P(f64)]
    L.orc_int4_prefill.restype = i32
    L.orc_int4_prefill.argtypes = [
        P(f32), P(u8), P(u8), P(f32), P(f32), P(i32), i32, P(i32), P(i32), i32,
        P(f32), i32, i32, i32, i32, f64, i32, f64, P(f32), P(f64)]
    L.orc_tq_full_dequant.restype = i32
    L.orc_tq_full_dequant.argtypes = [
        P(u8), P(i32), i32, P(f32), i32, i32, i32, i32, i64, i32, i32, i32, i32, i32,
        P(u16), P(u16)]
    L.orc_tq_slot_bytes.restype = i32
    L.orc_tq_slot_bytes.argtypes = [i32, i32, i32]
    L.orc_lloyd_max_gaussian.argtypes = [i32, P(f64)]
    L.orc_tq_encode.restype = i32
    L.orc_tq_encode.argtypes = [
        P(f32), P(f32), i64, i32, i32, i32, i32, P(f32), P(f32),
        P(i64), P(u8), i64, i32, i32]
    L.orc_tq_decode.restype = i32
    L.orc_tq_decode.argtypes = [
        P(f32), P(u8), P(i32), i32, P(i32), P(f32), P(f32), i32, i32,
        i32, i32, i32, i32, i32, i32, i32, i32, f64, P(i32), i32,
        P(f64), P(f64)]
    L.orc_fwht128_quant_fp8.argtypes = [P(u16), i64, P(u8), P(f32)]
    L.orc_fp8_pow2_scale.restype = f32
    L.orc_fp8_pow2_scale.argtypes = [f32]
    L.orc_convert.argtypes = [i32, C.c_void_p, C.c_void_p, i64]
    L.orc_exp_f32.restype = f32
    L.orc_exp_f32.argtypes = [f32]
    L.orc_kpool_compress_and_write.restype = i32
    L.orc_kpool_compress_and_write.argtypes = [
        P(u16), C.c_void_p, i32, P(f32), P(i64), P(u8), i64, i32, i32,
        P(u8), i64, i32, i32, P(u8), P(f32)]
    return L


def lib():
    global _lib
    with _lock:
        if _lib is None:
            # TQ_ORACLE_LIB names another build of this source (the
            # sanitizer test runs the pins against an ASan/UBSan build)
            alt = os.environ.get("TQ_ORACLE_LIB")
            _lib = _load(alt if alt else build())
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Route every oracle call through another build of the oracle (a test
    compiles a copy with one deliberate mistake to show that a pin catches
    it); the regular library is restored on exit."""
    global _lib
    prev = lib()
    with _lock:
        _lib = _load(path)
    try:
        yield
    finally:
        with _lock:
            _lib = prev


# ---------------------------------------------------------------- converters
def _convert(kind, x, in_dt, out_dt):
    x = np.ascontiguousarray(x, in_dt)
    out = np.empty(x.shape, out_dt)
    lib().orc_convert(kind, x.ctypes.data, out.ctypes.data, x.size)
    return out


def f32_to_bf16(x):
    return _convert(0, x, np.float32, np.uint16)


def bf16_to_f32(h):
    return _convert(1, h, np.uint16, np.float32)


def f32_to_f16(x):
    return _convert(2, x, np.float32, np.uint16)


def f16_to_f32(h):
    return _convert(3, h, np.uint16, np.float32)


def f32_to_e4m3(x):
    return _convert(4, x, np.float32, np.uint8)


def e4m3_to_f32(b):
    return _convert(5, b, np.uint8, np.float32)


def fp8_pow2_scale(absmax):
    return lib().orc_fp8_pow2_scale(float(absmax))


# -------------------------------------------------------------------- FWHT
def fwht_f32(x):
    """Unnormalized FWHT along the last axis in fp32 (rows processed in turn)."""
    y = np.ascontiguousarray(np.array(x, np.float32, copy=True))
    d = y.shape[-1]
    flat = y.reshape(-1, d)
    for r in range(flat.shape[0]):
        lib().orc_fwht_f32(_p(flat[r], C.c_float), d)
    return y


def fwht_f64(x):
    y = np.ascontiguousarray(np.array(x, np.float64, copy=True))
    d = y.shape[-1]
    flat = y.reshape(-1, d)
    for r in range(flat.shape[0]):
        lib().orc_fwht_f64(_p(flat[r], C.c_double), d)
    return y


# ---------------------------------------------------------------- INT4 write
def int4_quantize_row(x):
    x = np.ascontiguousarray(x, np.float32)
    d = x.shape[0]
    packed = np.zeros(d // 2, np.uint8)
    word = np.zeros(1, np.float32)
    lib().orc_int4_quantize_row(_p(x, C.c_float), d, _p(packed, C.c_uint8), _p(word, C.c_float))
    return packed, word[0]


def int4_dequant_row(packed, word, d):
    packed = np.ascontiguousarray(packed, np.uint8)
    out = np.zeros(d, np.float64)
    lib().orc_int4_dequant_row(_p(packed, C.c_uint8), float(word), d, _p(out, C.c_double))
    return out


def reshape_and_cache_int4(key_bits, value_bits, kv_dtype, slot_mapping, signs,
                           key_cache, value_cache, k_scale, v_scale):
    """In-place CPU write of the INT4 caches.

    key_bits/value_bits: [T, Hk, D] arrays holding the source values (float32
    for kv_dtype DT_F32, or the uint16 bit patterns for DT_F16 / DT_BF16).
    Caches: [NB, bs, Hk, D/2] u8; scale words [NB, bs, Hk] f32.
    """
    T, hk, d = key_bits.shape
    nb, bs = key_cache.shape[0], key_cache.shape[1]
    key_bits = np.ascontiguousarray(key_bits)
    value_bits = np.ascontiguousarray(value_bits)
    slot_mapping = np.ascontiguousarray(slot_mapping, np.int64)
    signs = np.ascontiguousarray(signs, np.float32)
    for a in (key_cache, value_cache, k_scale, v_scale):
        assert a.flags.c_contiguous
    rc = lib().orc_reshape_and_cache_int4(
        key_bits.ctypes.data, value_bits.ctypes.data, kv_dtype, T, hk, d,
        _p(slot_mapping, C.c_int64), _p(signs, C.c_float),
        _p(key_cache, C.c_uint8), _p(value_cache, C.c_uint8),
        _p(k_scale, C.c_float), _p(v_scale, C.c_float), nb, bs)
    assert rc == 0


def int4_decode(q, key_cache, value_cache, k_scale, v_scale, block_table,
                seq_lens, signs, num_splits, sm_scale, rows=None):
    """fp64 INT4 decode attention; returns (out [R, D] f64, lse [R] f64)."""
    q = np.ascontiguousarray(q, np.float32)
    B, hq, d = q.shape
    hk = key_cache.shape[2]
    bs = key_cache.shape[1]
    block_table = np.ascontiguousarray(block_table, np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    signs = np.ascontiguousarray(signs, np.float32)
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int32)
    n = B * hq if rows is None else rows.shape[0]
    out = np.zeros((n, d), np.float64)
    lse = np.zeros(n, np.float64)
    rc = lib().orc_int4_decode(
        _p(q, C.c_float), _p(np.ascontiguousarray(key_cache), C.c_uint8),
        _p(np.ascontiguousarray(value_cache), C.c_uint8),
        _p(np.ascontiguousarray(k_scale), C.c_float),
        _p(np.ascontiguousarray(v_scale), C.c_float),
        _p(block_table, C.c_int32), block_table.shape[1], _p(seq_lens, C.c_int32),
        _p(signs, C.c_float), B, hq, hk, d, bs, num_splits, float(sm_scale),
        _p(rows, C.c_int32), 0 if rows is None else rows.shape[0],
        _p(out, C.c_double), _p(lse, C.c_double))
    assert rc == 0
    return out, lse


# ------------------------------------------------------------- TurboQuant
def int4_prefill(q, key_cache, value_cache, k_scale, v_scale, block_table, cu_seqlens_q,
                 seq_lens, signs, sm_scale, window=0, softcap=0.0, sinks=None):
    """[int4] _attn_packed 2D mode: q [T, Hq, D] f32 -> out [T, Hq, D] f64.
    window = 1 + window_size[0] (0: none); softcap 0: none; sinks [Hq] or None."""
    q = np.ascontiguousarray(q, np.float32)
    T, hq, d = q.shape
    hk = key_cache.shape[2]
    bt = np.ascontiguousarray(block_table, np.int32)
    cu = np.ascontiguousarray(cu_seqlens_q, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    assert cu.shape == (sl.shape[0] + 1,) and cu[-1] == T
    sk = None if sinks is None else np.ascontiguousarray(sinks, np.float32)
    out = np.zeros((T, hq, d), np.float64)
    rc = lib().orc_int4_prefill(
        _p(q, C.c_float), _p(np.ascontiguousarray(key_cache), C.c_uint8),
        _p(np.ascontiguousarray(value_cache), C.c_uint8), _p(np.ascontiguousarray(k_scale), C.c_float),
        _p(np.ascontiguousarray(v_scale), C.c_float), _p(bt, C.c_int32), bt.shape[1],
        _p(cu, C.c_int32), _p(sl, C.c_int32), sl.shape[0],
        _p(np.ascontiguousarray(signs, np.float32), C.c_float), hq, hk, d, key_cache.shape[1],
        float(sm_scale), int(window), float(softcap), _p(sk, C.c_float), _p(out, C.c_double))
    if rc != 0:
        raise ValueError("int4_prefill: invalid arguments")
    return out


def tq_slot_bytes(d, key_fmt, val_fmt):
    return lib().orc_tq_slot_bytes(d, key_fmt, val_fmt)


def lloyd_max_gaussian(levels):
    c = np.zeros(levels, np.float64)
    lib().orc_lloyd_max_gaussian(levels, _p(c, C.c_double))
    return c


def tq_encode(key, value, key_fmt, val_fmt, centroids, rot_signs, slot_mapping,
              kv_cache):
    """In-place CPU encode of fp32 key/value [T, Hk, D] into the slot cache
    [NB, bs, Hk, slot_bytes] u8."""
    key = np.ascontiguousarray(key, np.float32)
    value = np.ascontiguousarray(value, np.float32)
    T, hk, d = key.shape
    nb, bs, _, sb = kv_cache.shape
    assert kv_cache.flags.c_contiguous
    cen = None if centroids is None else np.ascontiguousarray(centroids, np.float32)
    rs = None if rot_signs is None else np.ascontiguousarray(rot_signs, np.float32)
    slot_mapping = np.ascontiguousarray(slot_mapping, np.int64)
    rc = lib().orc_tq_encode(
        _p(key, C.c_float), _p(value, C.c_float), T, hk, d, key_fmt, val_fmt,
        _p(cen, C.c_float), _p(rs, C.c_float), _p(slot_mapping, C.c_int64),
        _p(kv_cache, C.c_uint8), nb, bs, sb)
    assert rc == 0


def tq_decode(q, kv_cache, block_table, seq_lens, centroids, rot_signs, key_fmt,
              val_fmt, norm_correction, num_splits, sm_scale, rows=None):
    q = np.ascontiguousarray(q, np.float32)
    B, hq, d = q.shape
    nb, bs, hk, sb = kv_cache.shape
    block_table = np.ascontiguousarray(block_table, np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    cen = None if centroids is None else np.ascontiguousarray(centroids, np.float32)
    rs = None if rot_signs is None else np.ascontiguousarray(rot_signs, np.float32)
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int32)
    n = B * hq if rows is None else rows.shape[0]
    out = np.zeros((n, d), np.float64)
    lse = np.zeros(n, np.float64)
    rc = lib().orc_tq_decode(
        _p(q, C.c_float), _p(np.ascontiguousarray(kv_cache), C.c_uint8),
        _p(block_table, C.c_int32), block_table.shape[1], _p(seq_lens, C.c_int32),
        _p(cen, C.c_float), _p(rs, C.c_float), B, hq, hk, d, bs, sb, key_fmt,
        val_fmt, int(norm_correction), num_splits, float(sm_scale),
        _p(rows, C.c_int32), 0 if rows is None else rows.shape[0],
        _p(out, C.c_double), _p(lse, C.c_double))
    assert rc == 0
    return out, lse


# ---------------------------------------------------------- FWHT-128 + FP8
def tq_full_dequant(kv_cache, block_table, d, key_fmt, val_fmt, max_seq, num_blocks=None,
                    centroids=None, norm_correction=False):
    """[tq] _tq_full_dequant_kv on host arrays: kv_cache [NB, bs, Hk, slot]
    u8 -> (k, v) [B, Hk, max_seq, d] uint16 fp16 bit patterns."""
    kv = np.ascontiguousarray(kv_cache, np.uint8)
    nb, bs, hk, sb = kv.shape
    bt = np.ascontiguousarray(block_table, np.int32)
    B = bt.shape[0]
    cen = None if centroids is None else np.ascontiguousarray(centroids, np.float32)
    k = np.zeros((B, hk, max_seq, d), np.uint16)
    v = np.zeros((B, hk, max_seq, d), np.uint16)
    rc = lib().orc_tq_full_dequant(
        _p(kv, C.c_uint8), _p(bt, C.c_int32), bt.shape[1], _p(cen, C.c_float), B, hk, d, bs,
        nb if num_blocks is None else num_blocks, sb, key_fmt, val_fmt,
        1 if norm_correction else 0, max_seq, _p(k, C.c_uint16), _p(v, C.c_uint16))
    if rc != 0:
        raise ValueError("tq_full_dequant: invalid arguments")
    return k, v


def fwht128_quant_fp8(x_bf16_bits):
    """x: [rows, 128] uint16 bf16 bit patterns -> (y [rows,128] u8, scale [rows] f32)."""
    x = np.ascontiguousarray(x_bf16_bits, np.uint16)
    rows = x.shape[0]
    y = np.zeros((rows, 128), np.uint8)
    s = np.zeros(rows, np.float32)
    if rows:
        lib().orc_fwht128_quant_fp8(_p(x, C.c_uint16), rows, _p(y, C.c_uint8), _p(s, C.c_float))
    return y, s


# ------------------------------------------------ pooled key compression
_SCORE_DT = {"f32": DT_F32, "f16": DT_F16, "bf16": DT_BF16}


def exp_f32(x):
    """e^x rounded to the nearest fp32 (the kpool softmax exponential)."""
    return lib().orc_exp_f32(float(np.float32(x)))


def kpool_compress_and_write(slot_k_bits, slot_score, ape, loc=None, kv_cache=None,
                             write_mask=None, round_scale=True,
                             return_compressed=False, score_dtype="f32"):
    """[kpool] kpool_compress_and_write_cache on host arrays.

    slot_k_bits: [n, P, 128] uint16 bf16 bit patterns. slot_score: [n, P, 128]
    float32 for score_dtype "f32", else uint16 f16 / bf16 bit patterns.
    ape: [P, 128] float32. loc: [n] int64 flat entry index. kv_cache:
    [num_blocks, block_size, 132] uint8, written in place. write_mask: [n]
    bool or None. Returns (codes [n, 128] u8, scales [n] f32) when
    ``return_compressed``, else None.
    """
    k = np.ascontiguousarray(slot_k_bits, np.uint16)
    n, P, hd = k.shape
    sdt = _SCORE_DT[score_dtype]
    sc = np.ascontiguousarray(slot_score, np.float32 if sdt == DT_F32 else np.uint16)
    assert sc.shape == k.shape
    a = np.ascontiguousarray(ape, np.float32)
    assert a.shape == (P, hd)
    lo = None if loc is None else np.ascontiguousarray(loc, np.int64)
    wm = None if write_mask is None else np.ascontiguousarray(write_mask, np.uint8)
    nb = bs = 0
    if kv_cache is not None:
        assert kv_cache.dtype == np.uint8 and kv_cache.flags.c_contiguous
        nb, bs = kv_cache.shape[0], kv_cache.shape[1]
        assert kv_cache.shape[2] == hd + 4
    ck = cs = None
    if return_compressed:
        ck = np.zeros((n, hd), np.uint8)
        cs = np.zeros(n, np.float32)
    rc = lib().orc_kpool_compress_and_write(
        _p(k, C.c_uint16), sc.ctypes.data, sdt, _p(a, C.c_float), _p(lo, C.c_int64),
        _p(wm, C.c_uint8), n, P, hd, _p(kv_cache, C.c_uint8), nb, bs,
        1 if round_scale else 0, _p(ck, C.c_uint8), _p(cs, C.c_float))
    if rc != 0:
        raise ValueError("kpool_compress_and_write: invalid arguments")
    return (ck, cs) if return_compressed else None
