"""MI355X (gfx950) quantized paged-KV decode attention and cache writers.

Thin Python binding over the C ABI of ``libtq_amd.so`` (declared in
``include/tq.h``): argument marshalling only -- every step of the path runs
in the library's HIP kernels. torch supplies device memory and streams.

    tq_reshape_and_cache_int4   RHT + INT4 paged-cache write
    tq_encode_and_cache         TurboQuant combined-slot cache write
    tq_decode_attention         split-KV decode (stage 1 + stage 2)
    tq_decode_attention_static  the same, with the library's static
                                workspace (for callers that cannot allocate)
    fwht128_quant_fp8           Hadamard-128 + power-of-two-scale FP8
    tq_prefill_attention_int4   multi-query (prefill) attention over the
                                INT4 cache
    tq_full_dequant_kv          bulk TurboQuant slot dequant to fp16 K/V
    tq_kpool_compress_and_write_cache
                                pooled-softmax key compression into the
                                FP8 indexer page

The library is loaded on first use; when it is missing or cannot be loaded
the call raises (there is no fallback implementation).
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq_amd.so")

TQ_OK, TQ_EINVAL, TQ_ENOTSUP, TQ_ELAUNCH = 0, -1, -2, -3
DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2
KEY_INT4, KEY_FP8, KEY_MSE3, KEY_MSE4 = 0, 1, 2, 3
VAL_INT4, VAL_U3, VAL_U4, VAL_FP8 = 0, 1, 2, 3
FLAG_GENERIC = 1
FLAG_WIDE = 2


class TQError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class PrefillArgs(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32), ("num_seqs", C.c_int32), ("Hq", C.c_int32),
        ("Hk", C.c_int32), ("D", C.c_int32), ("block_size", C.c_int32),
        ("max_blocks", C.c_int32), ("window", C.c_int32), ("num_tokens", C.c_int64),
        ("num_blocks", C.c_int64), ("sm_scale", C.c_float), ("softcap", C.c_float),
        ("query", C.c_void_p), ("cu_seqlens_q", C.c_void_p), ("seq_lens", C.c_void_p),
        ("block_table", C.c_void_p), ("key_cache", C.c_void_p), ("value_cache", C.c_void_p),
        ("k_scale_cache", C.c_void_p), ("v_scale_cache", C.c_void_p), ("rht_signs", C.c_void_p),
        ("sinks", C.c_void_p), ("output_scale", C.c_void_p), ("out", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_int64),
    ]


class DecodeArgs(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32), ("flags", C.c_uint32),
        ("B", C.c_int32), ("Hq", C.c_int32), ("Hk", C.c_int32), ("D", C.c_int32),
        ("block_size", C.c_int32), ("max_blocks", C.c_int32), ("num_kv_splits", C.c_int32),
        ("key_fmt", C.c_int32), ("val_fmt", C.c_int32), ("norm_correction", C.c_int32),
        ("sm_scale", C.c_float), ("num_blocks", C.c_int64),
        ("query", C.c_void_p), ("block_table", C.c_void_p), ("seq_lens", C.c_void_p),
        ("key_cache", C.c_void_p), ("value_cache", C.c_void_p),
        ("k_scale_cache", C.c_void_p), ("v_scale_cache", C.c_void_p), ("rht_signs", C.c_void_p),
        ("kv_cache", C.c_void_p), ("slot_bytes", C.c_int32),
        ("centroids", C.c_void_p), ("rot_signs", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_int64),
        ("out", C.c_void_p), ("lse", C.c_void_p),
    ]


_lock = threading.Lock()
_lib = None

# Every entry point the header declares: (name, restype, argtypes).
SYMBOLS = {
    "tq_last_error": (C.c_char_p, []),
    "tq_version": (C.c_int, []),
    "tq_reshape_and_cache_int4": (C.c_int, [
        C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
        C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int32,
        C.c_void_p]),
    "tq_encode_and_cache": (C.c_int, [
        C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
        C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int64,
        C.c_int32, C.c_void_p]),
    "tq_decode_workspace_bytes": (C.c_size_t, [C.c_int32] * 5),
    "tq_slot_bytes": (C.c_int32, [C.c_int32] * 3),
    "tq_decode_attention": (C.c_int, [C.POINTER(DecodeArgs), C.c_void_p]),
    "tq_decode_attention_static": (C.c_int, [C.POINTER(DecodeArgs), C.c_void_p]),
    "fwht128_quant_fp8": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]),
    "tq_prefill_attention_int4": (C.c_int, [C.POINTER(PrefillArgs), C.c_void_p]),
    "tq_prefill_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int32, C.c_int32, C.c_int32]),
    "tq_full_dequant_kv": (C.c_int, [
        C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
        C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
        C.c_void_p, C.c_void_p, C.c_void_p]),
    "tq_kpool_compress_and_write_cache": (C.c_int, [
        C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
        C.c_int32, C.c_int32, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
        C.c_void_p, C.c_void_p]),
}


def lib():
    """Load libtq_amd.so (raises when it is absent: no fallback path)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    "libtq_amd.so is not built (run quantized_paged_kv_tq_amd/build.py "
                    "or __graft_entry__.build())")
            L = C.CDLL(LIB_PATH)
            for name, (res, args) in SYMBOLS.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def last_error() -> str:
    return lib().tq_last_error().decode()


def _check(code):
    if code != TQ_OK:
        raise TQError(code, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    if isinstance(stream, C.c_void_p):
        return stream
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return C.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, device=None):
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


_DT = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}


def prepare_reshape(key, value, key_cache, value_cache, slot_mapping, *, k_scale_cache,
                    v_scale_cache, rht_signs):
    """Validate and marshal a tq_reshape_and_cache_int4 call (see Prepared)."""
    T, hk, d = key.shape
    if value.shape != key.shape or value.dtype != key.dtype:
        raise ValueError("key and value must share shape and dtype")
    if key.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % key.dtype)
    for t, n in ((key, "key"), (value, "value")):
        _need(t, key.dtype, n)
    _need(slot_mapping, torch.int64, "slot_mapping")
    _need(rht_signs, torch.float32, "rht_signs")
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, torch.uint8, n)
    for t, n in ((k_scale_cache, "k_scale_cache"), (v_scale_cache, "v_scale_cache")):
        _need(t, torch.float32, n)
    nb, bs = key_cache.shape[0], key_cache.shape[1]
    if tuple(key_cache.shape) != (nb, bs, hk, d // 2) or value_cache.shape != key_cache.shape:
        raise ValueError("cache shape must be [NB, bs, Hk, D/2]")
    if tuple(k_scale_cache.shape) != (nb, bs, hk) or v_scale_cache.shape != k_scale_cache.shape:
        raise ValueError("scale cache shape must be [NB, bs, Hk]")
    if slot_mapping.shape != (T,) or rht_signs.shape != (d,):
        raise ValueError("slot_mapping must be [T], rht_signs [D]")
    args = (_ptr(key), _ptr(value), _DT[key.dtype], T, hk, d, _ptr(slot_mapping),
            _ptr(rht_signs), _ptr(key_cache), _ptr(value_cache), _ptr(k_scale_cache),
            _ptr(v_scale_cache), nb, bs)
    keep = [key, value, key_cache, value_cache, slot_mapping, k_scale_cache, v_scale_cache,
            rht_signs]
    return Prepared(lib().tq_reshape_and_cache_int4, args, keep)


def tq_reshape_and_cache_int4(key, value, key_cache, value_cache, slot_mapping, *,
                              k_scale_cache, v_scale_cache, rht_signs, stream=None):
    """RHT + INT4 write of key/value [T, Hk, D] into the paged caches
    ([NB, bs, Hk, D/2] u8 and [NB, bs, Hk] f32 scale words), in place."""
    prepare_reshape(key, value, key_cache, value_cache, slot_mapping, k_scale_cache=k_scale_cache,
                    v_scale_cache=v_scale_cache, rht_signs=rht_signs).run(stream, key.device)


def prepare_encode(key, value, kv_cache, slot_mapping, *, key_fmt, val_fmt, centroids=None,
                   rot_signs=None):
    """Validate and marshal a tq_encode_and_cache call (see Prepared)."""
    T, hk, d = key.shape
    if value.shape != key.shape or value.dtype != key.dtype:
        raise ValueError("key and value must share shape and dtype")
    if key.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % key.dtype)
    for t, n in ((key, "key"), (value, "value")):
        _need(t, key.dtype, n)
    _need(slot_mapping, torch.int64, "slot_mapping")
    _need(kv_cache, torch.uint8, "kv_cache")
    if kv_cache.dim() != 4 or kv_cache.shape[2] != hk:
        raise ValueError("kv_cache must be [NB, bs, Hk, slot_bytes]")
    nb, bs, _, sb = kv_cache.shape
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    keep = [key, value, kv_cache, slot_mapping]
    for t, n in ((centroids, "centroids"), (rot_signs, "rot_signs")):
        if t is not None:
            _need(t, torch.float32, n)
            keep.append(t)
    args = (_ptr(key), _ptr(value), _DT[key.dtype], T, hk, d, key_fmt, val_fmt, _ptr(slot_mapping),
            _ptr(centroids) if centroids is not None else None,
            _ptr(rot_signs) if rot_signs is not None else None, _ptr(kv_cache), sb, nb, bs)
    return Prepared(lib().tq_encode_and_cache, args, keep)


def tq_encode_and_cache(key, value, kv_cache, slot_mapping, *, key_fmt, val_fmt, centroids=None,
                        rot_signs=None, stream=None):
    """TurboQuant encode of key/value [T, Hk, D] into the combined-slot cache
    [NB, bs, Hk, slot_bytes] u8, in place."""
    prepare_encode(key, value, kv_cache, slot_mapping, key_fmt=key_fmt, val_fmt=val_fmt,
                   centroids=centroids, rot_signs=rot_signs).run(stream, key.device)


def tq_decode_workspace_bytes(B, Hq, Hk, D, num_kv_splits):
    return lib().tq_decode_workspace_bytes(B, Hq, Hk, D, num_kv_splits)


def tq_slot_bytes(D, key_fmt, val_fmt):
    return lib().tq_slot_bytes(D, key_fmt, val_fmt)


class Prepared:
    """A library call whose arguments are marshalled once: ``run(stream)``
    re-issues it (used by timing loops, where per-call marshalling would
    dominate a microsecond-scale kernel)."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def run(self, stream=None, device=None):
        s = _stream(stream, device if device is not None else self._keep[0].device)
        _check(self._fn(*self._args, s))


def prepare_decode(query, block_table, seq_lens, *, num_kv_splits, sm_scale=None,
                   key_cache=None, value_cache=None, k_scale_cache=None, v_scale_cache=None,
                   rht_signs=None, kv_cache=None, key_fmt=KEY_INT4, val_fmt=VAL_INT4,
                   centroids=None, rot_signs=None, norm_correction=False, num_kv_heads=None,
                   workspace=None, out=None, lse=None, flags=0, static_workspace=False):
    """Validate and marshal a tq_decode_attention call; returns (Prepared, out, lse).
    static_workspace=True marshals tq_decode_attention_static instead, which
    takes its workspace from the library (no workspace argument)."""
    B, hq, d = query.shape
    _need(query, torch.float32, "query")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    if key_fmt == KEY_INT4:
        nb, bs, hk = key_cache.shape[0], key_cache.shape[1], key_cache.shape[2]
        _need(key_cache, torch.uint8, "key_cache")
        _need(value_cache, torch.uint8, "value_cache")
        _need(k_scale_cache, torch.float32, "k_scale_cache")
        _need(v_scale_cache, torch.float32, "v_scale_cache")
        _need(rht_signs, torch.float32, "rht_signs")
        if tuple(key_cache.shape) != (nb, bs, hk, d // 2) or value_cache.shape != key_cache.shape:
            raise ValueError("INT4 caches must be [NB, bs, Hk, D/2]")
        if tuple(k_scale_cache.shape) != (nb, bs, hk) or v_scale_cache.shape != k_scale_cache.shape:
            raise ValueError("scale caches must be [NB, bs, Hk]")
        slot_bytes = 0
    else:
        _need(kv_cache, torch.uint8, "kv_cache")
        nb, bs, hk, slot_bytes = kv_cache.shape
        if centroids is not None:
            _need(centroids, torch.float32, "centroids")
        if rot_signs is not None:
            _need(rot_signs, torch.float32, "rot_signs")
    if num_kv_heads is not None and num_kv_heads != hk:
        raise ValueError("num_kv_heads does not match the cache")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks], seq_lens [B]")
    dev = query.device
    if static_workspace:
        if workspace is not None:
            raise ValueError("the static entry point takes no workspace")
    elif workspace is None:
        nbytes = tq_decode_workspace_bytes(B, hq, hk, d, num_kv_splits)
        workspace = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty(B, hq, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(B, hq, dtype=torch.float32, device=dev)
    if not static_workspace:
        _need(workspace, torch.float32, "workspace")
        if workspace.numel() * 4 < tq_decode_workspace_bytes(B, hq, hk, d, num_kv_splits):
            raise ValueError("workspace too small")
    _need(out, torch.float32, "out")
    _need(lse, torch.float32, "lse")
    a = DecodeArgs()
    a.struct_size = C.sizeof(DecodeArgs)
    a.flags = flags
    a.B, a.Hq, a.Hk, a.D = B, hq, hk, d
    a.block_size, a.max_blocks, a.num_kv_splits = bs, block_table.shape[1], num_kv_splits
    a.key_fmt, a.val_fmt, a.norm_correction = key_fmt, val_fmt, int(bool(norm_correction))
    a.sm_scale = (1.0 / d ** 0.5) if sm_scale is None else sm_scale
    a.num_blocks = nb
    a.query, a.block_table, a.seq_lens = _ptr(query), _ptr(block_table), _ptr(seq_lens)
    a.key_cache, a.value_cache = _ptr(key_cache), _ptr(value_cache)
    a.k_scale_cache, a.v_scale_cache = _ptr(k_scale_cache), _ptr(v_scale_cache)
    a.rht_signs = _ptr(rht_signs)
    a.kv_cache, a.slot_bytes = _ptr(kv_cache), slot_bytes
    a.centroids, a.rot_signs = _ptr(centroids), _ptr(rot_signs)
    a.workspace, a.out, a.lse = _ptr(workspace), _ptr(out), _ptr(lse)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * 4
    keep = [query, block_table, seq_lens, key_cache, value_cache, k_scale_cache, v_scale_cache,
            rht_signs, kv_cache, centroids, rot_signs, workspace, out, lse]
    fn = lib().tq_decode_attention_static if static_workspace else lib().tq_decode_attention
    return Prepared(fn, (C.byref(a),), keep + [a]), out, lse


def tq_decode_attention(query, block_table, seq_lens, *, stream=None, **kw):
    """Split-KV decode attention; returns (out [B, Hq, D] f32, lse [B, Hq] f32).

    INT4 format: key_cache/value_cache [NB, bs, Hk, D/2] u8, k/v_scale_cache
    [NB, bs, Hk] f32, rht_signs [D]. TurboQuant formats: kv_cache
    [NB, bs, Hk, slot_bytes] u8 (+ centroids for centroid keys).
    workspace/out/lse may be passed pre-allocated (no allocation then).
    """
    call, out, lse = prepare_decode(query, block_table, seq_lens, **kw)
    call.run(stream, query.device)
    return out, lse


def tq_decode_attention_static(query, block_table, seq_lens, *, stream=None, **kw):
    """tq_decode_attention through the library's static workspace (the C
    entry point allocates nothing; see include/tq.h). Calls that overlap on
    one GPU share that workspace and race."""
    call, out, lse = prepare_decode(query, block_table, seq_lens, static_workspace=True, **kw)
    call.run(stream, query.device)
    return out, lse


def fwht128_quant_fp8(x, y=None, scale=None, stream=None):
    """x [rows, 128] bf16 -> (y [rows, 128] float8_e4m3fn, scale [rows, 1] f32)."""
    if x.dim() != 2 or x.shape[1] != 128:
        raise ValueError("x must be [rows, 128]")
    _need(x, torch.bfloat16, "x")
    rows = x.shape[0]
    if y is None:
        y = torch.empty(rows, 128, dtype=torch.float8_e4m3fn, device=x.device)
    if scale is None:
        scale = torch.empty(rows, 1, dtype=torch.float32, device=x.device)
    if y.shape != (rows, 128) or scale.numel() != rows:
        raise ValueError("y must be [rows, 128], scale [rows, 1]")
    _check(lib().fwht128_quant_fp8(_ptr(x), rows, _ptr(y), _ptr(scale), _stream(stream, x.device)))
    return y, scale


def prepare_kpool(kv_cache, slot_k, slot_score, ape, loc, *, write_mask=None, round_scale=True,
                  compressed_k=None, compressed_scale=None):
    """Validate and marshal a tq_kpool_compress_and_write_cache call (see
    Prepared). kv_cache may be None when compressed_k/compressed_scale are
    given."""
    if slot_k.dim() != 3:
        raise ValueError("slot_k must be [n_pools, pool_size, head_dim]")
    n, P, hd = slot_k.shape
    _need(slot_k, torch.bfloat16, "slot_k")
    if slot_score.dtype not in _DT:
        raise TypeError("unsupported slot_score dtype %s" % slot_score.dtype)
    _need(slot_score, slot_score.dtype, "slot_score")
    _need(ape, torch.float32, "ape")
    if slot_score.shape != slot_k.shape or tuple(ape.shape) != (P, hd):
        raise ValueError("slot_score must match slot_k, ape must be [pool_size, head_dim]")
    keep = [slot_k, slot_score, ape]
    nb = bs = 0
    if kv_cache is not None:
        _need(kv_cache, torch.uint8, "kv_cache")
        if kv_cache.dim() != 3 or kv_cache.shape[2] != hd + 4:
            raise ValueError("kv_cache must be [num_blocks, block_size, head_dim + 4]")
        nb, bs = kv_cache.shape[0], kv_cache.shape[1]
        _need(loc, torch.int64, "loc")
        if loc.shape != (n,):
            raise ValueError("loc must be [n_pools]")
        keep += [kv_cache, loc]
    if write_mask is not None:
        if write_mask.dtype not in (torch.bool, torch.uint8):
            raise TypeError("write_mask must be bool or uint8")
        _need(write_mask, write_mask.dtype, "write_mask")
        if write_mask.shape != (n,):
            raise ValueError("write_mask must be [n_pools]")
        keep.append(write_mask)
    if compressed_k is not None:
        if compressed_k.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError("compressed_k must be float8_e4m3fn or uint8")
        _need(compressed_k, compressed_k.dtype, "compressed_k")
        _need(compressed_scale, torch.float32, "compressed_scale")
        if tuple(compressed_k.shape) != (n, hd) or compressed_scale.numel() != n:
            raise ValueError("compressed_k must be [n_pools, head_dim], compressed_scale [n_pools]")
        keep += [compressed_k, compressed_scale]
    args = (_ptr(slot_k), _ptr(slot_score), _DT[slot_score.dtype], _ptr(ape),
            _ptr(loc) if kv_cache is not None else None, _ptr(write_mask), n, P, hd,
            _ptr(kv_cache), nb, bs, 1 if round_scale else 0, _ptr(compressed_k),
            _ptr(compressed_scale))
    return Prepared(lib().tq_kpool_compress_and_write_cache, args, keep)


def tq_kpool_compress_and_write_cache(kv_cache, slot_k, slot_score, ape, loc, *, write_mask=None,
                                      round_scale=True, return_compressed=False,
                                      write_cache=True, stream=None):
    """Compress each pool of slot_k [n, P, 128] bf16 (softmax over P of
    slot_score + ape, per dimension) into one FP8 entry written at loc [n] of
    the indexer cache [num_blocks, block_size, 132] u8. Returns (codes [n, 128]
    float8_e4m3fn, scales [n] f32) when return_compressed, else None."""
    n, _, hd = slot_k.shape
    ck = cs = None
    if return_compressed:
        ck = torch.empty(n, hd, dtype=torch.float8_e4m3fn, device=slot_k.device)
        cs = torch.empty(n, dtype=torch.float32, device=slot_k.device)
    prepare_kpool(kv_cache if write_cache else None, slot_k, slot_score, ape, loc,
                  write_mask=write_mask, round_scale=round_scale, compressed_k=ck,
                  compressed_scale=cs).run(stream, slot_k.device)
    return (ck, cs) if return_compressed else None


def tq_prefill_workspace_bytes(num_tokens, Hq, Hk, D):
    """Workspace bytes that put tq_prefill_attention_int4 on the matrix cores
    (0 when that path does not apply)."""
    return lib().tq_prefill_workspace_bytes(num_tokens, Hq, Hk, D)


def prepare_prefill(query, key_cache, value_cache, block_table, cu_seqlens_q, seq_lens, *,
                    k_scale_cache, v_scale_cache, rht_signs, sm_scale=None, window=0,
                    softcap=0.0, sinks=None, output_scale=None, out=None, workspace="auto"):
    """Validate and marshal a tq_prefill_attention_int4 call; returns (Prepared, out).
    out is [T, Hq, D] f32, or float8_e4m3fn when output_scale ([1] f32) is given.
    workspace: "auto" allocates what the matrix-core path needs (none when it
    does not apply), None takes the vector path, or a device tensor."""
    T, hq, d = query.shape
    _need(query, torch.float32, "query")
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, torch.uint8, n)
    for t, n in ((k_scale_cache, "k_scale_cache"), (v_scale_cache, "v_scale_cache"),
                 (rht_signs, "rht_signs")):
        _need(t, torch.float32, n)
    for t, n in ((block_table, "block_table"), (cu_seqlens_q, "cu_seqlens_q"),
                 (seq_lens, "seq_lens")):
        _need(t, torch.int32, n)
    nb, bs, hk, _ = key_cache.shape
    if tuple(key_cache.shape) != (nb, bs, hk, d // 2) or value_cache.shape != key_cache.shape:
        raise ValueError("cache shape must be [NB, bs, Hk, D/2]")
    ns = seq_lens.shape[0]
    if cu_seqlens_q.shape != (ns + 1,) or block_table.dim() != 2 or block_table.shape[0] != ns:
        raise ValueError("cu_seqlens_q must be [num_seqs + 1], block_table [num_seqs, max_blocks]")
    keep = [query, key_cache, value_cache, block_table, cu_seqlens_q, seq_lens, k_scale_cache,
            v_scale_cache, rht_signs]
    if sinks is not None:
        _need(sinks, torch.float32, "sinks")
        if sinks.shape != (hq,):
            raise ValueError("sinks must be [Hq]")
        keep.append(sinks)
    odt = torch.float32
    if output_scale is not None:
        _need(output_scale, torch.float32, "output_scale")
        keep.append(output_scale)
        odt = torch.float8_e4m3fn
    if out is None:
        out = torch.empty(T, hq, d, dtype=odt, device=query.device)
    _need(out, odt, "out")
    if tuple(out.shape) != (T, hq, d):
        raise ValueError("out must be [T, Hq, D]")
    keep.append(out)
    a = PrefillArgs()
    a.struct_size = C.sizeof(PrefillArgs)
    a.num_seqs, a.Hq, a.Hk, a.D = ns, hq, hk, d
    a.block_size, a.max_blocks, a.window = bs, block_table.shape[1], int(window)
    a.num_tokens, a.num_blocks = T, nb
    a.sm_scale = float(d ** -0.5 if sm_scale is None else sm_scale)
    a.softcap = float(softcap)
    a.query, a.cu_seqlens_q, a.seq_lens = _ptr(query), _ptr(cu_seqlens_q), _ptr(seq_lens)
    a.block_table, a.key_cache, a.value_cache = _ptr(block_table), _ptr(key_cache), _ptr(value_cache)
    a.k_scale_cache, a.v_scale_cache, a.rht_signs = (_ptr(k_scale_cache), _ptr(v_scale_cache),
                                                     _ptr(rht_signs))
    a.sinks, a.output_scale, a.out = _ptr(sinks), _ptr(output_scale), _ptr(out)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        nbytes = tq_prefill_workspace_bytes(T, hq, hk, d)
        workspace = (torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=query.device)
                     if nbytes > 0 else None)
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        keep.append(workspace)
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    keep.append(a)
    return Prepared(lib().tq_prefill_attention_int4, (C.byref(a),), keep), out


def tq_prefill_attention_int4(query, key_cache, value_cache, block_table, cu_seqlens_q, seq_lens,
                              *, stream=None, **kw):
    """Multi-query (prefill) attention over the INT4 caches; returns out
    [T, Hq, D] (f32, or float8_e4m3fn with output_scale)."""
    call, out = prepare_prefill(query, key_cache, value_cache, block_table, cu_seqlens_q,
                                seq_lens, **kw)
    call.run(stream, query.device)
    return out


def prepare_full_dequant(kv_cache, block_table, *, head_dim, key_fmt, val_fmt, max_seq,
                         centroids=None, norm_correction=False, k_out=None, v_out=None):
    """Validate and marshal a tq_full_dequant_kv call; returns (Prepared, k, v)
    with k, v [B, Hk, max_seq, D] float16."""
    _need(kv_cache, torch.uint8, "kv_cache")
    _need(block_table, torch.int32, "block_table")
    if kv_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("kv_cache must be [NB, bs, Hk, slot_bytes], block_table [B, max_blocks]")
    nb, bs, hk, sb = kv_cache.shape
    B = block_table.shape[0]
    keep = [kv_cache, block_table]
    if centroids is not None:
        _need(centroids, torch.float32, "centroids")
        keep.append(centroids)
    shape = (B, hk, max_seq, head_dim)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.float16, device=kv_cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.float16, device=kv_cache.device)
    for t, n in ((k_out, "k_out"), (v_out, "v_out")):
        _need(t, torch.float16, n)
        if tuple(t.shape) != shape:
            raise ValueError("%s must be [B, Hk, max_seq, D]" % n)
        keep.append(t)
    args = (_ptr(kv_cache), _ptr(block_table), block_table.shape[1], _ptr(centroids), B, hk,
            head_dim, bs, nb, sb, key_fmt, val_fmt, 1 if norm_correction else 0, max_seq,
            _ptr(k_out), _ptr(v_out))
    return Prepared(lib().tq_full_dequant_kv, args, keep), k_out, v_out


def tq_full_dequant_kv(kv_cache, block_table, *, stream=None, **kw):
    """Dequantize every TurboQuant slot below max_seq to fp16 (k, v) [B, Hk, max_seq, D]."""
    call, k, v = prepare_full_dequant(kv_cache, block_table, **kw)
    call.run(stream, kv_cache.device)
    return k, v
