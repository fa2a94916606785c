"""Seeded synthetic inputs for the decode, cache-write and FWHT-FP8 paths.

This module draws random inputs and lays out page tables; it holds none of
the method's arithmetic (no rotation, quantization or attention), so the
tests can feed the very same arrays to the HIP library and to the CPU oracle.

Seeds: ``numpy.random.default_rng([workload_id, tensor_id])``. Normal draws
are made in fp32 and rounded to the stated storage dtype by torch's own cast.
The +-1 rotation signs come from torch's CPU generator seeded as the
int4_per_token_head.py page does in ``_get_rht_signs`` (round 0).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

RHT_SEED = 0x9E3779B9
RHT_ROUND_STRIDE = 0x517CC1B7


def rht_signs(d: int, round_idx: int = 0) -> np.ndarray:
    """+-1 float32 sign vector of length d, drawn with torch's CPU generator."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(RHT_SEED + round_idx * RHT_ROUND_STRIDE)
    s = 2.0 * torch.bernoulli(torch.full((d,), 0.5), generator=gen) - 1.0
    return s.to(torch.float32).numpy()


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([workload_id, tensor_id])


def to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to bf16/f16 with torch's cast; return the uint16 bits
    (or the fp32 array itself for dtype 'f32')."""
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f32":
        return t.numpy().copy()
    raise ValueError(dtype)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of bf16/f16 bit patterns to fp32 (torch's cast)."""
    if dtype == "f32":
        return np.asarray(bits, np.float32)
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(torch.float32).numpy()


@dataclass
class DecodeWorkload:
    """Paged decode workload: shapes plus seeded arrays (numpy, host)."""
    name: str
    wid: int
    B: int
    hq: int
    hk: int
    d: int
    block_size: int
    num_splits: int
    seq_lens: np.ndarray
    num_blocks: int
    max_blocks: int
    block_table: np.ndarray          # [B, max_blocks] int32
    slot_mapping: np.ndarray         # [T] int64, tokens of all sequences in order
    kv_dtype: str = "bf16"
    extra: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def _page_tables(wid, B, seq_lens, block_size, max_blocks, num_blocks=None):
    pages_per = [(int(s) + block_size - 1) // block_size for s in seq_lens]
    need = sum(pages_per)
    nb = need if num_blocks is None else num_blocks
    assert nb >= need
    perm = rng(wid, 2).permutation(nb).astype(np.int32)
    bt = np.zeros((B, max_blocks), np.int32)
    slots = []
    pos = 0
    for b in range(B):
        n = pages_per[b]
        assert n <= max_blocks
        bt[b, :n] = perm[pos:pos + n]
        pos += n
        t = np.arange(int(seq_lens[b]), dtype=np.int64)
        slots.append(bt[b, t // block_size].astype(np.int64) * block_size + t % block_size)
    slot_mapping = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return nb, bt, slot_mapping


def decode_workload(name: str, d: int = 128) -> DecodeWorkload:
    """Shapes of the INT4 and TurboQuant decode workloads.

    tiny_int4      B=2 Hq=4 Hk=1 D=64 bs=16 seq {37,100}, 32-page pool, S=4, f16 K/V
    llama8b_int4   B=32 Hq=32 Hk=8 D=128 bs=16 seq ~ U{1024..8192}, S=8, bf16 K/V
    llama8b_int4_8k  as above with every seq_len = 8192
    long_int4      B=1 Hq=64 Hk=8 D=128 bs=64 seq 131072, S=64
    tq_mixed       B=16 Hq=32 Hk=4 D=128 bs=16 seq 16384, S=32 (d selects
                   another head dimension for the same shape)
    """
    if name == "tiny_int4":
        seq = np.array([37, 100], np.int32)
        # the 32-page pool is split 16/16 over the two block-table rows
        perm = rng(1, 2).permutation(32).astype(np.int32)
        bt = perm.reshape(2, 16).copy()
        slots = []
        for b in range(2):
            t = np.arange(int(seq[b]), dtype=np.int64)
            slots.append(bt[b, t // 16].astype(np.int64) * 16 + t % 16)
        return DecodeWorkload(name, 1, 2, 4, 1, 64, 16, 4, seq, 32, 16, bt,
                              np.concatenate(slots), kv_dtype="f16")
    if name in ("llama8b_int4", "llama8b_int4_8k"):
        B = 32
        if name == "llama8b_int4":
            seq = rng(2, 1).integers(1024, 8192, size=B, endpoint=True).astype(np.int32)
        else:
            seq = np.full(B, 8192, np.int32)
        nb, bt, sm = _page_tables(2, B, seq, 16, 512)
        return DecodeWorkload(name, 2, B, 32, 8, 128, 16, 8, seq, nb, 512, bt, sm)
    if name == "long_int4":
        seq = np.array([131072], np.int32)
        nb, bt, sm = _page_tables(4, 1, seq, 64, 2048)
        return DecodeWorkload(name, 4, 1, 64, 8, 128, 64, 64, seq, nb, 2048, bt, sm)
    if name == "tq_mixed":
        seq = np.full(16, 16384, np.int32)
        nb, bt, sm = _page_tables(3, 16, seq, 16, 1024)
        return DecodeWorkload(name, 3, 16, 32, 4, d, 16, 32, seq, nb, 1024, bt, sm)
    raise KeyError(name)


def custom_decode_workload(wid, B, hq, hk, d, block_size, num_splits, seq_lens,
                           extra_pages=0, kv_dtype="bf16", max_blocks=None):
    """Small decode workload with explicit shapes (tests). extra_pages adds
    unused pages to the pool so that the permutation scatters the used ones."""
    seq_lens = np.asarray(seq_lens, np.int32)
    need = sum((int(s) + block_size - 1) // block_size for s in seq_lens)
    mb = max_blocks or max(1, max((int(s) + block_size - 1) // block_size for s in seq_lens))
    nb, bt, sm = _page_tables(wid, B, seq_lens, block_size, mb, need + extra_pages)
    return DecodeWorkload(f"custom{wid}", wid, B, hq, hk, d, block_size, num_splits,
                          seq_lens, nb, mb, bt, sm, kv_dtype=kv_dtype)


def kv_source(w: DecodeWorkload, tokens: slice | None = None, outliers: bool | None = None):
    """K and V source rows [T, Hk, D] as storage-dtype bits (uint16) or fp32.

    Values ~ N(0,1) drawn in fp32. For the Llama-shaped workloads each kv
    head gets 4 seeded outlier channels (choice of 4 of D, no replacement)
    scaled by 10 before rounding, in K and in V.
    """
    T = w.total_tokens
    if outliers is None:
        outliers = w.name.startswith("llama8b")
    g = rng(w.wid, 3)
    k = g.standard_normal((T, w.hk, w.d), dtype=np.float32)
    v = g.standard_normal((T, w.hk, w.d), dtype=np.float32)
    if outliers:
        go = rng(w.wid, 4)
        for h in range(w.hk):
            ch = go.choice(w.d, 4, replace=False)
            k[:, h, ch] *= 10.0
            v[:, h, ch] *= 10.0
    if tokens is not None:
        k, v = k[tokens], v[tokens]
    return to_bits(k, w.kv_dtype), to_bits(v, w.kv_dtype)


def query(w: DecodeWorkload, bf16_valued: bool = False) -> np.ndarray:
    """q [B, Hq, D] fp32 ~ N(0,1) (optionally holding bf16-rounded values)."""
    q = rng(w.wid, 5).standard_normal((w.B, w.hq, w.d), dtype=np.float32)
    if bf16_valued:
        q = bits_to_f32(to_bits(q, "bf16"), "bf16")
    return q


def prefill_queries(w: DecodeWorkload, query_lens, bf16_valued: bool = False):
    """Multi-query (prefill) queries over a decode workload whose seq_lens
    count context + query tokens: cu_seqlens_q [B + 1] int32 and q [T, Hq, D]
    fp32 ~ N(0,1), T = sum(query_lens)."""
    ql = np.asarray(query_lens, np.int64)
    assert ql.shape == (w.B,)
    cu = np.zeros(w.B + 1, np.int32)
    cu[1:] = np.cumsum(ql)
    q = rng(w.wid, 6).standard_normal((int(cu[-1]), w.hq, w.d), dtype=np.float32)
    if bf16_valued:
        q = bits_to_f32(to_bits(q, "bf16"), "bf16")
    return cu, q


def sink_values(w: DecodeWorkload, spread: float = 2.0):
    """Per-query-head attention sinks [Hq] fp32 ~ U(-spread, spread)."""
    return rng(w.wid, 7).uniform(-spread, spread, w.hq).astype(np.float32)


def write_workload(num_tokens=65536, hk=8, d=128, block_size=16, skip_frac=0.05,
                   dtype="bf16", wid=5):
    """Cache-write workload: K/V [T, Hk, D], slot_mapping = a seeded
    permutation of 0..T-1 with round(skip_frac*T) seeded entries set to -1;
    the cache holds exactly T slots (T / block_size pages)."""
    g = rng(wid, 1)
    k = g.standard_normal((num_tokens, hk, d), dtype=np.float32)
    v = g.standard_normal((num_tokens, hk, d), dtype=np.float32)
    nb = (num_tokens + block_size - 1) // block_size
    slots = rng(wid, 2).permutation(num_tokens).astype(np.int64)
    n_skip = int(round(skip_frac * num_tokens))
    if n_skip:
        slots[rng(wid, 3).choice(num_tokens, n_skip, replace=False)] = -1
    return dict(key=to_bits(k, dtype), value=to_bits(v, dtype), slot_mapping=slots,
                num_blocks=nb, block_size=block_size, hk=hk, d=d, dtype=dtype)


def fwht_rows(rows=1048576, wid=6):
    """[rows, 128] bf16 bit patterns ~ N(0,1)."""
    x = rng(wid, 1).standard_normal((rows, 128), dtype=np.float32)
    return to_bits(x, "bf16")


def kpool_workload(n_pools=262144, pool_size=4, score_dtype="bf16", block_size=64,
                   mask_frac=0.0, skip_frac=0.0, score_offset=0.0, wid=11):
    """Pooled key-compression workload: slot_k [n, P, 128] bf16 ~ N(0,1);
    slot_score [n, P, 128] ~ N(score_offset, 1) in score_dtype; ape [P, 128]
    f32 ~ N(0, 0.25); loc = a seeded permutation of the n entries of an
    indexer cache of ceil(n / block_size) pages, with round(skip_frac*n)
    seeded entries set to -1; write_mask = None, or True with probability
    1 - mask_frac per pool."""
    g = rng(wid, 1)
    k = g.standard_normal((n_pools, pool_size, 128), dtype=np.float32)
    sc = g.standard_normal((n_pools, pool_size, 128), dtype=np.float32) + np.float32(score_offset)
    ape = (0.5 * rng(wid, 2).standard_normal((pool_size, 128))).astype(np.float32)
    nb = max(1, (n_pools + block_size - 1) // block_size)
    loc = rng(wid, 3).permutation(n_pools).astype(np.int64)
    n_skip = int(round(skip_frac * n_pools))
    if n_skip:
        loc[rng(wid, 4).choice(n_pools, n_skip, replace=False)] = -1
    mask = None
    if mask_frac > 0:
        mask = rng(wid, 5).random(n_pools) >= mask_frac
    return dict(slot_k=to_bits(k, "bf16"), slot_score=to_bits(sc, score_dtype), ape=ape,
                loc=loc, write_mask=mask, num_blocks=nb, block_size=block_size,
                pool_size=pool_size, score_dtype=score_dtype)


def random_tq_fp8_u4_cache(w: DecodeWorkload, slot_bytes: int, wid_tensor=8):
    """Random FP8-key / 4-bit-value TurboQuant slots: key bytes uniform over
    the finite E4M3 codes (0x7F / 0xFF, the NaN codes, are replaced by
    0x7E / 0xFE), uniform value nibbles, fp16 scales of either sign with
    magnitude in [2^-6, 2^0) and fp16 zeros in [-2, 2). For decode inputs
    that do not depend on any writer."""
    g = rng(w.wid, wid_tensor)
    d = w.d
    cache = np.zeros((w.num_blocks, w.block_size, w.hk, slot_bytes), np.uint8)
    keys = g.integers(0, 256, size=cache.shape[:3] + (d,), dtype=np.uint8)
    keys[(keys & 0x7F) == 0x7F] -= 1
    cache[..., :d] = keys
    cache[..., d:d + d // 2] = g.integers(0, 256, size=cache.shape[:3] + (d // 2,), dtype=np.uint8)
    mag = np.exp2(g.uniform(-6, 0, size=cache.shape[:3]))
    sign = np.where(g.random(size=cache.shape[:3]) < 0.25, -1.0, 1.0)
    sc = (sign * mag).astype(np.float16)
    zr = g.uniform(-2, 2, size=cache.shape[:3]).astype(np.float16)
    cache[..., d + d // 2:d + d // 2 + 2] = sc[..., None].view(np.uint8).reshape(cache.shape[:3] + (2,))
    cache[..., d + d // 2 + 2:d + d // 2 + 4] = zr[..., None].view(np.uint8).reshape(cache.shape[:3] + (2,))
    return cache


def random_tq_cache(w: DecodeWorkload, key_fmt: int, val_fmt: int, slot_bytes: int,
                    wid_tensor=10):
    """Random TurboQuant slots of any format (key_fmt 1 FP8 / 2 centroid-3 /
    3 centroid-4, val_fmt 1 U3 / 2 U4 / 3 FP8): uniform bytes, with E4M3 NaN
    codes (0x7F / 0xFF) replaced by 0x7E / 0xFE, fp16 norms in [2^-2, 2^4),
    fp16 value scales of either sign with magnitude in [2^-6, 2^0) and fp16
    zeros in [-2, 2)."""
    g = rng(w.wid, wid_tensor)
    d = w.d
    shp = (w.num_blocks, w.block_size, w.hk)
    cache = g.integers(0, 256, size=shp + (slot_bytes,), dtype=np.uint8)

    def f16_field(off, vals):
        cache[..., off:off + 2] = vals.astype(np.float16)[..., None].view(np.uint8).reshape(shp + (2,))

    if key_fmt == 1:
        kps = d
        keys = cache[..., :d]
        keys[(keys & 0x7F) == 0x7F] -= 1
    else:
        mse = (d * (3 if key_fmt == 2 else 4) + 7) // 8
        kps = mse + 2
        f16_field(mse, np.exp2(g.uniform(-2, 4, size=shp)))
    if val_fmt == 3:
        vals = cache[..., kps:kps + d]
        vals[(vals & 0x7F) == 0x7F] -= 1
    else:
        vdb = (d * (3 if val_fmt == 1 else 4) + 7) // 8
        sign = np.where(g.random(size=shp) < 0.25, -1.0, 1.0)
        f16_field(kps + vdb, sign * np.exp2(g.uniform(-6, 0, size=shp)))
        f16_field(kps + vdb + 2, g.uniform(-2, 2, size=shp))
    return cache


def random_tq_mse3_u3_cache(w: DecodeWorkload, slot_bytes: int, wid_tensor=9):
    """Random 3-bit-centroid-key / 3-bit-value TurboQuant slots: uniform index
    bytes, fp16 norms in [2^-2, 2^4), fp16 value scales of either sign with
    magnitude in [2^-6, 2^0) and fp16 zeros in [-2, 2). For decode inputs
    that do not depend on any writer."""
    g = rng(w.wid, wid_tensor)
    d = w.d
    shp = (w.num_blocks, w.block_size, w.hk)
    cache = np.zeros(shp + (slot_bytes,), np.uint8)
    kb = 3 * d // 8
    cache[..., :kb] = g.integers(0, 256, size=shp + (kb,), dtype=np.uint8)
    nrm = np.exp2(g.uniform(-2, 4, size=shp)).astype(np.float16)
    cache[..., kb:kb + 2] = nrm[..., None].view(np.uint8).reshape(shp + (2,))
    vo = kb + 2
    cache[..., vo:vo + kb] = g.integers(0, 256, size=shp + (kb,), dtype=np.uint8)
    mag = np.exp2(g.uniform(-6, 0, size=shp))
    sign = np.where(g.random(size=shp) < 0.25, -1.0, 1.0)
    sc = (sign * mag).astype(np.float16)
    zr = g.uniform(-2, 2, size=shp).astype(np.float16)
    so = vo + kb
    cache[..., so:so + 2] = sc[..., None].view(np.uint8).reshape(shp + (2,))
    cache[..., so + 2:so + 4] = zr[..., None].view(np.uint8).reshape(shp + (2,))
    return cache


def random_int4_cache(w: DecodeWorkload, wid_tensor=7):
    """Uniformly random INT4 cache bytes plus valid scale words (positive
    normal scales in [2^-4, 2^2) with a random 4-bit zero-point in the low
    mantissa bits). For decode inputs that do not depend on any writer."""
    g = rng(w.wid, wid_tensor)
    shape = (w.num_blocks, w.block_size, w.hk, w.d // 2)
    kc = g.integers(0, 256, size=shape, dtype=np.uint8)
    vc = g.integers(0, 256, size=shape, dtype=np.uint8)
    words = []
    for _ in range(2):
        s = np.exp2(g.uniform(-4, 2, size=shape[:3])).astype(np.float32)
        zp = g.integers(0, 16, size=shape[:3], dtype=np.uint32)
        words.append(((s.view(np.uint32) & np.uint32(0xFFFFFFF0)) | zp).view(np.float32))
    return kc, vc, words[0], words[1]
