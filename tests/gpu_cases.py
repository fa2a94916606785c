"""Shared builders for the GPU parity tests: seeded inputs from the workload
module, caches filled by the CPU oracle (never by the HIP path), and device
copies for the library under test."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

DEV = torch.device("cuda:0")
ATOL = 1e-3   # max |out - oracle|
RTOL_L2 = 1e-4  # ||out - oracle||_2 / ||oracle||_2

DT_CODE = {"f32": oracle.DT_F32, "f16": oracle.DT_F16, "bf16": oracle.DT_BF16}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def src_to_dev(bits, dtype):
    if dtype == "f32":
        return to_dev(bits)
    return to_dev(bits.view(np.int16), TORCH_DT[dtype])


def int4_caches(w: W.DecodeWorkload, kb=None, vb=None):
    """Oracle-written INT4 caches for workload w (host arrays)."""
    if kb is None:
        kb, vb = W.kv_source(w)
    s = W.rht_signs(w.d)
    shape = (w.num_blocks, w.block_size, w.hk, w.d // 2)
    kc = np.zeros(shape, np.uint8)
    vc = np.zeros(shape, np.uint8)
    ks = np.zeros(shape[:3], np.float32)
    vs = np.zeros(shape[:3], np.float32)
    oracle.reshape_and_cache_int4(kb, vb, DT_CODE[w.kv_dtype], w.slot_mapping, s, kc, vc, ks, vs)
    return dict(kc=kc, vc=vc, ks=ks, vs=vs, signs=s, kb=kb, vb=vb)


def gpu_int4_decode(w, q, c, num_splits=None, flags=0, seq_lens=None):
    import quantized_paged_kv_tq_amd as tq
    out, lse = tq.tq_decode_attention(
        to_dev(q), to_dev(w.block_table), to_dev(w.seq_lens if seq_lens is None else seq_lens),
        num_kv_splits=w.num_splits if num_splits is None else num_splits,
        key_cache=to_dev(c["kc"]), value_cache=to_dev(c["vc"]),
        k_scale_cache=to_dev(c["ks"]), v_scale_cache=to_dev(c["vs"]),
        rht_signs=to_dev(c["signs"]), flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, w.d).astype(np.float64), lse.cpu().numpy().ravel()


def assert_close(got, ref, got_lse=None, ref_lse=None, what=""):
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref).max() if got.size else 0.0
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got - ref)
    assert err <= ATOL and rel <= RTOL_L2, "%s: max|err| %.3g rel-L2 %.3g" % (what, err, rel)
    if got_lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), fin), what
        if fin.any():
            assert np.abs(got_lse[fin] - ref_lse[fin]).max() <= 1e-4, what
    return err, rel


def tq_case(w: W.DecodeWorkload, key_fmt, val_fmt, rot_signs=None):
    """Oracle-encoded TurboQuant cache for workload w."""
    kb, vb = W.kv_source(w)
    k = W.bits_to_f32(kb, w.kv_dtype)
    v = W.bits_to_f32(vb, w.kv_dtype)
    sb = oracle.tq_slot_bytes(w.d, key_fmt, val_fmt)
    cache = np.zeros((w.num_blocks, w.block_size, w.hk, sb), np.uint8)
    cen = None
    if key_fmt in (oracle.KEY_MSE3, oracle.KEY_MSE4):
        bits = 3 if key_fmt == oracle.KEY_MSE3 else 4
        cen = (oracle.lloyd_max_gaussian(1 << bits) / np.sqrt(w.d)).astype(np.float32)
    oracle.tq_encode(k, v, key_fmt, val_fmt, cen, rot_signs, w.slot_mapping, cache)
    return cache, cen


def gpu_tq_decode(w, q, cache, cen, key_fmt, val_fmt, rot_signs=None, norm_correction=False,
                  num_splits=None, flags=0, seq_lens=None):
    import quantized_paged_kv_tq_amd as tq
    out, lse = tq.tq_decode_attention(
        to_dev(q), to_dev(w.block_table), to_dev(w.seq_lens if seq_lens is None else seq_lens),
        flags=flags,
        num_kv_splits=w.num_splits if num_splits is None else num_splits,
        kv_cache=to_dev(cache), key_fmt=key_fmt, val_fmt=val_fmt,
        centroids=None if cen is None else to_dev(cen),
        rot_signs=None if rot_signs is None else to_dev(rot_signs),
        norm_correction=norm_correction)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, w.d).astype(np.float64), lse.cpu().numpy().ravel()


def oracle_rows(fn, n_rows, threads=None):
    """Run an oracle decode fn(rows) -> (out [R, D], lse [R]) over all rows
    0..n_rows-1 on a thread pool (the oracle releases the GIL), in chunks;
    returns the concatenated (out, lse)."""
    import concurrent.futures as cf
    import os
    if threads is None:
        try:
            threads = len(os.sched_getaffinity(0))
        except AttributeError:
            threads = os.cpu_count() or 1
        threads = max(1, min(16, threads))
    rows = np.arange(n_rows, dtype=np.int32)
    chunks = [c for c in np.array_split(rows, max(1, min(n_rows, 4 * threads))) if c.size]
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        parts = list(pool.map(fn, chunks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
