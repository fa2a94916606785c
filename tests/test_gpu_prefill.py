"""GPU parity of the INT4 multi-query (prefill) attention against the fp64
oracle (int4_per_token_head.py, _attn_packed in its 2D mode), through the C
ABI: causal ranges from the context length, sliding windows, softcap, sinks,
GQA 1-8, D = 64 and 128, fp32 and FP8 output."""
import numpy as np
import pytest
import torch

import oracle
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import ATOL, RTOL_L2, int4_caches, to_dev

pytestmark = pytest.mark.gpu


def _case(wid, B, hq, hk, d, bs, ctx, qlen, extra_pages=3):
    seq = np.asarray(ctx) + np.asarray(qlen)
    w = W.custom_decode_workload(wid, B, hq, hk, d, bs, 1, seq, extra_pages=extra_pages)
    c = int4_caches(w)
    cu, q = W.prefill_queries(w, qlen)
    return w, c, cu, q


# "auto": the matrix-core path where it applies (D = 128, g <= 8); None: the
# vector kernel
PATHS = pytest.mark.parametrize("path", ["auto", None], ids=["mfma", "valu"])


def _gpu(w, c, cu, q, window=0, softcap=0.0, sinks=None, output_scale=None, path="auto"):
    import quantized_paged_kv_tq_amd as tq
    out = tq.tq_prefill_attention_int4(
        to_dev(q), to_dev(c["kc"]), to_dev(c["vc"]), to_dev(w.block_table), to_dev(cu),
        to_dev(w.seq_lens), k_scale_cache=to_dev(c["ks"]), v_scale_cache=to_dev(c["vs"]),
        rht_signs=to_dev(c["signs"]), sm_scale=w.sm_scale, window=window, softcap=softcap,
        sinks=None if sinks is None else to_dev(sinks),
        output_scale=None if output_scale is None else to_dev(np.array([output_scale], np.float32)),
        workspace=path)
    torch.cuda.synchronize()
    return out


def _check(w, c, cu, q, path="auto", **kw):
    print("prefill case: B=%d Hq=%d Hk=%d D=%d bs=%d seq=%s q=%s %s path=%s" % (
        w.B, w.hq, w.hk, w.d, w.block_size, list(w.seq_lens), list(np.diff(cu)), kw, path),
        flush=True)
    want = oracle.int4_prefill(q, c["kc"], c["vc"], c["ks"], c["vs"], w.block_table, cu,
                               w.seq_lens, c["signs"], w.sm_scale, **kw)
    got = _gpu(w, c, cu, q, path=path, **kw).cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    assert err.max() <= ATOL, err.max()
    nrm = np.linalg.norm(want)
    if nrm > 0:
        assert np.linalg.norm(got - want) / nrm <= RTOL_L2


@pytest.mark.parametrize("window,softcap,sinks", [(0, 0.0, False), (5, 0.0, False),
                                                  (0, 3.0, False), (0, 0.0, True),
                                                  (7, 2.5, True)])
@pytest.mark.parametrize("d", [64, 128])
@PATHS
def test_tiny_features(window, softcap, sinks, d, path):
    w, c, cu, q = _case(201, 3, 4, 2, d, 16, ctx=[0, 13, 40], qlen=[9, 5, 1])
    _check(w, c, cu, q, path=path, window=window, softcap=softcap,
           sinks=W.sink_values(w) if sinks else None)


@pytest.mark.parametrize("hq,hk", [(32, 8), (16, 2), (8, 8), (12, 2), (6, 3), (32, 2), (40, 2)])
@PATHS
def test_gqa_d128(hq, hk, path):
    w, c, cu, q = _case(202 + hq + hk, 3, hq, hk, 128, 16, ctx=[100, 0, 300], qlen=[40, 70, 3])
    _check(w, c, cu, q, path=path)
    _check(w, c, cu, q, path=path, window=33, softcap=30.0, sinks=W.sink_values(w))


@PATHS
def test_empty_sequences_and_block_64(path):
    w, c, cu, q = _case(210, 4, 8, 2, 128, 64, ctx=[0, 70, 5, 0], qlen=[17, 0, 0, 65])
    _check(w, c, cu, q, path=path, window=20)


def test_long_context_unstaged_block_table():
    # 33,000 context tokens at bs 16: more pages than the LDS staging holds
    w, c, cu, q = _case(211, 2, 8, 2, 64, 16, ctx=[33000, 50], qlen=[2, 3], extra_pages=0)
    _check(w, c, cu, q)
    _check(w, c, cu, q, window=4096, sinks=W.sink_values(w))


@pytest.mark.parametrize("scale", [0.02, 0.25])
@PATHS
def test_fp8_output_within_one_step(scale, path):
    w, c, cu, q = _case(212, 3, 16, 4, 128, 16, ctx=[64, 0, 200], qlen=[30, 20, 4])
    want = oracle.int4_prefill(q, c["kc"], c["vc"], c["ks"], c["vs"], w.block_table, cu,
                               w.seq_lens, c["signs"], w.sm_scale, softcap=20.0)
    got = _gpu(w, c, cu, q, softcap=20.0, output_scale=scale, path=path)
    dec = got.float().cpu().numpy().astype(np.float64)
    inv = float(np.float32(1.0) / np.float32(scale))
    v = np.clip(want * inv, -448, 448)
    # the code must be one of the E4M3 values bracketing [v - tol, v + tol]
    grid = np.unique(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy())
    grid = grid[np.isfinite(grid)].astype(np.float64)
    tol = ATOL * inv
    lo = grid[np.clip(np.searchsorted(grid, v - tol, side="right") - 1, 0, len(grid) - 1)]
    hi = grid[np.clip(np.searchsorted(grid, v + tol, side="left"), 0, len(grid) - 1)]
    assert np.all((dec >= lo) & (dec <= hi))


@pytest.mark.parametrize("window,sinks", [(0, False), (50, True)])
@PATHS
def test_wide_score_range(window, sinks, path):
    """Queries scaled by 40: scores spread over tens of units, so each lane
    group's reference maximum moves many times along the visible range (and
    the sink, when present, sits far below or far above it)."""
    w, c, cu, q = _case(213, 2, 8, 2, 128, 16, ctx=[400, 37], qlen=[60, 9])
    _check(w, c, cu, q * 40.0, path=path, window=window, sinks=W.sink_values(w) if sinks else None)


def test_matrix_core_path_chunks_past_4096_tokens():
    """4,200 query tokens: the matrix-core path runs them as two chunks of
    decode entries (4,096 + 104) through one workspace."""
    import quantized_paged_kv_tq_amd as tq
    assert tq.tq_prefill_workspace_bytes(4200, 2, 1, 128) > 0
    w, c, cu, q = _case(214, 2, 2, 1, 128, 16, ctx=[30, 0], qlen=[2100, 2100])
    _check(w, c, cu, q, path="auto", window=700, sinks=W.sink_values(w))
