"""Pins of the oracle's INT4 multi-query ("2D", prefill) attention
(int4_per_token_head.py, _attn_packed in 2D mode as unified_attention_int4
wraps it): causal visibility from the context length, the sliding window,
softcap and sinks.

- A query that is the last token of its sequence reduces to the decode
  oracle (pinned in test_oracle_attention.py).
- Brute force on tiny inputs: every cache row dequantized by the pinned row
  decoder, the query rotated with scipy's Hadamard matrix, masks, softcap
  (numpy tanh), sinks and the softmax written as dense NumPy.
- Closed forms: a window of 1 returns the unrotated dequantized value row of
  the query's own position; changing keys after a query's position does not
  change its output.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from quantized_paged_kv_tq_amd import workloads as W

from gpu_cases import int4_caches


def _setup(wid, B, hq, hk, d, bs, ctx, qlen, extra_pages=3):
    seq = np.asarray(ctx) + np.asarray(qlen)
    w = W.custom_decode_workload(wid, B, hq, hk, d, bs, 1, seq, extra_pages=extra_pages)
    c = int4_caches(w)
    cu, q = W.prefill_queries(w, qlen)
    return w, c, cu, q


def _run(w, c, cu, q, **kw):
    return oracle.int4_prefill(q, c["kc"], c["vc"], c["ks"], c["vs"], w.block_table, cu,
                               w.seq_lens, c["signs"], w.sm_scale, **kw)


def _brute(w, c, cu, q, window=0, softcap=0.0, sinks=None):
    d, hq, hk, bs = w.d, w.hq, w.hk, w.block_size
    H = scipy.linalg.hadamard(d).astype(np.float64)
    s = c["signs"].astype(np.float64)
    nb = w.num_blocks
    K = np.zeros((nb, bs, hk, d))
    V = np.zeros((nb, bs, hk, d))
    for blk in range(nb):
        for off in range(bs):
            for h in range(hk):
                K[blk, off, h] = oracle.int4_dequant_row(c["kc"][blk, off, h], c["ks"][blk, off, h], d)
                V[blk, off, h] = oracle.int4_dequant_row(c["vc"][blk, off, h], c["vs"][blk, off, h], d)
    qr = (q.astype(np.float64) * s) @ H.T
    out = np.zeros(q.shape)
    g = hq // hk
    for b in range(w.B):
        ql = int(cu[b + 1] - cu[b])
        seq = int(w.seq_lens[b])
        t = np.arange(seq)
        pages = w.block_table[b, t // bs]
        for i in range(ql):
            pos = seq - ql + i
            vis = t <= pos
            if window > 0:
                vis &= (pos - t) < window
            for h in range(hq):
                kk = K[pages, t % bs, h // g][vis]
                vv = V[pages, t % bs, h // g][vis]
                if kk.shape[0] == 0:
                    continue
                sc = (w.sm_scale / d) * (kk @ qr[cu[b] + i, h])
                if softcap > 0:
                    sc = softcap * np.tanh(sc / softcap)
                logits = sc if sinks is None else np.append(sc, sinks[h])
                p = np.exp(logits - logits.max())
                o = (p[:kk.shape[0]] @ vv) / p.sum()
                out[cu[b] + i, h] = (o @ H.T) * s / d
    return out


@pytest.mark.parametrize("window,softcap,sinks", [(0, 0.0, False), (5, 0.0, False),
                                                  (0, 3.0, False), (0, 0.0, True),
                                                  (7, 2.5, True)])
def test_brute_force_tiny(window, softcap, sinks):
    w, c, cu, q = _setup(101, 3, 4, 2, 64, 16, ctx=[0, 13, 40], qlen=[9, 5, 1])
    sk = W.sink_values(w) if sinks else None
    got = _run(w, c, cu, q, window=window, softcap=softcap, sinks=sk)
    want = _brute(w, c, cu, q, window=window, softcap=softcap, sinks=sk)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_last_query_token_is_decode():
    w, c, cu, q = _setup(102, 3, 8, 2, 128, 16, ctx=[30, 0, 77], qlen=[4, 6, 2])
    got = _run(w, c, cu, q)
    last = cu[1:] - 1
    dec, _ = oracle.int4_decode(q[last], c["kc"], c["vc"], c["ks"], c["vs"], w.block_table,
                                w.seq_lens, c["signs"], 0, w.sm_scale)
    np.testing.assert_allclose(got[last].reshape(-1, w.d), dec, rtol=0, atol=1e-13)
    dec3, _ = oracle.int4_decode(q[last], c["kc"], c["vc"], c["ks"], c["vs"], w.block_table,
                                 w.seq_lens, c["signs"], 3, w.sm_scale)
    np.testing.assert_allclose(got[last].reshape(-1, w.d), dec3, rtol=0, atol=1e-12)


def test_window_of_one_returns_own_value_row():
    w, c, cu, q = _setup(103, 2, 4, 1, 64, 16, ctx=[20, 3], qlen=[6, 4])
    got = _run(w, c, cu, q, window=1)
    H = scipy.linalg.hadamard(w.d).astype(np.float64)
    s = c["signs"].astype(np.float64)
    for b in range(w.B):
        ql = int(cu[b + 1] - cu[b])
        for i in range(ql):
            pos = int(w.seq_lens[b]) - ql + i
            blk, off = w.block_table[b, pos // w.block_size], pos % w.block_size
            v = oracle.int4_dequant_row(c["vc"][blk, off, 0], c["vs"][blk, off, 0], w.d)
            want = (v @ H.T) * s / w.d
            for h in range(w.hq):
                np.testing.assert_allclose(got[cu[b] + i, h], want, rtol=0, atol=1e-13)


def test_causality_and_empty_sequences():
    w, c, cu, q = _setup(104, 3, 4, 2, 64, 16, ctx=[10, 5, 0], qlen=[6, 0, 3])
    base = _run(w, c, cu, q, window=4, softcap=5.0)
    # perturb every key and value after position ctx + 2 of sequence 0
    b, ql = 0, 6
    seq = int(w.seq_lens[b])
    c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    for t in range(seq - ql + 3, seq):
        blk, off = w.block_table[b, t // w.block_size], t % w.block_size
        c2["kc"][blk, off] ^= 0x5A
        c2["vc"][blk, off] ^= 0xA5
    pert = _run(w, c2, cu, q, window=4, softcap=5.0)
    np.testing.assert_array_equal(pert[:3], base[:3])        # positions ctx .. ctx + 2
    assert np.abs(pert[3:6] - base[3:6]).max() > 1e-3        # later queries see the change
    np.testing.assert_array_equal(pert[6:], base[6:])        # other sequences


def test_sink_limits():
    w, c, cu, q = _setup(105, 2, 4, 2, 64, 16, ctx=[12, 30], qlen=[3, 2])
    base = _run(w, c, cu, q)
    np.testing.assert_allclose(_run(w, c, cu, q, sinks=np.full(w.hq, -1e4, np.float32)), base,
                               rtol=0, atol=1e-15)
    tiny = _run(w, c, cu, q, sinks=np.full(w.hq, 200.0, np.float32))
    assert np.abs(tiny).max() < 1e-60
    np.testing.assert_allclose(_run(w, c, cu, q, softcap=1e9), base, rtol=0, atol=1e-12)
