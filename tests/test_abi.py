"""C ABI checks that need no GPU: the library loads, exports every function
include/tq.h declares, sizes its tables as documented and rejects invalid
arguments with the documented codes before launching anything."""
import ctypes as C
import os
import re

import pytest

import quantized_paged_kv_tq_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tq.LIB_PATH):
        import quantized_paged_kv_tq_amd.build as b
        b.build(verbose=False)
    return tq.lib()


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert set(names) == {"tq_last_error", "tq_version", "tq_reshape_and_cache_int4",
                          "tq_encode_and_cache", "tq_decode_workspace_bytes", "tq_slot_bytes",
                          "tq_decode_attention", "tq_decode_attention_static",
                          "fwht128_quant_fp8",
                          "tq_kpool_compress_and_write_cache", "tq_prefill_attention_int4",
                          "tq_prefill_workspace_bytes", "tq_full_dequant_kv"}
    raw = C.CDLL(tq.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(tq.SYMBOLS) == set(names)


def test_sizes(L):
    assert L.tq_version() == 2
    assert tq.tq_slot_bytes(128, tq.KEY_FP8, tq.VAL_U4) == 208
    assert tq.tq_slot_bytes(128, tq.KEY_MSE3, tq.VAL_U3) == 112
    assert tq.tq_slot_bytes(128, tq.KEY_INT4, tq.VAL_U4) == -1
    assert tq.tq_slot_bytes(96, tq.KEY_FP8, tq.VAL_U4) == -1
    # per-split partials + the balanced decode's piece slots (2 * nw * Hq rows,
    # (nw = 2048 / (Hk * ceil(g / 4)) workgroups), then B + 1 prefix sums
    # padded to 4 words
    assert tq.tq_decode_workspace_bytes(32, 32, 8, 128, 8) == \
        ((32 * 32 * 8 + 2 * 256 * 32) * 129 + 36) * 4
    assert tq.tq_decode_workspace_bytes(2, 4, 1, 64, 4) == ((2 * 4 * 4 + 2 * 2048 * 4) * 65 + 4) * 4
    assert tq.tq_decode_workspace_bytes(1, 64, 8, 128, 64) == ((64 * 64 + 2 * 128 * 64) * 129 + 4) * 4
    assert tq.tq_decode_workspace_bytes(2, 4, 0, 64, 4) == 0


def test_decode_args_layout_matches_header(tmp_path):
    """ctypes' view of tq_decode_args has the C compiler's offsets."""
    fields = [f[0] for f in tq.DecodeArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "tq.h"\nint main(void){\n'
                   + "".join('printf("%%zu\\n", offsetof(tq_decode_args, %s));\n' % f for f in fields)
                   + 'printf("%zu\\n", sizeof(tq_decode_args));return 0;}\n')
    exe = tmp_path / "layout"
    import subprocess
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    want = [getattr(tq.DecodeArgs, f).offset for f in fields] + [C.sizeof(tq.DecodeArgs)]
    assert got == want


def _args(**kw):
    a = tq.DecodeArgs()
    a.struct_size = C.sizeof(tq.DecodeArgs)
    a.B, a.Hq, a.Hk, a.D = 2, 4, 1, 64
    a.block_size, a.max_blocks, a.num_kv_splits, a.num_blocks = 16, 16, 4, 32
    a.key_fmt, a.val_fmt = tq.KEY_INT4, tq.VAL_INT4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(D=63), tq.TQ_EINVAL),
    (dict(D=96), tq.TQ_EINVAL),
    (dict(D=256), tq.TQ_ENOTSUP),
    (dict(Hq=6, Hk=4), tq.TQ_EINVAL),
    (dict(Hq=130, Hk=2), tq.TQ_ENOTSUP),
    (dict(num_kv_splits=0), tq.TQ_EINVAL),
    (dict(num_kv_splits=257), tq.TQ_EINVAL),
    (dict(block_size=0), tq.TQ_EINVAL),
    (dict(key_fmt=tq.KEY_INT4, val_fmt=tq.VAL_U4), tq.TQ_ENOTSUP),
    (dict(key_fmt=7), tq.TQ_ENOTSUP),
    (dict(struct_size=8), tq.TQ_EINVAL),
    (dict(), tq.TQ_EINVAL),  # null device pointers
])
def test_decode_rejects_invalid(L, kw, code):
    a = _args(**kw)
    assert L.tq_decode_attention(C.byref(a), None) == code
    assert tq.last_error() != ""


def test_decode_rejects_small_workspace(L):
    need = tq.tq_decode_workspace_bytes(2, 4, 1, 64, 4)
    kw = dict(query=16, block_table=16, seq_lens=16, workspace=16, out=16, key_cache=16,
              value_cache=16, k_scale_cache=16, v_scale_cache=16, rht_signs=16)
    a = _args(workspace_bytes=need - 4, **kw)
    assert L.tq_decode_attention(C.byref(a), None) == tq.TQ_EINVAL
    assert "workspace_bytes" in tq.last_error()


def test_decode_null_args_and_empty_batch(L):
    assert L.tq_decode_attention(None, None) == tq.TQ_EINVAL
    assert L.tq_decode_attention(C.byref(_args(B=0)), None) == tq.TQ_OK
    assert tq.last_error() == ""


def test_tq_format_checks(L):
    a = _args(key_fmt=tq.KEY_FP8, val_fmt=tq.VAL_U4, D=128, query=16, block_table=16,
              seq_lens=16, workspace=16, out=16, kv_cache=16, slot_bytes=192)
    assert L.tq_decode_attention(C.byref(a), None) == tq.TQ_EINVAL  # slot too small
    a = _args(key_fmt=tq.KEY_MSE3, val_fmt=tq.VAL_U3, D=128, query=16, block_table=16,
              seq_lens=16, workspace=16, out=16, kv_cache=16, slot_bytes=112)
    assert L.tq_decode_attention(C.byref(a), None) == tq.TQ_EINVAL  # no centroids


def test_writer_and_fwht_validation(L):
    f = L.tq_reshape_and_cache_int4
    assert f(None, None, 0, 0, 8, 128, None, None, None, None, None, None, 4, 16, None) == tq.TQ_OK
    assert f(None, None, 0, 5, 8, 128, None, None, None, None, None, None, 4, 16, None) == tq.TQ_EINVAL
    assert f(None, None, 0, 5, 8, 96, None, None, None, None, None, None, 4, 16, None) == tq.TQ_EINVAL
    assert f(None, None, 0, 5, 8, 32, None, None, None, None, None, None, 4, 16, None) == tq.TQ_ENOTSUP
    assert f(None, None, 9, 5, 8, 128, None, None, None, None, None, None, 4, 16, None) == tq.TQ_ENOTSUP
    assert f(None, None, 0, -1, 8, 128, None, None, None, None, None, None, 4, 16, None) == tq.TQ_EINVAL
    g = L.fwht128_quant_fp8
    assert g(None, 0, None, None, None) == tq.TQ_OK
    assert g(None, 3, None, None, None) == tq.TQ_EINVAL
    assert g(None, -3, None, None, None) == tq.TQ_EINVAL
    assert g(16, 3, 17, 16, None) == tq.TQ_EINVAL  # misaligned output


def test_binding_requires_library(monkeypatch):
    monkeypatch.setattr(tq, "_lib", None)
    monkeypatch.setattr(tq, "LIB_PATH", "/nonexistent/libtq_amd.so")
    with pytest.raises(ImportError):
        tq.lib()


def test_tq_writer_validation(L):
    f = L.tq_encode_and_cache
    # key, value, dtype, T, Hk, D, key_fmt, val_fmt, slots, centroids, rot_signs, cache,
    # slot_bytes, num_blocks, block_size, stream
    ok = (tq.DTYPE_BF16, 0, 8, 128, tq.KEY_FP8, tq.VAL_U4)
    assert f(None, None, *ok, None, None, None, None, 208, 4, 16, None) == tq.TQ_OK
    assert tq.last_error() == ""
    assert f(None, None, tq.DTYPE_BF16, 5, 8, 128, tq.KEY_FP8, tq.VAL_U4, None, None, None, None,
             208, 4, 16, None) == tq.TQ_EINVAL  # null pointers
    assert f(None, None, tq.DTYPE_BF16, 0, 8, 128, tq.KEY_FP8, tq.VAL_U4, None, None, None, None,
             192, 4, 16, None) == tq.TQ_EINVAL  # slot too small
    assert f(None, None, tq.DTYPE_BF16, 0, 8, 128, tq.KEY_FP8, tq.VAL_U4, None, None, None, None,
             216, 4, 16, None) == tq.TQ_EINVAL  # not a multiple of 16
    assert f(None, None, tq.DTYPE_BF16, 0, 8, 128, tq.KEY_INT4, tq.VAL_U4, None, None, None, None,
             208, 4, 16, None) == tq.TQ_EINVAL  # INT4 is not a combined-slot format
    assert f(None, None, tq.DTYPE_BF16, 0, 8, 96, tq.KEY_FP8, tq.VAL_U4, None, None, None, None,
             208, 4, 16, None) == tq.TQ_ENOTSUP
    assert f(None, None, 7, 0, 8, 128, tq.KEY_FP8, tq.VAL_U4, None, None, None, None,
             208, 4, 16, None) == tq.TQ_ENOTSUP
    assert f(16, 16, tq.DTYPE_BF16, 5, 8, 128, tq.KEY_MSE3, tq.VAL_U3, 16, None, None, 16,
             112, 4, 16, None) == tq.TQ_EINVAL  # centroid keys need the table
    assert f(16, 16, tq.DTYPE_BF16, 5, 8, 128, tq.KEY_FP8, tq.VAL_U4, 16, None, None, 8,
             208, 4, 16, None) == tq.TQ_EINVAL  # misaligned cache
    assert "kv_cache" in tq.last_error()


def test_tq_slot_bytes_match_the_oracle():
    """The library's slot sizes equal the oracle's for every TurboQuant key
    and value format (FP8 values included) at D = 64, 128, 256."""
    import oracle
    for d in (64, 128, 256):
        for kf in (tq.KEY_FP8, tq.KEY_MSE3, tq.KEY_MSE4):
            for vf in (tq.VAL_U3, tq.VAL_U4, tq.VAL_FP8):
                assert tq.tq_slot_bytes(d, kf, vf) == oracle.tq_slot_bytes(d, kf, vf), (d, kf, vf)
    assert tq.tq_slot_bytes(128, tq.KEY_FP8, 4) == -1


def test_kpool_validation(L):
    f = L.tq_kpool_compress_and_write_cache
    # (slot_k, slot_score, score_dtype, ape, loc, write_mask, n_pools, pool_size, head_dim,
    #  kv_cache, num_blocks, block_size, round_scale, compressed_k, compressed_scale, stream)
    ok = dict(sk=16, ss=16, dt=tq.DTYPE_BF16, ape=16, loc=16, wm=None, n=5, P=4, hd=128,
              kc=16, nb=4, bs=64, rs=1, ck=None, cs=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["sk"], a["ss"], a["dt"], a["ape"], a["loc"], a["wm"], a["n"], a["P"], a["hd"],
                 a["kc"], a["nb"], a["bs"], a["rs"], a["ck"], a["cs"], None)

    assert call(n=0) == tq.TQ_OK and tq.last_error() == ""
    assert call(hd=64) == tq.TQ_ENOTSUP
    assert call(P=0) == tq.TQ_EINVAL
    assert call(n=-1) == tq.TQ_EINVAL
    assert call(dt=7) == tq.TQ_EINVAL
    assert call(kc=None) == tq.TQ_EINVAL                    # no output at all
    assert call(kc=None, ck=16) == tq.TQ_EINVAL             # compressed_scale missing
    assert call(kc=None, ck=16, cs=16, wm=16) == tq.TQ_EINVAL  # mask with compressed output
    assert call(loc=None) == tq.TQ_EINVAL                   # cache without locations
    assert call(bs=0) == tq.TQ_EINVAL
    assert call(sk=None) == tq.TQ_EINVAL
    assert call(sk=8) == tq.TQ_EINVAL                       # misaligned
    assert call(kc=None, ck=4, cs=16) == tq.TQ_EINVAL       # misaligned compressed_k
    assert tq.last_error() != ""


def test_prefill_args_layout_matches_header(tmp_path):
    fields = [f[0] for f in tq.PrefillArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "tq.h"\nint main(void){\n'
                   + "".join('printf("%%zu\\n", offsetof(tq_prefill_args, %s));\n' % f for f in fields)
                   + 'printf("%zu\\n", sizeof(tq_prefill_args));return 0;}\n')
    exe = tmp_path / "layout"
    import subprocess
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    want = [getattr(tq.PrefillArgs, f).offset for f in fields] + [C.sizeof(tq.PrefillArgs)]
    assert got == want


def _pargs(**kw):
    a = tq.PrefillArgs()
    a.struct_size = C.sizeof(tq.PrefillArgs)
    a.num_seqs, a.Hq, a.Hk, a.D = 2, 8, 2, 128
    a.block_size, a.max_blocks, a.num_tokens, a.num_blocks = 16, 8, 10, 32
    a.sm_scale = 0.088
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), tq.TQ_ENOTSUP),
    (dict(D=256), tq.TQ_ENOTSUP),
    (dict(Hq=6, Hk=4), tq.TQ_EINVAL),
    (dict(Hk=0), tq.TQ_EINVAL),
    (dict(block_size=0), tq.TQ_EINVAL),
    (dict(window=-1), tq.TQ_EINVAL),
    (dict(softcap=-1.0), tq.TQ_EINVAL),
    (dict(softcap=float("nan")), tq.TQ_EINVAL),
    (dict(num_seqs=0), tq.TQ_EINVAL),
    (dict(struct_size=8), tq.TQ_EINVAL),
    (dict(), tq.TQ_EINVAL),  # null device pointers
])
def test_prefill_rejects_invalid(L, kw, code):
    a = _pargs(**kw)
    assert L.tq_prefill_attention_int4(C.byref(a), None) == code
    assert tq.last_error() != ""


def test_prefill_empty_and_null(L):
    assert L.tq_prefill_attention_int4(None, None) == tq.TQ_EINVAL
    assert L.tq_prefill_attention_int4(C.byref(_pargs(num_tokens=0)), None) == tq.TQ_OK
    assert tq.last_error() == ""
    # the layout before the workspace fields is still accepted
    old = C.sizeof(tq.PrefillArgs) - 16
    assert tq.PrefillArgs.workspace.offset == old
    assert L.tq_prefill_attention_int4(C.byref(_pargs(num_tokens=0, struct_size=old)), None) == tq.TQ_OK
    assert L.tq_prefill_attention_int4(C.byref(_pargs(struct_size=old - 8)), None) == tq.TQ_EINVAL


def test_prefill_workspace_bytes(L):
    # a plan of three int32 per token of a chunk (256-byte aligned), then the
    # decode workspace of one chunk with one split per entry
    def plan(n):
        return (n * 12 + 255) // 256 * 256
    assert tq.tq_prefill_workspace_bytes(10, 32, 8, 128) == \
        plan(10) + tq.tq_decode_workspace_bytes(10, 32, 8, 128, 1)
    # chunks of at most 4096 tokens
    assert tq.tq_prefill_workspace_bytes(10000, 8, 2, 128) == \
        plan(4096) + tq.tq_decode_workspace_bytes(4096, 8, 2, 128, 1)
    # no matrix-core path: D != 128, g > 32, no tokens
    assert tq.tq_prefill_workspace_bytes(10, 8, 2, 64) == 0
    assert tq.tq_prefill_workspace_bytes(10, 66, 2, 128) == 0
    assert tq.tq_prefill_workspace_bytes(10, 18, 2, 128) > 0
    assert tq.tq_prefill_workspace_bytes(0, 8, 2, 128) == 0


def test_full_dequant_validation(L):
    f = L.tq_full_dequant_kv
    # (kv, bt, max_blocks, cen, B, Hk, D, bs, nb, slot_bytes, key_fmt, val_fmt, nc, max_seq, k, v, stream)
    ok = dict(kv=16, bt=16, mb=4, cen=16, B=2, hk=2, D=128, bs=16, nb=8, sb=208, kf=tq.KEY_FP8,
              vf=tq.VAL_U4, nc=0, ms=64, k=16, v=16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["kv"], a["bt"], a["mb"], a["cen"], a["B"], a["hk"], a["D"], a["bs"], a["nb"],
                 a["sb"], a["kf"], a["vf"], a["nc"], a["ms"], a["k"], a["v"], None)

    assert call(ms=0) == tq.TQ_OK and tq.last_error() == ""
    assert call(D=96) == tq.TQ_ENOTSUP
    assert call(kf=tq.KEY_INT4, vf=tq.VAL_INT4) == tq.TQ_ENOTSUP
    assert call(sb=192) == tq.TQ_EINVAL          # smaller than the slot
    assert call(sb=216) == tq.TQ_EINVAL          # not a multiple of 16
    assert call(ms=65) == tq.TQ_EINVAL           # beyond max_blocks * block_size
    assert call(kf=tq.KEY_MSE3, vf=tq.VAL_U3, sb=112, cen=None) == tq.TQ_EINVAL
    assert call(kv=None) == tq.TQ_EINVAL
    assert call(k=8) == tq.TQ_EINVAL             # misaligned output


def test_static_decode_size_limit_and_empty_batch(L):
    """The static-workspace entry point rejects a call whose workspace would
    exceed its fixed maximum (before touching any GPU) and returns TQ_OK for
    an empty batch."""
    B, hq, hk, d, S = 4096, 64, 8, 128, 64
    assert tq.tq_decode_workspace_bytes(B, hq, hk, d, S) > 64 << 20
    a = _args(B=B, Hq=hq, Hk=hk, D=d, num_kv_splits=S)
    assert L.tq_decode_attention_static(C.byref(a), None) == tq.TQ_EINVAL
    assert "static maximum" in tq.last_error()
    assert L.tq_decode_attention_static(None, None) == tq.TQ_EINVAL
    assert L.tq_decode_attention_static(C.byref(_args(B=0)), None) == tq.TQ_OK
