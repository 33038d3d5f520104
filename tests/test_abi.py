"""The C ABI on the CPU: the library loads, exports every entry point that
include/inkattn.h declares, and rejects bad arguments on the host before any
HIP call.  No kernel is launched here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "inkattn.h")

ink = pytest.importorskip("attention_sconv_amd")

FAKE = 0x100000          # aligned non-NULL pointer; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(inkattn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(ink.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ink.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert ink.status_string(0) == "ok"
    assert "invalid" in ink.status_string(1)
    assert "unsupported" in ink.status_string(2)
    assert "HIP" in ink.status_string(3)
    assert "scratch" in ink.status_string(4)
    assert ink.status_string(99) == "unknown status"


def _sconv(**kw):
    args = dict(dtype=1, Hkv=4, d=128, seqs=1, toks=4, maxc=4, k=FAKE, v=FAKE, w=FAKE,
                st=FAKE, slot=FAKE, cu=FAKE, sm=FAKE, kc=FAKE, vc=FAKE)
    args.update(kw)
    return ink._lib._lib.inkattn_sconv(args["dtype"], args["Hkv"], args["d"], args["seqs"],
                                       args["toks"], args["maxc"], args["k"], args["v"],
                                       args["w"], args["st"], args["slot"], args["cu"],
                                       args["sm"], args["kc"], args["vc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), ink.ENOTSUP), (dict(d=64), ink.ENOTSUP), (dict(Hkv=0), ink.EINVAL),
    (dict(Hkv=65), ink.ENOTSUP), (dict(toks=-1), ink.EINVAL), (dict(k=None), ink.EINVAL),
    (dict(kc=None), ink.EINVAL), (dict(k=FAKE + 8), ink.EINVAL),
    (dict(toks=0), ink.OK), (dict(seqs=0), ink.OK),
])
def test_sconv_host_validation(kw, status):
    assert _sconv(**kw) == status


def _desc(**kw):
    a = dict(dtype=1, Hq=32, Hkv=4, d=128, bs=128, W=0, R=64)
    a.update(kw)
    return ink.AttnDesc(a["dtype"], a["Hq"], a["Hkv"], a["d"], a["bs"], a["W"], a["R"])


BAD_DESCS = [
    (dict(dtype=2), ink.ENOTSUP), (dict(d=64), ink.ENOTSUP), (dict(bs=16), ink.ENOTSUP),
    (dict(Hq=30), ink.EINVAL), (dict(Hkv=0), ink.EINVAL), (dict(W=-1), ink.EINVAL),
    (dict(R=0), ink.EINVAL), (dict(Hq=64, Hkv=2), ink.ENOTSUP),
]


@pytest.mark.parametrize("kw,status", BAD_DESCS)
def test_prefill_rejects_bad_desc(kw, status):
    lib = ink._lib._lib
    d = _desc(**kw)
    st = lib.inkattn_relattn_prefill(ctypes.byref(d), 1, 8, 8, FAKE, FAKE, FAKE, FAKE, 1,
                                     FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == status


def test_prefill_rejects_null_and_misaligned():
    lib = ink._lib._lib
    d = _desc()
    assert lib.inkattn_relattn_prefill(None, 1, 8, 8, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE,
                                       FAKE, FAKE, None, None) == ink.EINVAL
    assert lib.inkattn_relattn_prefill(ctypes.byref(d), 1, 8, 8, None, FAKE, FAKE, FAKE, 1,
                                       FAKE, FAKE, FAKE, FAKE, None, None) == ink.EINVAL
    assert lib.inkattn_relattn_prefill(ctypes.byref(d), 1, 8, 8, FAKE + 2, FAKE, FAKE, FAKE,
                                       1, FAKE, FAKE, FAKE, FAKE, None, None) == ink.EINVAL
    assert lib.inkattn_relattn_prefill(ctypes.byref(d), 1, 8, 8, FAKE, FAKE, FAKE, FAKE, 0,
                                       FAKE, FAKE, FAKE, FAKE, None, None) == ink.EINVAL
    # empty work is a no-op, even with NULL pointers
    assert lib.inkattn_relattn_prefill(ctypes.byref(d), 0, 0, 0, None, None, None, None, 1,
                                       None, None, None, None, None, None) == ink.OK


@pytest.mark.parametrize("kw,status", BAD_DESCS)
def test_decode_rejects_bad_desc(kw, status):
    lib = ink._lib._lib
    d = _desc(**kw)
    st = lib.inkattn_relattn_decode(ctypes.byref(d), 1, 100, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                    FAKE, FAKE, None, 0, FAKE, 1 << 30, None)
    assert st == status
    assert ink.inkattn_relattn_decode_workspace_size(d, 1, 100, 0) == 0


def test_decode_workspace_rules():
    d = _desc(W=4096, R=4096)
    B, L = 64, 16384
    s = ink.inkattn_relattn_decode_num_splits(d, B, L)
    need = ink.inkattn_relattn_decode_workspace_size(d, B, L, 0)
    rows = B * 32 * s
    assert need == rows * 128 * 4 + ((rows * 4 + 15) // 16) * 16
    assert ink.inkattn_relattn_decode_workspace_size(d, B, L, 3) == \
        B * 32 * 3 * 128 * 4 + ((B * 32 * 3 * 4 + 15) // 16) * 16
    lib = ink._lib._lib
    st = lib.inkattn_relattn_decode(ctypes.byref(d), B, L, FAKE, FAKE, FAKE, FAKE, 128, FAKE,
                                    FAKE, FAKE, None, 0, FAKE, need - 16, None)
    assert st == ink.EINVAL
    st = lib.inkattn_relattn_decode(ctypes.byref(d), B, L, FAKE, FAKE, FAKE, FAKE, 128, FAKE,
                                    FAKE, FAKE, None, -1, FAKE, need, None)
    assert st == ink.EINVAL
    st = lib.inkattn_relattn_decode(ctypes.byref(d), B, L, FAKE, FAKE, FAKE, FAKE, 128, FAKE,
                                    FAKE, FAKE, None, 0, FAKE + 4, need, None)
    assert st == ink.EINVAL


@pytest.mark.parametrize("kw,status", BAD_DESCS)
def test_decode_noalloc_rejects_bad_desc(kw, status):
    lib = ink._lib._lib
    d = _desc(**kw)
    st = lib.inkattn_relattn_decode_noalloc(ctypes.byref(d), 1, 100, FAKE, FAKE, FAKE, FAKE, 1,
                                            FAKE, FAKE, FAKE, None, 0, None)
    assert st == status


def test_decode_noalloc_rejects_partials_beyond_its_scratch():
    # 64 sequences x 32 heads x 16 splits of partials (16.9 MB) exceed the
    # 8 MiB static scratch: rejected before anything runs; the same call with
    # a workspace of its own is accepted by the host checks of the plain decode
    lib = ink._lib._lib
    d = _desc(W=0, R=1 << 20)
    B, L, S = 64, 1 << 20, 16
    need = ink.inkattn_relattn_decode_workspace_size(d, B, L, S)
    assert need > ink.NOALLOC_SCRATCH_BYTES
    st = lib.inkattn_relattn_decode_noalloc(ctypes.byref(d), B, L, FAKE, FAKE, FAKE, FAKE, 8192,
                                            FAKE, FAKE, FAKE, None, S, None)
    assert st == ink.ESCRATCH
    for bad in (dict(num_splits=-1), dict(num_seqs=-1)):
        args = dict(num_seqs=B, num_splits=S)
        args.update(bad)
        st = lib.inkattn_relattn_decode_noalloc(ctypes.byref(d), args["num_seqs"], L, FAKE, FAKE,
                                                FAKE, FAKE, 8192, FAKE, FAKE, FAKE, None,
                                                args["num_splits"], None)
        assert st == ink.EINVAL
    # misaligned output
    st = lib.inkattn_relattn_decode_noalloc(ctypes.byref(d), 1, L, FAKE, FAKE, FAKE, FAKE, 8192,
                                            FAKE, FAKE, FAKE + 4, None, 4, None)
    assert st == ink.EINVAL
    # nothing to do is a no-op
    assert lib.inkattn_relattn_decode_noalloc(ctypes.byref(d), 0, L, None, None, None, None, 1,
                                              None, None, None, None, 0, None) == ink.OK


def test_num_splits_heuristic():
    # enough (seq, kv-head, split) work-groups for one per compute unit, never
    # more splits than pages in the attended range
    sw = _desc(W=4096, R=4096)
    assert ink.inkattn_relattn_decode_num_splits(sw, 64, 16384) == 1
    assert ink.inkattn_relattn_decode_num_splits(sw, 16, 16384) == 4
    full = _desc(W=0, R=1 << 20)
    assert ink.inkattn_relattn_decode_num_splits(full, 4, 1 << 20) == 16
    assert ink.inkattn_relattn_decode_num_splits(full, 1, 100) == 1
    assert ink.inkattn_relattn_decode_num_splits(full, 1, 300) == 3


def test_prefill_and_decode_reject_bias_table_of_2gib():
    # the kernels address the [Hq][R] bias table with 32-bit byte offsets
    lib = ink._lib._lib
    big = _desc(dtype=1, Hq=32, R=1 << 25)            # 32 * 2^25 * 2 B = 2 GiB
    st = lib.inkattn_relattn_prefill(ctypes.byref(big), 1, 1, 1, FAKE, FAKE, FAKE, FAKE, 1,
                                     FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == ink.ENOTSUP
    big = _desc(dtype=1, Hq=32, R=1 << 25)            # 32 * 2^25 * 2 B = 2 GiB
    st = lib.inkattn_relattn_decode(ctypes.byref(big), 1, 100, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                    FAKE, FAKE, None, 0, FAKE, 1 << 30, None)
    assert st == ink.ENOTSUP
    big32 = _desc(dtype=0, Hq=32, R=1 << 24)          # fp32: 32 * 2^24 * 4 B = 2 GiB
    st = lib.inkattn_relattn_decode(ctypes.byref(big32), 1, 100, FAKE, FAKE, FAKE, FAKE, 1,
                                    FAKE, FAKE, FAKE, None, 0, FAKE, 1 << 30, None)
    assert st == ink.ENOTSUP


def test_probes_reject_bad_arguments():
    lib = ctypes.CDLL(ink.LIB_PATH)
    lib.inkattn_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p]
    lib.inkattn_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                              ctypes.c_void_p]
    assert lib.inkattn_probe_mfma_bf16(0, 10, FAKE, None) == ink.EINVAL
    assert lib.inkattn_probe_mfma_bf16(4, 0, FAKE, None) == ink.EINVAL
    assert lib.inkattn_probe_mfma_bf16(4, 10, None, None) == ink.EINVAL
    assert lib.inkattn_probe_stream_read(None, 1024, FAKE, None) == ink.EINVAL
    assert lib.inkattn_probe_stream_read(FAKE, 0, FAKE, None) == ink.EINVAL
    assert lib.inkattn_probe_stream_read(FAKE + 4, 1024, FAKE, None) == ink.EINVAL
    assert lib.inkattn_probe_stream_read(FAKE, 1000, FAKE, None) == ink.EINVAL
    assert lib.inkattn_probe_stream_read(FAKE, 1024, None, None) == ink.EINVAL


def _decode_mq(desc, **kw):
    args = dict(num_seqs=2, num_tokens=5, max_q_len=4, max_seq_len=100, q=FAKE, k=FAKE, v=FAKE,
                bt=FAKE, mb=4, cu=FAKE, sl=FAKE, bias=FAKE, out=FAKE, lse=None, splits=0,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return ink._lib._lib.inkattn_relattn_decode_mq(
        ctypes.byref(desc), args["num_seqs"], args["num_tokens"], args["max_q_len"],
        args["max_seq_len"], args["q"], args["k"], args["v"], args["bt"], args["mb"],
        args["cu"], args["sl"], args["bias"], args["out"], args["lse"], args["splits"],
        args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(max_q_len=0), 1), (dict(max_q_len=17), 2), (dict(num_tokens=1), 1),
    (dict(cu=None), 1), (dict(q=None), 1), (dict(ws=None), 1), (dict(ws_bytes=16), 1),
    (dict(q=FAKE + 4), 1), (dict(num_seqs=0), 0), (dict(num_tokens=0), 0),
    (dict(num_seqs=1000, num_tokens=2000, splits=1 << 20), 2),     # grid beyond 2^31 groups
])
def test_decode_mq_host_validation(kw, status):
    d = ink.make_desc(ink.BF16, 32, 4, 0, 128)
    assert _decode_mq(d, **kw) == status


def test_decode_mq_splits_and_workspace():
    d = ink.make_desc(ink.BF16, 32, 4, 4096, 4096)
    # one token per sequence: the same heuristic as plain decode
    assert ink.inkattn_relattn_decode_mq_num_splits(d, 64, 1, 16384) == \
        ink.inkattn_relattn_decode_num_splits(d, 64, 16384)
    # bf16, 9 tokens x 8 heads = 5 column tiles of 16, all in one work-group
    # per (split, kv-head, sequence): splits fill the 256 CUs once, capped by
    # the 34 pages a 4096 + 8 key range can touch
    assert ink.inkattn_relattn_decode_mq_num_splits(d, 16, 9, 16384) == 4
    assert ink.inkattn_relattn_decode_mq_num_splits(d, 2, 9, 16384) == 32
    assert ink.inkattn_relattn_decode_mq_num_splits(d, 1, 9, 16384) == 34
    # fp32 keeps one work-group per column tile: 5 tiles, fewer splits
    d32 = ink.make_desc(ink.FP32, 32, 4, 4096, 4096)
    assert ink.inkattn_relattn_decode_mq_num_splits(d32, 16, 9, 16384) == 1
    assert ink.inkattn_relattn_decode_mq_num_splits(d32, 2, 9, 16384) == 7
    n = ink.inkattn_relattn_decode_mq_workspace_size(d, 2, 10, 9, 16384, 3)
    rows = 10 * 32 * 3
    assert n == rows * 128 * 4 + ((rows * 4 + 15) // 16) * 16
    assert ink.inkattn_relattn_decode_mq_workspace_size(d, 2, 10, 17, 16384, 3) == 0


def _sconv_paged(**kw):
    args = dict(dtype=ink.BF16, Hkv=4, d=128, seqs=2, toks=10, maxlen=8, k=FAKE, v=FAKE,
                w=FAKE, cu=FAKE, sl=FAKE, sbt=FAKE, msb=4, ks=FAKE, vs=FAKE, slot=FAKE,
                kc=FAKE, vc=FAKE)
    args.update(kw)
    return ink._lib._lib.inkattn_sconv_paged(
        args["dtype"], args["Hkv"], args["d"], args["seqs"], args["toks"], args["maxlen"],
        args["k"], args["v"], args["w"], args["cu"], args["sl"], args["sbt"], args["msb"],
        args["ks"], args["vs"], args["slot"], args["kc"], args["vc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 2), (dict(d=64), 2), (dict(Hkv=0), 1), (dict(Hkv=65), 2),
    (dict(seqs=-1), 1), (dict(seqs=0), 0), (dict(toks=0), 0), (dict(msb=0), 1),
    (dict(sl=None), 1), (dict(sbt=None), 1), (dict(ks=None), 1), (dict(vs=None), 1),
    (dict(ks=FAKE + 8), 1), (dict(kc=None), 1),
])
def test_sconv_paged_host_validation(kw, status):
    assert _sconv_paged(**kw) == status


def _sconv_out(**kw):
    args = dict(dtype=ink.BF16, C=1024, seqs=2, toks=10, maxlen=8, x=FAKE, w=FAKE, st=FAKE,
                slot=FAKE, cu=FAKE, y=FAKE + (1 << 20))
    args.update(kw)
    return ink._lib._lib.inkattn_sconv_out(
        args["dtype"], args["C"], args["seqs"], args["toks"], args["maxlen"], args["x"],
        args["w"], args["st"], args["slot"], args["cu"], args["y"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 2), (dict(C=0), 1), (dict(C=12), 1), (dict(C=8200), 2),
    (dict(seqs=-1), 1), (dict(seqs=0), 0), (dict(toks=0), 0), (dict(maxlen=0), 0),
    (dict(x=None), 1), (dict(w=None), 1), (dict(st=None), 1), (dict(slot=None), 1),
    (dict(cu=None), 1), (dict(y=None), 1), (dict(x=FAKE + 8), 1),
    (dict(y=FAKE), 1),                                        # in place
    (dict(y=FAKE + 10 * 1024 * 2 - 16), 1),                   # y starts inside x
    (dict(x=FAKE + (1 << 20) + 16), 1),                       # x starts inside y
])
def test_sconv_out_host_validation(kw, status):
    assert _sconv_out(**kw) == status


def _sconv_fp8(**kw):
    args = dict(dtype=ink.BF16, Hkv=4, d=128, seqs=2, toks=10, maxlen=8, k=FAKE, v=FAKE,
                w=FAKE, st=FAKE, slot=FAKE, cu=FAKE, sm=FAKE, ks=0.02, vs=0.03, kc=FAKE,
                vc=FAKE)
    args.update(kw)
    return ink._lib._lib.inkattn_sconv_fp8(
        args["dtype"], args["Hkv"], args["d"], args["seqs"], args["toks"], args["maxlen"],
        args["k"], args["v"], args["w"], args["st"], args["slot"], args["cu"], args["sm"],
        args["ks"], args["vs"], args["kc"], args["vc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 2), (dict(d=64), 2), (dict(Hkv=0), 1), (dict(seqs=0), 0),
    (dict(toks=0), 0), (dict(ks=0.0), 1), (dict(vs=-1.0), 1), (dict(ks=float("inf")), 1),
    (dict(vs=float("nan")), 1), (dict(ks=1e-39), 1),            # reciprocal overflows
    (dict(ks=0.0, seqs=0), 1),                                   # scales checked first
    (dict(kc=None), 1), (dict(kc=FAKE + 8), 1),
])
def test_sconv_fp8_host_validation(kw, status):
    assert _sconv_fp8(**kw) == status


def _decode_fp8(desc, **kw):
    args = dict(num_seqs=2, num_tokens=2, max_q_len=1, max_seq_len=100, q=FAKE, k=FAKE,
                v=FAKE, ks=0.02, vs=0.03, bt=FAKE, mb=1, cu=FAKE, sl=FAKE, bias=FAKE, out=FAKE,
                lse=None, splits=0, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return ink._lib._lib.inkattn_relattn_decode_fp8(
        ctypes.byref(desc), args["num_seqs"], args["num_tokens"], args["max_q_len"],
        args["max_seq_len"], args["q"], args["k"], args["v"], args["ks"], args["vs"],
        args["bt"], args["mb"], args["cu"], args["sl"], args["bias"], args["out"],
        args["lse"], args["splits"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0.0), 1), (dict(vs=float("inf")), 1), (dict(max_q_len=17), 2),
    (dict(cu=None), 1), (dict(k=None), 1), (dict(ws_bytes=16), 1), (dict(num_seqs=0), 0),
])
def test_decode_fp8_host_validation(kw, status):
    d = ink.make_desc(ink.BF16, 32, 4, 0, 128)
    assert _decode_fp8(d, **kw) == status


def test_decode_fp8_needs_bf16_queries():
    d = ink.make_desc(ink.FP32, 32, 4, 0, 128)
    assert _decode_fp8(d) == 2


def _prefill_fp8(desc, **kw):
    args = dict(num_seqs=2, num_tokens=5, max_q_len=4, q=FAKE, k=FAKE, v=FAKE, ks=0.5, vs=0.25,
                bt=FAKE, mb=4, cu=FAKE, sl=FAKE, bias=FAKE, out=FAKE, lse=None, ws=FAKE,
                ws_bytes=1 << 30)
    args.update(kw)
    return ink._lib._lib.inkattn_relattn_prefill_fp8(
        ctypes.byref(desc), args["num_seqs"], args["num_tokens"], args["max_q_len"], args["q"],
        args["k"], args["v"], args["ks"], args["vs"], args["bt"], args["mb"], args["cu"],
        args["sl"], args["bias"], args["out"], args["lse"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=0), ink.OK), (dict(num_tokens=0), ink.OK), (dict(max_q_len=0), ink.OK),
    (dict(ks=0.0), ink.EINVAL), (dict(vs=-1.0), ink.EINVAL), (dict(ks=float("inf")), ink.EINVAL),
    (dict(ks=float("nan")), ink.EINVAL), (dict(ws=None), ink.EINVAL), (dict(ws=FAKE + 8), ink.EINVAL),
    (dict(ws_bytes=1000), ink.EINVAL), (dict(mb=0), ink.EINVAL), (dict(q=None), ink.EINVAL),
    (dict(num_seqs=70000, mb=1), ink.ENOTSUP),
])
def test_prefill_fp8_host_validation(kw, status):
    d = ink.make_desc(ink.BF16, 32, 4, 0, 128)
    assert _prefill_fp8(d, **kw) == status


def test_prefill_fp8_rejects_fp32_and_sizes_workspace():
    assert _prefill_fp8(ink.make_desc(ink.FP32, 32, 4, 0, 128)) == ink.ENOTSUP
    d = ink.make_desc(ink.BF16, 32, 4, 2048, 2048)
    # two bf16 copies of each (sequence, block) page (4 kv-heads x 128 x 128)
    # plus an int32 block table, padded to 16 bytes
    pages = 3 * 10
    assert ink.inkattn_relattn_prefill_fp8_workspace_size(d, 3, 10) == \
        2 * pages * 4 * 128 * 128 * 2 + (pages * 4 + 15) // 16 * 16
    assert ink.inkattn_relattn_prefill_fp8_workspace_size(
        ink.make_desc(ink.FP32, 32, 4, 0, 128), 3, 10) == 0


def _prefill_fp8_mma(desc, **kw):
    args = dict(num_seqs=2, num_tokens=5, max_q_len=4, q=FAKE, k=FAKE, v=FAKE, ks=0.5, vs=0.25,
                bt=FAKE, mb=4, cu=FAKE, sl=FAKE, bias=FAKE, out=FAKE, lse=None)
    args.update(kw)
    return ink._lib._lib.inkattn_relattn_prefill_fp8_mma(
        ctypes.byref(desc), args["num_seqs"], args["num_tokens"], args["max_q_len"], args["q"],
        args["k"], args["v"], args["ks"], args["vs"], args["bt"], args["mb"], args["cu"],
        args["sl"], args["bias"], args["out"], args["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=0), ink.OK), (dict(num_tokens=0), ink.OK), (dict(max_q_len=0), ink.OK),
    (dict(ks=0.0), ink.EINVAL), (dict(vs=-1.0), ink.EINVAL), (dict(ks=float("inf")), ink.EINVAL),
    (dict(ks=float("nan")), ink.EINVAL), (dict(mb=0), ink.EINVAL), (dict(q=None), ink.EINVAL),
    (dict(k=FAKE + 8), ink.EINVAL), (dict(out=FAKE + 2), ink.EINVAL), (dict(num_seqs=-1), ink.EINVAL),
])
def test_prefill_fp8_mma_host_validation(kw, status):
    d = ink.make_desc(ink.BF16, 32, 4, 0, 128)
    assert _prefill_fp8_mma(d, **kw) == status


def test_prefill_fp8_mma_rejects_fp32():
    assert _prefill_fp8_mma(ink.make_desc(ink.FP32, 32, 4, 0, 128)) == ink.ENOTSUP
