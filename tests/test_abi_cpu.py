"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

from mla_latent_kv_partial_amd import _lib
from mla_latent_kv_partial_amd._lib import i32_array, i64_array, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ARG, SHAPE, ROPE, SEL, WS, DEV, UNSUP = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails on the host first


def _declared():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n)


def test_version_and_empty_error():
    assert lib.mla_version() >= 100
    assert isinstance(lib.mla_last_error(), bytes)


def _rope(**kw):
    a = dict(dtype=0, x=FAKE, y=FAKE, batch=2, tokens=3, inner=4, feat=16, sb=192, st=64, si=16, rot=16,
             theta=1e4, offs=[1, 2], n=2)
    a.update(kw)
    return lib.mla_rope_partial_interleaved(a["dtype"], a["x"], a["y"], a["batch"], a["tokens"], a["inner"],
                                            a["feat"], a["sb"], a["st"], a["si"], a["rot"], a["theta"],
                                            i64_array(a["offs"]), a["n"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), ARG),
    (dict(rot=15), ROPE), (dict(rot=0), ROPE), (dict(rot=18), ROPE),
    (dict(theta=0.0), ROPE), (dict(theta=float("inf")), ROPE), (dict(theta=float("nan")), ROPE),
    (dict(offs=[-1, 0]), ROPE), (dict(n=3, offs=[0, 1, 2]), ROPE),
    (dict(feat=1024, rot=1024), UNSUP),
    (dict(offs=[2 ** 53, 0]), UNSUP),
])
def test_rope_rejections(kw, code):
    assert _rope(**kw) == code
    assert lib.mla_last_error() != b""


def test_rope_empty_is_a_no_op():
    assert _rope(batch=0, offs=[0], n=1) == OK
    assert _rope(tokens=0) == OK


def _decode(**kw):
    a = dict(dtype=1, b=2, h=64, r=512, dr=64, w=100, kv=[100, 50], sel=None, cnt=None, chunk=32, s_max=4,
             scale=0.07, sel_idx=None, pdt=0)
    a.update(kw)
    return lib.mla_decode_latent_attn(
        a["dtype"], FAKE, FAKE, 64 * 64, 64, FAKE, 100 * 576, 576, FAKE, 100 * 576, 576, a["b"], a["h"], a["r"],
        a["dr"], a["w"], i32_array(a["kv"]), a["sel_idx"], None if a["cnt"] is None else i32_array(a["cnt"]),
        a["scale"], a["chunk"], a["pdt"], FAKE, FAKE, a["s_max"], None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=[0, 5]), SHAPE), (dict(kv=[101, 5]), SHAPE),
    (dict(s_max=3), SHAPE),
    (dict(cnt=[0, -1], sel_idx=FAKE), SEL), (dict(cnt=[-2, -1], sel_idx=FAKE), SEL),
    (dict(cnt=[5, -1], sel_idx=None), ARG),
    (dict(chunk=0), ARG), (dict(h=0), ARG), (dict(dtype=3), ARG), (dict(scale=float("nan")), ARG),
    (dict(r=2048), UNSUP), (dict(dr=512), UNSUP), (dict(pdt=5), ARG),
])
def test_decode_rejections(kw, code):
    assert _decode(**kw) == code


def test_decode_empty_batch_is_ok():
    assert _decode(b=0, kv=[]) == OK


@pytest.mark.parametrize("pdt,ns,code", [(0, [0, 1], SHAPE), (1, [5, 1], SHAPE), (2, [1, 1], ARG)])
def test_combine_rejections(pdt, ns, code):
    assert lib.mla_decode_combine(pdt, FAKE, FAKE, 2, 4, 8, 4, i32_array(ns), FAKE, None, None) == code


def test_combine_v_rejections():
    ns = i32_array([2, 1])
    assert lib.mla_decode_combine_v(7, 0, FAKE, FAKE, 2, 4, 8, 4, ns, FAKE, 4, 4, FAKE, None, None, None) == ARG
    assert lib.mla_decode_combine_v(1, 0, FAKE, FAKE, 2, 4, 8, 4, ns, FAKE, 4, 0, FAKE, None, None, None) == ARG
    assert lib.mla_decode_combine_v(1, 0, FAKE, FAKE, 2, 4, 8, 4, ns, FAKE, 4, 4, None, None, None, None) == ARG
    assert lib.mla_decode_combine_v(1, 0, FAKE, FAKE, 2, 4, 8, 4, i32_array([5, 1]), FAKE, 4, 4, FAKE, None, None,
                                    None) == SHAPE
    assert lib.mla_decode_combine_v(1, 0, FAKE, FAKE, 2, 4, 2048, 4, ns, FAKE, 4, 4, FAKE, None, None, None) == UNSUP
    assert lib.mla_decode_combine_v(1, 0, FAKE, FAKE, 0, 4, 8, 4, ns, FAKE, 4, 4, FAKE, None, None, None) == OK
    assert lib.mla_decode_combine_v(1, 3, FAKE, FAKE, 2, 4, 8, 4, ns, FAKE, 4, 4, FAKE, None, None, None) == ARG


def test_stream_probe_rejections():
    kv = i32_array([5, 3])
    probe = lambda dt=1, rope=0x1400, r=512, dr=64, st=576, kvl=kv, w=8: lib.mla_decode_stream_probe(
        dt, ctypes.c_void_p(0x1000), 8 * st, st, ctypes.c_void_p(rope), 8 * st, st, 2, r, dr, w, kvl, 32, None)
    assert probe(dt=0) == UNSUP                        # fp32 cache
    assert probe(rope=0x2000) == UNSUP                 # not packed: rope is not latent + 512
    assert probe(r=256) == UNSUP
    assert probe(kvl=i32_array([9, 3])) == SHAPE       # kv_len beyond the width
    assert lib.mla_decode_stream_probe(1, FAKE, 0, 576, FAKE, 0, 576, 0, 512, 64, 8, kv, 32, None) == OK


def test_absorb_rejections():
    assert lib.mla_absorb_q(5, FAKE, 1, 1, FAKE, FAKE, 1, 1, 1, 1, 1, None) == ARG
    assert lib.mla_absorb_q(0, None, 1, 1, FAKE, FAKE, 1, 1, 1, 1, 1, None) == ARG
    assert lib.mla_absorb_v(0, FAKE, FAKE, FAKE, 1, 0, 1, 1, 1, None) == ARG
    assert lib.mla_absorb_v(0, FAKE, FAKE, FAKE, 0, 1, 1, 1, 1, None) == OK


def _query(**kw):
    a = dict(dtype=1, qn=FAKE, qr=FAKE, qo=FAKE, w=FAKE, ql=FAKE, b=2, h=4, dn=16, dr=8, dv=16, r=32, pos=[3, 0],
             theta=1e4, sb=1, sh=1)
    a.update(kw)
    return lib.mla_decode_query(a["dtype"], a["qn"], a["sb"], a["sh"], a["qr"], a["qo"], 1, 1, a["w"], a["ql"],
                                a["b"], a["h"], a["dn"], a["dr"], a["dv"], a["r"],
                                None if a["pos"] is None else i64_array(a["pos"]), a["theta"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), ARG), (dict(h=0), ARG), (dict(qn=None), ARG), (dict(qo=None), ARG), (dict(pos=None), ARG),
    (dict(sb=-1), ARG), (dict(dr=7), ROPE), (dict(dr=0), ROPE), (dict(theta=-1.0), ROPE),
    (dict(theta=float("inf")), ROPE), (dict(pos=[3, -1]), ROPE), (dict(dr=514), UNSUP),
    (dict(pos=[2 ** 53, 0]), UNSUP),
])
def test_decode_query_rejections(kw, code):
    assert _query(**kw) == code


def test_decode_query_empty_batch_is_ok():
    assert _query(b=0, pos=[0]) == OK


def _prefill(ws=None, size=0, ptr=FAKE, **kw):
    a = dict(dtype=1, b=1, t=16, k=16, h=4, ql=32, r=32, dn=16, dr=8, dv=16, offs=[0], theta=1e4, pad=None)
    a.update(kw)
    sz = ctypes.c_size_t(size)
    code = lib.mla_prefill_reconstructed(
        a["dtype"], a["b"], a["t"], a["k"], a["h"], a["ql"], a["r"], a["dn"], a["dr"], a["dv"], ptr, ptr, ptr,
        ptr, ptr, i64_array(a["offs"]), a["theta"], None if a["pad"] is None else i32_array(a["pad"]), 0.1,
        ws, ctypes.byref(sz), ptr, None)
    return code, sz.value


def test_prefill_workspace_query_fits_either_path():
    """The size query with NULL data pointers suffices whichever path the real
    pointers select: 16-byte aligned bf16 buffers of the GLM head geometry take
    the MFMA path, misaligned ones the generic path (fp32 intermediates).  The
    calls stop at the negative offset, after the workspace check."""
    glm = dict(t=64, k=64, h=2, ql=64, r=64, dn=128, dr=64, dv=128)
    code, need = _prefill(ptr=None, **glm)
    assert code == OK and need > 0
    ws = ctypes.c_void_p(0x100000)
    for ptr in (ctypes.c_void_p(0x2000), ctypes.c_void_p(0x2008)):     # aligned, then misaligned
        assert _prefill(ws=ws, size=need, ptr=ptr, offs=[-1], **glm)[0] == ROPE
    # the generic path alone needs more than the MFMA path for these shapes
    assert _prefill(ws=ws, size=need // 2, ptr=ctypes.c_void_p(0x2008), offs=[-1], **glm)[0] == WS


def test_prefill_workspace_query_and_rejections():
    code, need = _prefill()
    assert code == OK and need > 0
    assert _prefill(ws=ctypes.c_void_p(0x10000), size=need - 1)[0] == WS
    assert _prefill(ws=ctypes.c_void_p(0x10010), size=need)[0] == WS        # misaligned
    assert _prefill(t=17)[0] == SHAPE                                          # keys < tokens
    assert _prefill(dr=7)[0] == ROPE
    assert _prefill(theta=-1.0)[0] == ROPE
    assert _prefill(dn=250)[0] == UNSUP
    assert _prefill(ws=ctypes.c_void_p(0x10000), size=need, offs=[-1])[0] == ROPE
    assert _prefill(ws=ctypes.c_void_p(0x10000), size=need, pad=[17])[0] == SHAPE


def _topk(batch=2, lens=(10, 3), top_k=4, stride=16, scores=FAKE, sel=FAKE, ws=None, size=None):
    counts = i32_array([7] * max(batch, 1))
    sz = None if size is None else ctypes.byref(size)
    code = lib.mla_dsa_topk_select(scores, stride, batch, i32_array(list(lens)), top_k, sel, counts, ws, sz, None)
    return code, [counts[i] for i in range(max(batch, 1))]


def test_dsa_topk_workspace_query():
    # rows of 2..8 segments of 16384 scores whose candidates fit take the
    # two-stage path: 131328 bytes each; the query launches nothing
    size = ctypes.c_size_t(123)
    assert _topk(lens=(131072, 3), top_k=2048, stride=131072, size=size)[0] == OK
    assert size.value == 131328
    size = ctypes.c_size_t(123)
    assert _topk(lens=(131072, 131072), top_k=2048, stride=131072, size=size)[0] == OK
    assert size.value == 2 * 131328
    for lens, k in (((16384, 3), 64), ((300000, 5), 64), ((131072, 5), 4096)):   # one segment, 19, 8 x 4096
        size = ctypes.c_size_t(123)
        assert _topk(lens=lens, top_k=k, stride=max(lens), size=size)[0] == OK and size.value == 0
    small = ctypes.c_size_t(131327)
    assert _topk(lens=(131072, 3), top_k=2048, stride=131072, ws=ctypes.c_void_p(0x10000), size=small)[0] == WS
    enough = ctypes.c_size_t(131328)
    assert _topk(lens=(131072, 3), top_k=2048, stride=131072, ws=ctypes.c_void_p(0x10010), size=enough)[0] == WS


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ARG), (dict(top_k=0), ARG), (dict(scores=None), ARG),
    (dict(lens=(0, 3)), SHAPE), (dict(lens=(2 ** 30 + 1, 3)), SHAPE), (dict(lens=(17, 3)), SHAPE),
    (dict(sel=None), ARG),
])
def test_dsa_topk_rejections(kw, code):
    assert _topk(**kw)[0] == code
    assert lib.mla_last_error() != b""


def test_dsa_topk_all_dense_rows_launch_nothing():
    # every row is not longer than top_k: counts -1, nothing enqueued, sel_idx may be NULL
    code, counts = _topk(lens=(4, 3), top_k=4, sel=None)
    assert code == OK and counts == [-1, -1]
    assert _topk(batch=0)[0] == OK


def _append(**kw):
    a = dict(dtype=1, batch=2, tokens=1, r=512, dr=64, eps=1e-6, pos=[3, 4], theta=1e4, slot=0, lt=576, rt=576,
             kv=FAKE, w=FAKE)
    a.update(kw)
    return lib.mla_append_compressed(a["dtype"], a["kv"], 576, 576, a["batch"], a["tokens"], a["r"], a["dr"], a["w"],
                                     a["eps"], i64_array(a["pos"]), a["theta"], FAKE, 576 * 8, a["lt"], FAKE,
                                     576 * 8, a["rt"], a["slot"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), ARG), (dict(eps=-1.0), ARG), (dict(eps=float("inf")), ARG), (dict(slot=-1), ARG),
    (dict(dr=63), ROPE), (dict(theta=0.0), ROPE), (dict(pos=[-1, 0]), ROPE), (dict(kv=None), ARG),
    (dict(lt=0), ARG), (dict(dr=1024), UNSUP),
])
def test_append_rejections(kw, code):
    assert _append(**kw) == code
    assert lib.mla_last_error() != b""


def test_append_empty_is_a_no_op():
    assert _append(batch=0, pos=[0]) == OK
    assert _append(tokens=0) == OK


def test_o_proj_workspace_query_and_rejections():
    need = ctypes.c_size_t(7)
    assert lib.mla_o_proj_workspace_bytes(1, 8, 8192, 6144, ctypes.byref(need)) == OK and need.value == 0
    assert lib.mla_o_proj_workspace_bytes(1, 4096, 8192, 6144, ctypes.byref(need)) == OK
    assert need.value == 4096 * 8192 * 2
    assert lib.mla_o_proj_workspace_bytes(0, 4096, 8192, 6144, ctypes.byref(need)) == OK and need.value == 0
    assert lib.mla_o_proj_workspace_bytes(3, 8, 8, 8, ctypes.byref(need)) == ARG
    assert lib.mla_o_proj(1, FAKE, -1, 8, FAKE, 8, FAKE, None, 0, None) == ARG
    assert lib.mla_o_proj(1, None, 8, 8, FAKE, 8, FAKE, None, 0, None) == ARG
    # the GEMM path needs its workspace
    assert lib.mla_o_proj(1, FAKE, 4096, 8192, FAKE, 6144, FAKE, None, 0, None) == WS
    assert lib.mla_o_proj(1, FAKE, 4096, 8192, FAKE, 6144, FAKE, FAKE, 100, None) == WS
    assert lib.mla_o_proj(1, FAKE, 0, 8192, FAKE, 6144, FAKE, None, 0, None) == OK
