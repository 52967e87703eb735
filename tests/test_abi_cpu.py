"""Host-side checks that need no GPU: the library loads, exports every entry
point that include/csa.h declares, and rejects bad arguments with the right
status before anything is enqueued (no compute call is made)."""

import ctypes as C
import os
import re

import pytest

from sparse_attention_csa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "csa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.csa_abi_version() == 4


def _status(fn, *args):
    return fn(*args)


def test_compress_rejects_bad_arguments():
    lib = L.lib()
    P = 1 << 20  # never dereferenced: validation fails first
    # null content
    s = lib.csa_compress(1, None, P, 512, None, None, None, None, None, None, None,
                         1, 8, 512, 4, P, 1, None, 2, 0, None)
    assert s == L.CSA_ERR_ARG and "content_a" in L.last_error()
    # T not a multiple of m
    s = lib.csa_compress(1, P, P, 512, None, None, None, None, None, None, None,
                         1, 6, 512, 4, P, 1, None, 2, 0, None)
    assert s == L.CSA_ERR_ARG
    # unsupported width
    s = lib.csa_compress(1, P, P, 1, None, None, None, None, None, None, None,
                         1, 8, 100, 4, P, 1, None, 2, 0, None)
    assert s == L.CSA_ERR_UNSUPPORTED
    # entries beyond E_cap
    s = lib.csa_compress(1, P, P, 512, None, None, None, None, None, None, None,
                         1, 8, 512, 4, P, 1, None, 2, 1, None)
    assert s == L.CSA_ERR_ARG and "E_cap" in L.last_error()
    # E4M3 / MXFP4 output without scales
    for out_dt in (2, 3):
        s = lib.csa_compress(1, P, P, 512, None, None, None, None, None, None, None,
                             1, 8, 512, 4, P, out_dt, None, 2, 0, None)
        assert s == L.CSA_ERR_ARG


def test_index_topk_rejects_bad_arguments():
    lib = L.lib()
    P = 1 << 20
    ws_need = lib.csa_index_topk_workspace(2, 1, 1024, 64)
    assert ws_need >= 2 * 1024 * 4
    args = dict(dt=1, q=P, qs=None, w=P, k_=P, ks=None, pos=P, ne=P, B=2, Tq=1, H_I=64, d_I=128,
                E=1024, m=4, k=64, vis=0, sb=0, ti=P, tc=P, sc=None, ws=P, wsb=ws_need, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.csa_index_topk(*a.values())

    assert call(H_I=65) == L.CSA_ERR_UNSUPPORTED
    assert call(d_I=96) == L.CSA_ERR_UNSUPPORTED
    assert call(k=4096) == L.CSA_ERR_UNSUPPORTED
    assert call(k=0) == L.CSA_ERR_ARG
    assert call(dt=2) == L.CSA_ERR_ARG  # E4M3 without scales
    assert call(dt=3) == L.CSA_ERR_ARG  # MXFP4 without scales
    assert call(dt=3, qs=None, ks=P) == L.CSA_ERR_ARG
    assert call(dt=4) == L.CSA_ERR_ARG  # no such format
    assert call(sb=2) == L.CSA_ERR_ARG  # score_bf16 is 0 or 1
    assert call(wsb=ws_need - 1) == L.CSA_ERR_WORKSPACE
    assert call(ws=None) == L.CSA_ERR_WORKSPACE
    assert call(pos=None) == L.CSA_ERR_ARG


def test_attend_rejects_bad_arguments():
    lib = L.lib()
    P = 1 << 20
    need = lib.csa_attend_workspace(1, 1, 64, 512, 640)
    base = [1, P, P, 100, P, P, 512, P, 128, None, 128, None, P, 0.04, 1, 1, 64, 512, P, None, P,
            need, None]
    ok = list(base)
    bad_c = list(base); bad_c[17] = 384
    assert lib.csa_attend(*bad_c) == L.CSA_ERR_UNSUPPORTED
    bad_h = list(base); bad_h[16] = 129
    assert lib.csa_attend(*bad_h) == L.CSA_ERR_UNSUPPORTED
    bad_w = list(base); bad_w[8] = 64  # W_cap < n_win
    assert lib.csa_attend(*bad_w) == L.CSA_ERR_ARG
    bad_dt = list(base); bad_dt[0] = 2
    assert lib.csa_attend(*bad_dt) == L.CSA_ERR_UNSUPPORTED
    no_ws = list(base); no_ws[20] = None
    assert lib.csa_attend(*no_ws) == L.CSA_ERR_WORKSPACE
    del ok


def test_layer_rejects_bad_descriptors():
    lib = L.lib()
    d = L.LayerDesc(kind=3, H=64, c=512, H_I=64, d_I=128, m=4, overlap=1, k=512, n_win=128,
                    vis=0, kv_dtype=1, idx_dtype=1, scale=0.044)
    s = L.LayerState()
    io = L.DecodeIO()
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "kind" in L.last_error()
    d.kind = L.CSA_LAYER_CSA
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG  # empty state
    d.n_win = 1000
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_UNSUPPORTED
    d.n_win = 128
    d.split_rows = 40  # batch-invariant split size: a multiple of 16
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "split_rows" in L.last_error()
    d.split_rows = 16  # (512 + 128) / 16 = 40 splits fit; 2304 rows at most
    assert lib.hybrid_layer_workspace(C.byref(d), 8, 1, 32768) > 0
    d.split_rows = 2320
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_UNSUPPORTED and "split_rows" in L.last_error()
    d.split_rows = 0
    assert lib.hybrid_layer_workspace(C.byref(d), 8, 1, 32768) > 0
    d.score_bf16 = 2
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "score_bf16" in L.last_error()
    d.score_bf16 = 0
    d.idx_dtype = 5
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "idx_dtype" in L.last_error()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "sparse_attention_csa_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle", src, flags=re.M), fn
            assert "workloads" not in re.findall(r"^\s*(?:from|import)\s+(\w+)", src, flags=re.M), fn


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_LIB", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libcsa.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        L.lib()


def test_layer_rejects_bad_pages():
    """The paged cache's arguments are checked before anything is enqueued
    (the state's pointers here are never dereferenced)."""
    lib = L.lib()
    d = L.LayerDesc(kind=L.CSA_LAYER_CSA, H=64, c=512, H_I=64, d_I=128, m=4, overlap=1, k=512, n_win=128,
                    vis=0, kv_dtype=1, idx_dtype=1, scale=0.044)
    s = L.LayerState(B=2, E_cap=4096)
    fake = 1 << 20
    for n in ("kv_cache", "n_entries", "win_ring", "tail", "idx_cache", "idx_tail"):
        setattr(s, n, fake)
    io = L.DecodeIO()
    s.block_table = fake
    for P in (24, 0, -32, 8192):  # not a power of two; 8192 does not divide E_cap
        s.page_entries = P
        st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
        assert st == L.CSA_ERR_ARG and "page_entries" in L.last_error(), (P, L.last_error())
    s.page_entries = 32
    s.block_table = fake + 4
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "block_table" in L.last_error()
    s.block_table = fake  # a valid paged state: the next check is the io's
    st = lib.hybrid_layer_decode(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "pos" in L.last_error()
    st = lib.hybrid_layer_prefill(C.byref(d), C.byref(s), C.byref(L.PrefillIO()), None, 0, None)
    assert st == L.CSA_ERR_ARG and "page_entries" not in L.last_error()


def test_prefill_chunk_arguments():
    """Aligned chunks must start and end on block boundaries; per-sequence
    chunks (seq_pos0 with seq_len) need both arrays.  The checks fail before
    anything is enqueued (the pointers are never dereferenced)."""
    lib = L.lib()
    d = L.LayerDesc(kind=L.CSA_LAYER_HCA, H=64, c=512, m=128, overlap=0, n_win=128, vis=0, kv_dtype=1,
                    scale=0.044)
    s = L.LayerState(B=2, E_cap=64)
    fake = 1 << 20
    for n in ("kv_cache", "n_entries", "win_ring", "tail"):
        setattr(s, n, fake)
    io = L.PrefillIO(pos0=128, T=100)
    for n in ("q", "win", "streams", "out"):
        setattr(io, n, fake)
    st = lib.hybrid_layer_prefill(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_UNSUPPORTED and "block boundaries" in L.last_error()
    io.seq_pos0 = fake
    st = lib.hybrid_layer_prefill(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_ARG and "seq_len" in L.last_error()
    io.seq_len = fake
    st = lib.hybrid_layer_prefill(C.byref(d), C.byref(s), C.byref(io), None, 0, None)
    assert st == L.CSA_ERR_WORKSPACE  # the chunk itself is accepted
