"""GPU parity at sizes the oracle finishes in seconds: the HIP path (through
the C ABI) against the float64 oracle on the same seeded inputs, element by
element, with the tolerance rules of tests/compare.py.  Shapes span several
tiles and a ragged tail (visible-entry counts that are not tile multiples)."""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as OL
from oracle.formats import Stored
from tests.compare import (ambiguous_e4m3_keys, ambiguous_mxfp4_keys, assert_close, assert_entry_close,
                           check_selection, decode_err, gpu_entries, mxfp4_alternatives, prefill_err, score_bounds,
                           score_error_bound, topk_check, topk_check_bounds)

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _check_decode(g, sess, label):
    L_ = sess.g
    torch.cuda.synchronize()
    out, lse = f64(sess.io["out"]), f64(sess.io["lse"])
    n_ent = sess.state.n_entries.cpu().numpy()
    kvk = g["kv_dtype"]
    act = "bf16" if kvk == "fp8bf16" else kvk  # outputs are activations
    swaps_total = 0
    for b in range(g["B"]):
        print(f"[{label}] seq {b}", flush=True)
        ref = OL.decode_step(g, b)
        e0 = int(g["n_entries"][b])
        assert n_ent[b] == e0 + len(ref["folded_kv"]), "n_entries not advanced by the fold"
        if ref["folded_kv"]:
            gk = gpu_entries(sess.state, b, slice(e0, e0 + 1), kvk)
            assert_entry_close(gk, np.array(ref["folded_kv"][:1]), kvk, f"{label} folded kv b={b}")
        if g["kind"] == "csa":
            idk = g["idx_dtype"]
            if ref["folded_idx"]:
                _check_folded_key(g, sess, b, e0, ref["folded_idx"][0], label, ref["folded_idx_raw"][0])
            ids = sess.io["topk_idx"][b].cpu().numpy()
            cnt = int(sess.io["topk_cnt"][b].item())
            bd, amb = {}, {}
            if idk == "e4m3" and ref["folded_idx_raw"]:
                amb = ambiguous_e4m3_keys(ref["folded_idx_raw"][:1], [e0])
            elif idk == "mxfp4" and ref["folded_idx_raw"]:
                amb = ambiguous_mxfp4_keys(ref["folded_idx_raw"][:1], [e0])
            if amb:
                q = Stored(g["q_idx"][b], idk, g["q_scale"][b]).all()
                bd = score_bounds(q, np.asarray(g["w_idx"][b], np.float64), amb)
            ok, swaps, msg = check_selection(ids, cnt, g["k"], ref, decode_err(g, b, ref), bd,
                                             g.get("score_dtype", "f32"))
            assert ok, f"{label} b={b}: {msg}"
            swaps_total += swaps
            if swaps:
                ref = OL.decode_step(g, b, selected=ids[:cnt])
        assert_close(out[b], ref["o"], act, f"{label} out b={b}")
        assert np.abs(lse[b] - ref["lse"]).max() < 1e-3, f"{label} lse b={b}"
    _check_rings(g, sess, label)
    return swaps_total


def _check_rings(g, sess, label):
    """The step's token in the window ring and the compressor tail rings:
    bit-equal to the step's inputs (a copy)."""
    st = sess.state
    torch.cuda.synchronize()
    as_u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa
    streams = ("ca", "za", "cb", "zb")[:st.S]
    for b in range(g["B"]):
        t = int(g["pos"][b])
        if g.get("norm_rope"):
            # the ring receives the row prepared at t (normalised, rotated)
            from oracle import position as P
            from oracle.csa import store_as
            act = "bf16" if g["kv_dtype"] == "fp8bf16" else g["kv_dtype"]
            raw = Stored(g["x_new"][b][None], act).all()[0]
            want = store_as(P.prepare(raw, g["kv_norm_w"], g["norm_eps"], t, g["rope_inv_freq"]), act)
            assert_close(f64(st.win_ring[b, t % g["n_win"]])[None], want[None], act,
                         f"{label} prepared window row b={b}")
        else:
            assert np.array_equal(as_u16(st.win_ring[b, t % g["n_win"]]), g["x_new"][b]), f"{label} window ring b={b}"
        for si, name in enumerate(streams):
            assert np.array_equal(as_u16(st.tail[b, si, t % st.R]), g["new_" + name][b]), f"{label} tail {name} b={b}"
        if g["kind"] == "csa":
            for si, name in enumerate(("ca", "za", "cb", "zb")):
                assert np.array_equal(as_u16(st.idx_tail[b, si, t % st.R]), g["new_i" + name][b]), \
                    f"{label} indexer tail {name} b={b}"


def _check_folded_key(g, sess, b, e0, ref_row, label, raw_row=None):
    if g["idx_dtype"] == "mxfp4":
        # the stored codes and scales must be one of the roundings float32
        # accuracy allows (the oracle's own rounding in all but rare cases)
        codes = sess.state.idx_cache[b, e0].cpu().numpy()
        scales = sess.state.idx_scale[b, e0].cpu().numpy()
        got = Stored(codes[None], "mxfp4", scales[None]).all()[0]
        alts = mxfp4_alternatives(raw_row) if raw_row is not None else [ref_row]
        assert any(np.array_equal(got, a) for a in alts), f"{label} mxfp4 key b={b}"
    elif g["idx_dtype"] == "e4m3":
        codes = sess.state.idx_cache[b, e0].cpu().numpy()
        scale = sess.state.idx_scale[b, e0].cpu().numpy()
        got = Stored(codes[None], "e4m3", np.array([scale])).all()[0]
        # The scale may differ by float32 rounding (amax of a float32 vs a float64
        # fold); a code may differ by one quantum where the value sits on a
        # rounding tie.  Anything beyond float32 rounding counts as a code flip.
        q = np.abs(got - ref_row)
        step = np.abs(ref_row) / 8 + float(scale) * 2.0 ** -9
        assert np.all(q <= step * 1.0001), f"{label} e4m3 key b={b}"
        flips = q > 1e-5 * np.abs(ref_row).max()
        assert flips.mean() <= 0.02, f"{label} e4m3 key b={b}: {flips.mean():.3f} codes differ"
    else:
        gk = f64(sess.state.idx_cache[b, e0])
        assert_close(gk[None], ref_row[None], g["idx_dtype"], f"{label} folded key b={b}")


def test_tiny_fp32_whole_context(gpu_lib):
    from sparse_attention_csa_amd import _lib as L
    g = workloads.tiny_case()
    kv_ref, keys_ref = OL.tiny_entries(g)
    cu = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)  # noqa
    x, xi = cu(g["x"]), cu(g["x_idx"])
    kv = L.csa_compress(x, None, g["m"], score_w=cu(g["w_cmp"]))
    keys = L.csa_compress(xi, None, g["m"], score_w=cu(g["w_cmp_idx"]))
    torch.cuda.synchronize()
    assert_close(f64(kv)[0], kv_ref, "f32", "tiny kv entries")
    assert_close(f64(keys)[0], keys_ref, "f32", "tiny indexer keys")
    q_pos = cu(g["q_pos"], torch.int64)
    n_ent = torch.tensor([kv.shape[1]], dtype=torch.int32, device="cuda")
    ids, cnt = L.csa_index_topk(cu(g["q_idx"]), cu(g["w_idx"]), keys, q_pos, n_ent, g["m"], g["k"])
    lse = torch.empty((1, g["Tq"], g["H"]), dtype=torch.float32, device="cuda")
    out = L.csa_attend(cu(g["q"]), kv, ids, cnt, x, torch.zeros(1, dtype=torch.int64, device="cuda"),
                       g["n_win"], q_pos, g["scale"], sink=cu(g["sink"]), lse=lse)
    torch.cuda.synchronize()
    ids, cnt, out, lse = ids.cpu().numpy(), cnt.cpu().numpy(), f64(out), f64(lse)
    for i in range(g["Tq"]):
        o, l, sel, scores = OL.tiny_query(g, i, kv_ref, keys_ref)
        ok, swaps, msg = topk_check(ids[0, i], cnt[0, i], sel, scores, g["k"],
                                    err=lambda: score_error_bound(g["q_idx"][0][i], g["w_idx"][0][i],
                                                                  keys_ref[:len(scores)]))
        assert ok, f"query {i}: {msg}"
        if swaps:
            o, l, _, _ = OL.tiny_query(g, i, kv_ref, keys_ref, selected=ids[0, i, :cnt[0, i]])
        assert_close(out[0, i], o, "f32", f"tiny out q{i}")
        assert np.abs(lse[0, i] - l).max() < 1e-4


@pytest.mark.parametrize("vis", [0, 1])
def test_decode_csa_bf16_small(gpu_lib, vis):
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.flash_csa_decode(seed=31, B=3, n=4096, H=16, c=128, H_I=8, d_I=64, k=64)
    if vis:
        g["vis"] = 1
        g["pos"] = g["pos"] + 3  # t = n+3 completes block n/4: fold uses the new token
        g["tail_pos0"] = g["tail_pos0"] + 3
        g["n_entries"] = g["n_entries"] + 1
        g["E_cap"] += 1
        for key in ("kv_cache", "idx_cache"):
            pad = np.zeros_like(g[key][:, :1])
            g[key] = np.concatenate([g[key], pad], axis=1)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"csa-bf16-vis{vis}")


@pytest.mark.parametrize("H,c", [(16, 128), (64, 512)])
def test_decode_hca_bf16_small(gpu_lib, H, c):
    """c = 512 with H % 32 == 0 runs the MFMA kernel with several row splits
    (200 entries + 128 window rows: a ragged last tile) and the merge."""
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.flash_hca_decode(seed=32, B=3, n=128 * 200, H=H, c=c)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"hca-bf16-c{c}")


@pytest.mark.parametrize("pos_off", [1, 37, 127])
def test_decode_hca_bf16_no_fold(gpu_lib, pos_off):
    """A step inside a block (no entry completes): the fused-fold path only
    scores the token and appends it to the rings."""
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.flash_hca_decode(seed=35, B=3, n=128 * 200, H=64, c=512, pos_off=pos_off)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"hca-bf16-no-fold-{pos_off}")


@pytest.mark.parametrize("pos_off", [1, 3])
def test_decode_csa_fp8_no_fold(gpu_lib, pos_off):
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=36, B=2, n=4 * 3000, H=128, c=512, H_I=8, d_I=64, k=128, pos_off=pos_off)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"csa-fp8-no-fold-{pos_off}")


@pytest.mark.parametrize("n,pos_off", [(4 * 40, 2), (4 * 2, 0), (4 * 2, 3)])
def test_decode_csa_short_context(gpu_lib, n, pos_off):
    """Fewer visible entries than k (all selected) and a window that is not
    full yet (t + 1 < n_win), down to two compressed entries."""
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=37, B=2, n=n, H=128, c=512, H_I=8, d_I=64, k=128, pos_off=pos_off)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"csa-short-{n}-{pos_off}")


@pytest.mark.parametrize("n,pos_off", [(128 * 1, 0), (128 * 2, 3)])
def test_decode_hca_short_context(gpu_lib, n, pos_off):
    """HCA decode with one or two entries (the first fold) and a window that
    is not full yet."""
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.flash_hca_decode(seed=38, B=2, n=n, H=64, c=512, pos_off=pos_off)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"hca-short-{n}-{pos_off}")


def test_decode_csa_largest_k_and_window(gpu_lib):
    """The largest supported selection and window: k = 2048, n_win = 256
    (2304 rows per query in one split of the sparse kernel at most)."""
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=39, B=2, n=4 * 6000, H=128, c=512, H_I=16, d_I=128, k=2048, n_win=256)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, "csa-k2048-win256")


@pytest.mark.parametrize("H,c", [(16, 128), (128, 512)])
def test_decode_csa_fp8_indexer_small(gpu_lib, H, c):
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=33, B=2, n=4 * 3000, H=H, c=c, H_I=8, d_I=64, k=128)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"csa-fp8-c{c}")


def _check_prefill(g, sess, label, queries=None):
    torch.cuda.synchronize()
    out, lse = f64(sess.io["out"]), f64(sess.io["lse"])
    kvk = g["kv_dtype"]
    act = "bf16" if kvk == "fp8bf16" else kvk
    kv_new, idx_new = OL.prefill_entries(g, 0)
    E0, n_new = int(g["n_entries"][0]), len(kv_new)
    assert int(sess.state.n_entries[0].item()) == E0 + n_new
    assert_entry_close(gpu_entries(sess.state, 0, slice(E0, E0 + n_new), kvk), kv_new, kvk, f"{label} entries")
    if g["kind"] == "csa":
        assert_close(f64(sess.state.idx_cache[0, E0:E0 + n_new]), idx_new, g["idx_dtype"],
                     f"{label} keys")
    ids = sess.io["topk_idx"][0].cpu().numpy() if g["kind"] == "csa" else None
    cnt = sess.io["topk_cnt"][0].cpu().numpy() if g["kind"] == "csa" else None
    qs = range(g["T"]) if queries is None else queries
    for i in qs:
        ref = OL.prefill_query(g, 0, i, kv_new, idx_new)
        if g["kind"] == "csa":
            ok, swaps, msg = topk_check(ids[i], cnt[i], ref["sel"], ref["scores"], g["k"],
                                        err=prefill_err(g, 0, i, idx_new, len(ref["scores"])))
            assert ok, f"{label} q{i}: {msg}"
            if swaps:
                ref = OL.prefill_query(g, 0, i, kv_new, idx_new, selected=ids[i, :cnt[i]])
        assert_close(out[0, i], ref["o"], act, f"{label} out q{i}")
        assert np.abs(lse[0, i] - ref["lse"]).max() < 1e-3


@pytest.mark.parametrize("H,c", [(8, 64), (64, 512)])
def test_prefill_csa_and_hca_small(gpu_lib, H, c):
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill(seed=34, T=256, n0=1024, H=H, c=c, H_I=8, d_I=32, k=32,
                                   m_hca=128)
    for g, label in ((a, "prefill-csa"), (h, "prefill-hca")):
        sess = PrefillSession(g)
        sess.run()
        _check_prefill(g, sess, label)
