"""GPU parity of entry points and paths that the layer tests do not reach on
their own: hca_attend called directly, the compressor's e4m3 output, the
fused top-k's fallback when its bounded wait gives up, the MFMA prefill
scorer, and run-to-run determinism of the decode and prefill paths."""

import numpy as np
import pytest
import torch

import workloads
from oracle import csa as OC
from oracle import layer as OL
from oracle.formats import Stored
from tests.compare import assert_close
from tests.test_gpu_parity import _check_decode, _check_prefill

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("H,c,Tq", [(64, 512, 1), (64, 512, 3), (8, 128, 2)])
def test_hca_attend_direct(gpu_lib, H, c, Tq):
    """hca_attend on a cache with n_entries < E_cap: a window ring (win_pos0
    = 0) for one query per sequence, a linear window buffer (win_pos0 = its
    first position) for several consecutive queries."""
    from sparse_attention_csa_amd import _lib as L
    rng = np.random.default_rng(50 + Tq)
    B, m, n_win, E_cap = 3, 128, 128, 300
    n_ent = np.array([300, 211, 17], np.int32)
    t_last = np.array([300 * 128 + 77, 211 * 128 + 5, 17 * 128 + 100], np.int64)
    kv_bits = workloads.gen.bf16_bits(rng.standard_normal((B, E_cap, c)).astype(np.float32))
    q_bits = workloads.gen.bf16_bits(rng.standard_normal((B, Tq, H, c)).astype(np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    # raw window rows of positions t_last - (n_win - 1) - (Tq - 1) .. t_last
    n_rows = n_win + Tq - 1
    win_rows = workloads.gen.bf16_bits(rng.standard_normal((B, n_rows, c)).astype(np.float32))
    first = t_last - (n_rows - 1)
    q_pos = first[:, None] + (n_win - 1) + np.arange(Tq)[None, :]
    if Tq == 1:
        W_cap = n_win
        win = np.zeros((B, W_cap, c), np.uint16)
        for b in range(B):
            for r in range(n_rows):
                win[b, (first[b] + r) % W_cap] = win_rows[b, r]
        win_pos0 = np.zeros(B, np.int64)
    else:
        win, win_pos0 = win_rows, first
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device="cuda")
    out = L.hca_attend(_dev_bf16(q_bits), _dev_bf16(kv_bits), torch.from_numpy(n_ent).cuda(), m,
                       _dev_bf16(win), torch.from_numpy(win_pos0).cuda(), n_win,
                       torch.from_numpy(q_pos).cuda(), 1.0 / np.sqrt(c),
                       sink=torch.from_numpy(sink).cuda(), lse=lse)
    torch.cuda.synchronize()
    out, lse = f64(out), f64(lse)
    for b in range(B):
        kv = Stored(kv_bits[b], "bf16")
        rows = Stored(win_rows[b], "bf16")
        for i in range(Tq):
            t = int(q_pos[b, i])
            o, l = OC.hca_query(Stored(q_bits[b, i], "bf16").all(), t, kv, int(n_ent[b]),
                                lambda p: rows.rows(np.asarray(p) - int(first[b])), sink, m, n_win,
                                1.0 / np.sqrt(c))
            assert_close(out[b, i], o, "bf16", f"hca_attend b={b} q{i}")
            assert np.abs(lse[b, i] - l).max() < 1e-3


def test_compress_e4m3_output(gpu_lib):
    """csa_compress writing e4m3 entries with one scale per entry (the
    indexer-key format), overlapping branches with the previous block given,
    at an offset into a larger cache."""
    from sparse_attention_csa_amd import _lib as L
    rng = np.random.default_rng(60)
    B, T, c, m, E_cap, first = 2, 64, 128, 4, 40, 7
    st = {n: workloads.gen.bf16_bits(rng.standard_normal((B, T, c)).astype(np.float32))
          for n in ("ca", "za", "cb", "zb")}
    prev = {n: workloads.gen.bf16_bits(rng.standard_normal((B, m, c)).astype(np.float32)) for n in ("cb", "zb")}
    ba = rng.standard_normal((m, c)).astype(np.float32)
    bb = rng.standard_normal((m, c)).astype(np.float32)
    out = torch.zeros((B, E_cap, c), dtype=torch.uint8, device="cuda")
    scale = torch.ones((B, E_cap), dtype=torch.float32, device="cuda")
    d = {n: _dev_bf16(v) for n, v in st.items()}
    L.csa_compress(d["ca"], d["za"], m, bias_a=torch.from_numpy(ba).cuda(), content_b=d["cb"],
                   logits_b=d["zb"], bias_b=torch.from_numpy(bb).cuda(),
                   prev_content_b=_dev_bf16(prev["cb"]), prev_logits_b=_dev_bf16(prev["zb"]),
                   out=out, out_scale=scale, out_first_entry=first)
    torch.cuda.synchronize()
    codes, scales = out.cpu().numpy(), scale.cpu().numpy()
    for b in range(B):
        dec = lambda v: Stored(v[b], "bf16").all()  # noqa: E731
        ent = OC.compress(dec(st["ca"]), dec(st["za"]), m, ba, dec(st["cb"]), dec(st["zb"]), bb,
                          Stored(prev["cb"][b], "bf16").all(), Stored(prev["zb"][b], "bf16").all())
        ref, ref_scale = OC.e4m3_quantize_rows(ent)
        got = Stored(codes[b, first:first + T // m], "e4m3", scales[b, first:first + T // m]).all()
        # the scale is formed from float32 fold values: within their accuracy
        assert np.allclose(scales[b, first:first + T // m], ref_scale, rtol=1e-5, atol=0)
        step = np.abs(ref) / 8 + scales[b, first:first + T // m, None] * 2.0 ** -9
        assert np.all(np.abs(got - ref) <= step * 1.0001)
        flips = np.abs(got - ref) > 1e-5 * np.abs(ref).max(axis=1, keepdims=True)
        assert flips.mean() <= 0.02, f"b={b}: {flips.mean():.3f} codes differ"
        # rows outside the written range are untouched
        assert np.all(codes[b, :first] == 0) and np.all(codes[b, first + T // m:] == 0)


@pytest.mark.parametrize("which", ["flash_bf16", "pro_e4m3"])
def test_fused_topk_fallback_when_the_wait_gives_up(gpu_lib, which):
    """With a poll budget of zero every waiting scoring workgroup gives up at
    once and flags its row; the resolve then rebuilds each row's selection
    from its scores.  Results must still match the oracle, and every kernel
    exits normally."""
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import DecodeSession
    if which == "flash_bf16":
        g = workloads.flash_csa_decode(seed=71, B=4, n=4 * 20000, H=64, c=512, H_I=64, d_I=128, k=512)
    else:
        g = workloads.pro_csa_decode(seed=72, B=2, n=4 * 30000, H=128, c=512, H_I=64, d_I=128, k=1024)
    prev = L.set_fused_wait_polls(0)
    try:
        sess = DecodeSession(g)
        sess.run()
        torch.cuda.synchronize()
    finally:
        L.set_fused_wait_polls(prev)
    _check_decode(g, sess, f"fallback-{which}")
    # the same session again with the default budget: the workspace was left
    # clean by the fallback
    sess.state.n_entries.copy_(torch.from_numpy(g["n_entries"]).cuda())
    sess.run()
    _check_decode(g, sess, f"after-fallback-{which}")


def test_prefill_csa_mfma_indexer(gpu_lib):
    """64 indexer heads of dim 128 (bf16) and 2 x 64 queries: more rows than
    the decode selection takes, so the MFMA prefill scorer runs (checked via
    the timing hook) over two 1024-entry chunks, the last a ragged tile; every
    query checked against the oracle."""
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import PrefillSession
    a, _ = workloads.flash_prefill(seed=35, B=2, T=64, n0=4500, H=64, c=512, H_I=64, d_I=128, k=64,
                                   m_hca=128)
    sess = PrefillSession(a)
    L.profile_enable(True)
    try:
        L.profile_collect()
        sess.run()
        torch.cuda.synchronize()
        ran = L.profile_collect()
    finally:
        L.profile_enable(False)
    assert "index_score_prefill" in ran, f"prefill scorer did not run: {sorted(ran)}"
    for b in range(2):
        _check_prefill_b(a, sess, b)


def _check_prefill_b(g, sess, b):
    from tests.compare import prefill_err, topk_check
    out = f64(sess.io["out"])
    kv_new, idx_new = OL.prefill_entries(g, b)
    ids = sess.io["topk_idx"][b].cpu().numpy()
    cnt = sess.io["topk_cnt"][b].cpu().numpy()
    for i in range(g["T"]):
        ref = OL.prefill_query(g, b, i, kv_new, idx_new)
        ok, swaps, msg = topk_check(ids[i], cnt[i], ref["sel"], ref["scores"], g["k"],
                                    err=prefill_err(g, b, i, idx_new, len(ref["scores"])))
        assert ok, f"b={b} q{i}: {msg}"
        if swaps:
            ref = OL.prefill_query(g, b, i, kv_new, idx_new, selected=ids[i, :cnt[i]])
        assert_close(out[b, i], ref["o"], "bf16", f"prefill b={b} q{i}")


def _bits_of(io, names):
    return {n: io[n].view(torch.uint8).cpu().numpy().copy() if io[n].dtype != torch.uint8
            else io[n].cpu().numpy().copy() for n in names if io.get(n) is not None}


@pytest.mark.parametrize("which", ["pro_csa", "flash_csa", "flash_hca", "flash_hca_nofold"])
def test_decode_is_deterministic(gpu_lib, which):
    """The same decode step run three times from the same state gives
    bit-identical outputs, lse, top-k and stored entries."""
    from sparse_attention_csa_amd.harness import DecodeSession
    if which == "pro_csa":
        g = workloads.pro_csa_decode(seed=81, B=4, n=4 * 30000, H=128, c=512, H_I=64, d_I=128, k=1024)
    elif which == "flash_csa":
        g = workloads.flash_csa_decode(seed=82, B=8, n=4 * 8192, H=64, c=512, H_I=64, d_I=128, k=512)
    elif which == "flash_hca":
        g = workloads.flash_hca_decode(seed=83, B=8, n=128 * 600, H=64, c=512)
    else:
        g = workloads.flash_hca_decode(seed=84, B=8, n=128 * 600, H=64, c=512, pos_off=9)
    sess = DecodeSession(g)
    names = ("out", "lse", "topk_idx", "topk_cnt")
    runs = []
    for _ in range(3):
        sess.state.n_entries.copy_(torch.from_numpy(g["n_entries"]).cuda())
        sess.run()
        torch.cuda.synchronize()
        r = _bits_of(sess.io, names)
        r["kv"] = sess.state.kv_cache.view(torch.uint8)[:, -1].cpu().numpy().copy()
        runs.append(r)
    for r in runs[1:]:
        for n in runs[0]:
            assert np.array_equal(r[n], runs[0][n]), f"{which}: {n} differs between runs"
    _check_decode(g, sess, f"determinism-{which}")


def test_prefill_is_deterministic(gpu_lib):
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill(seed=85, B=1, T=512, n0=8192, H=64, c=512, H_I=64, d_I=128, k=128)
    for g in (a, h):
        res = []
        for _ in range(2):
            sess = PrefillSession(g)
            sess.run()
            torch.cuda.synchronize()
            res.append(_bits_of(sess.io, ("out", "lse", "topk_idx", "topk_cnt")))
        for n in res[0]:
            assert np.array_equal(res[0][n], res[1][n]), f"prefill {g['kind']}: {n} differs"


@pytest.mark.parametrize("m,in_dt,out_dt,lw,bias", [(128, "bf16", "bf16", "c", True), (128, "f32", "f32", "c", False),
                                                    (32, "bf16", "f32", "1", True), (64, "f32", "bf16", "1", False)])
def test_compress_long_blocks(gpu_lib, m, in_dt, out_dt, lw, bias):
    """csa_compress of long one-branch blocks (the HCA shape; the sliced
    compressor, four wavefronts splitting each coordinate's sources): f32 /
    bf16 inputs and outputs, per-coordinate or scalar logits, with and
    without positional biases, written at an offset into a larger cache,
    against the oracle's fold of the same stored inputs."""
    from sparse_attention_csa_amd import _lib as L
    rng = np.random.default_rng(61 + m)
    B, c, n_ent, first, E_cap = 2, 512, 6, 3, 12
    T = m * n_ent
    zw = c if lw == "c" else 1
    ca = rng.standard_normal((B, T, c)).astype(np.float32)
    za = (2.0 * rng.standard_normal((B, T, zw))).astype(np.float32)
    if in_dt == "bf16":
        ca_s, za_s = workloads.gen.bf16_bits(ca), workloads.gen.bf16_bits(za)
        d_ca, d_za = _dev_bf16(ca_s), _dev_bf16(za_s)
        ca = np.stack([Stored(ca_s[b], "bf16").all() for b in range(B)])
        za = np.stack([Stored(za_s[b], "bf16").all() for b in range(B)])
    else:
        d_ca, d_za = torch.from_numpy(ca).cuda(), torch.from_numpy(za).cuda()
    ba = rng.standard_normal((m, c)).astype(np.float32) if bias else None
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    out = torch.zeros((B, E_cap, c), dtype=odt, device="cuda")
    L.csa_compress(d_ca, d_za, m, bias_a=torch.from_numpy(ba).cuda() if bias else None, out=out,
                   out_first_entry=first)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    for b in range(B):
        ref = OC.compress(ca[b], za[b], m, ba)
        g = got[b, first:first + n_ent]
        err = np.abs(g - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert err.max() <= (1e-5 if out_dt == "f32" else 2.0 ** -8), f"b={b}: row errors {err}"
        assert np.all(got[b, :first] == 0) and np.all(got[b, first + n_ent:] == 0)
