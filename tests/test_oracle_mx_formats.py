"""Pins for the oracle's low-precision formats (the pages' FP4 indexer path,
the 576-byte main entry, bf16 index scores): format tables, torch's own
E8M0 conversion, hand-computed blocks, the pages' byte counts, and two
independent MXFP4 encoders (oracle and input generator) agreeing."""

import math

import numpy as np
import torch

import workloads
from oracle import csa
from oracle import formats as F


def test_e2m1_decoder_matches_the_format_table():
    # OCP MX E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7), sign bit 3
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = F.e2m1_to_f64(np.arange(16))
    assert list(got[:8]) == table
    assert list(got[8:]) == [-v for v in table]


def test_e8m0_decoder_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(F.e8m0_to_f64(codes), ref)
    assert np.isnan(F.e8m0_to_f64(np.array([255]))[0])


def test_mxfp4_blocks_by_hand():
    b1 = np.zeros(32)
    b1[:8] = [6.0, 3.0, -1.5, 0.25, 0.75, 5.0, 1.25, -2.5]
    # amax 6: floor(log2 6) = 2, scale 2**0; 0.25 -> 0 and 0.75 -> 1 (ties
    # to the even code), 5 -> 4, 1.25 -> 1, -2.5 -> -2
    b2 = np.full(32, 0.1)
    b2[3] = 7.0  # amax 7: scale 1, 7 saturates to 6; 0.1 -> 0
    b3 = np.full(32, 0.1)  # amax 0.1: floor(log2 0.1) = -4, scale 2**-6; 6.4 -> 6
    b4 = np.zeros(32)  # all zero: zero codes, smallest scale
    x = np.concatenate([b1, b2, b3, b4])
    packed, scales, vals = F.mxfp4_quantize(x)
    assert list(scales) == [127, 127, 127 - 6, 0]
    assert list(vals[:8]) == [6.0, 3.0, -1.5, 0.0, 1.0, 4.0, 1.0, -2.0]
    assert vals[32 + 3] == 6.0 and np.all(np.delete(vals[32:64], 3) == 0.0)
    assert np.allclose(vals[64:96], 6 * 2.0 ** -6)
    assert np.all(vals[96:] == 0.0)
    # the round trip through the packed bytes
    assert np.array_equal(F.mxfp4_decode(packed, scales), vals)
    assert packed.shape == (64,)


def test_mxfp4_error_bound_and_full_range():
    """Away from saturation each element is within half an E2M1 step of the
    value (step 0.5, 1, 2 times the block scale); the block maximum uses the
    top of the range."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128)) * np.exp(rng.standard_normal((50, 1)) * 3)
    _, scales, v = F.mxfp4_quantize(x)
    s = np.repeat(F.e8m0_to_f64(scales), 32, axis=-1)
    a = np.abs(x) / s
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    ok = a <= 6
    assert np.all(np.abs(v - x)[ok] <= 0.5 * step[ok] * s[ok] + 1e-300)
    amax = np.abs(x).reshape(50, 4, 32).max(-1) / F.e8m0_to_f64(scales)
    assert np.all((amax >= 4) & (amax < 8))


def test_two_independent_mxfp4_encoders_agree():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    p1, s1, _ = F.mxfp4_quantize(x.astype(np.float64))
    p2, s2 = workloads.gen.mxfp4_rows(x)
    assert np.array_equal(s1, s2) and np.array_equal(p1, p2)


def test_pages_byte_counts():
    """An FP4 key of 128 values: 64 bytes plus four one-byte scales for
    groups of 32; the main entry: 448 FP8 + 64 BF16 = 576 bytes (book ch. 8)."""
    p, s, _ = F.mxfp4_quantize(np.ones(128))
    assert p.nbytes == 64 and s.nbytes == 4
    rows, sc = workloads.gen.fp8bf16_rows(np.ones((3, 512), np.float32))
    assert rows.shape == (3, 576) and sc.shape == (3,)


def test_fp8bf16_entry_decode_and_store():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    rows, sc = workloads.gen.fp8bf16_rows(x)
    got = F.Stored(rows, "fp8bf16", sc).all()
    head = torch.from_numpy(np.clip(x[:, :448] / sc[:, None], -448, 448)).to(torch.float8_e4m3fn)
    ref_head = head.to(torch.float64).numpy() * sc.astype(np.float64)[:, None]
    ref_tail = torch.from_numpy(x[:, 448:]).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got[:, :448], ref_head) and np.array_equal(got[:, 448:], ref_tail)
    # the oracle's own rounding of produced entries matches the stored form
    assert np.array_equal(csa.store_as(x.astype(np.float64), "fp8bf16"), got)


def test_bf16_scores_select_the_lower_id_on_a_rounded_tie():
    """Two scores apart in float32 but equal once rounded to bf16: the
    selection on bf16 scores takes the lower id, the float32 one the
    larger score."""
    rng = np.random.default_rng(3)
    kv = F.Stored(rng.standard_normal((8, 4)).astype(np.float32), "f32")
    K = np.zeros((8, 2), np.float32)
    K[:, 0] = [1.0, 2.0, 3.0, 1.001, 0.5, 0.25, 0.1, 0.2]  # scores 1.0 and 1.001 share a bf16 value
    keys = F.Stored(K, "f32")
    q = np.ones((1, 4))
    qi = np.array([[1.0, 0.0]])
    w = np.array([1.0])
    win = lambda p: np.zeros((len(p), 4))  # noqa: E731
    _, _, sel32, _ = csa.csa_query(q, qi, w, 4 * 8, kv, keys, 8, win, None, 4, 3, 1, 0.5)
    _, _, sel16, sc16 = csa.csa_query(q, qi, w, 4 * 8, kv, keys, 8, win, None, 4, 3, 1, 0.5, score_dtype="bf16")
    assert list(sel32) == [1, 2, 3] and list(sel16) == [0, 1, 2]
    assert sc16[0] == sc16[3] == 1.0
