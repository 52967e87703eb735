"""GPU parity of the paged compressed cache ("DeepSeek-V4" book ch. 13
"Aligning original-token blocks"): the layer's compressed entries, indexer
keys and their scales live in pages of a pool that all sequences share,
found through a block table.  With one 128-token unit per table slot a CSA
layer's page holds 32 entries (m = 4) and an HCA layer's one (m = 128), so
the cases below give a CSA and an HCA layer one and the same table.  Pages
sit in a seeded random order, and pool rows that no sequence owns hold
all-ones bytes (NaN in every float format), so a row read from the wrong
place shows.

Every case is checked twice: against the oracle with the rules of the
per-sequence layout (tests/compare.py), and bit for bit against the same
case run on the per-sequence layout (paging moves rows, not arithmetic):
outputs, lse, top-k ids and counts, and the entries a call appends."""

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as OL
from tests.cases import decode_from_prefill, prefix_case
from tests.compare import assert_close, check_selection, decode_err
from tests.test_gpu_parity import _check_decode, _check_prefill, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["fused-fold", "fold-kernel"])
def _fold_path(request, gpu_lib):
    """Each case twice: the decode fold inside the scan / the dense
    attention where the step allows it (the default), and in the separate
    fold kernel; both layouts take the same path, so their results compare
    bit for bit."""
    from sparse_attention_csa_amd import _lib as L
    prev = L.set_fold_fusion(request.param == "fused-fold")
    yield request.param
    L.set_fold_fusion(prev)


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def _same_io(io_a, io_b, label):
    for name in ("out", "lse", "topk_idx", "topk_cnt"):
        if io_a.get(name) is None:
            continue
        assert np.array_equal(_bits(io_a[name]), _bits(io_b[name])), f"{label}: {name} differs from the per-sequence layout"


def _same_entries(st_a, st_b, n_ent, label):
    """The entries both states hold (the first n_ent of each sequence), bit for bit."""
    for name in ("kv_cache", "kv_scale", "idx_cache", "idx_scale"):
        a, b = getattr(st_a, name), getattr(st_b, name)
        if a is None:
            continue
        for s in range(a.shape[0]):
            n = int(n_ent[s])
            assert np.array_equal(_bits(a[s, :n]), _bits(b[s, :n])), f"{label}: {name} of sequence {s}"


def _decode_both(g, gp, label, same_path=True):
    """same_path: both layouts run the same kernels (else, as for pages
    the scan's paged form does not take, only the oracle's checks apply)."""
    from sparse_attention_csa_amd.harness import DecodeSession
    paged = DecodeSession(gp)
    flat = DecodeSession(g)
    paged.run()
    flat.run()
    torch.cuda.synchronize()
    _check_decode(gp, paged, label)
    if same_path:
        _same_io(paged.io, flat.io, label)
        _same_entries(paged.state, flat.state, flat.state.n_entries.cpu().numpy(), label)
    return paged


@pytest.mark.parametrize("idx,pos_off", [("bf16", 0), ("e4m3", 0), ("e4m3", 2), ("mxfp4", 1)])
def test_decode_csa_and_hca_share_one_block_table(gpu_lib, idx, pos_off):
    """A CSA layer (pages of 32 entries; the scan's paged form for bf16, e4m3
    and MXFP4 keys, the sparse gather's) and an HCA layer (pages of one
    entry; the dense kernel's paged form) of the same 2 x 12,032-token
    sequences, through one table of 95 units."""
    B, n, nb = 2, 128 * 94, 95
    table, n_pages = workloads.block_table(B, nb, seed=160 + pos_off)
    if idx == "bf16":  # (the Flash-shaped case: bf16 keys, a fold in the step)
        csa = workloads.flash_csa_decode(seed=161, B=B, n=n, H=64, c=512, H_I=64, d_I=128, k=256)
    else:
        csa = workloads.pro_csa_decode(seed=161, B=B, n=n, H=128, c=512, H_I=64, d_I=128, k=256, idx_dtype=idx,
                                       score_dtype="bf16" if idx == "mxfp4" else "f32", pos_off=pos_off)
    hca = workloads.flash_hca_decode(seed=162, B=B, n=n, H=64, c=512, pos_off=pos_off)
    _decode_both(csa, workloads.with_pages(csa, 32, table, n_pages), f"paged-csa-{idx}-{pos_off}")
    _decode_both(hca, workloads.with_pages(hca, 1, table, n_pages), f"paged-hca-{pos_off}")


@pytest.mark.parametrize("kind,P", [("csa", 16), ("csa", 8), ("hca", 4), ("hca", 256), ("fp8bf16", 32)])
def test_decode_other_page_sizes(gpu_lib, kind, P, _fold_path):
    """Pages of 16 CSA entries (the smallest the scan's paged form takes),
    8 (the VALU scorer), 4 and 256 HCA entries (an allocation unit of
    several 128-token groups), and the 576-byte FP8 + BF16 entry (the
    generic attention kernel) in pages of 32."""
    if kind == "hca":
        g = workloads.flash_hca_decode(seed=163, B=3, n=128 * 300, H=64, c=512)
    else:
        g = workloads.pro_csa_decode(seed=164, B=2, n=4 * 3000, H=128, c=512, H_I=64, d_I=128, k=256)
        if kind == "fp8bf16":
            g = workloads.with_fp8bf16_cache(g)
    # (pages of 8 entries go to the VALU scorer and the fold kernel, while
    # the per-sequence layout may fold inside the scan)
    same = not (kind == "csa" and P < 16 and _fold_path == "fused-fold")
    _decode_both(g, workloads.with_pages(g, P, seed=165 + P), f"paged-{kind}-{P}", same)


def test_prefill_csa_and_hca_share_one_block_table(gpu_lib):
    """A 256-token chunk after 1024 tokens: the chunk's entries written into
    pages by the compressor, scored by the prefill scorer's paged form and
    gathered by the attention kernels' paged forms, both layers on one
    table of 11 units."""
    from sparse_attention_csa_amd.harness import PrefillSession
    B, nb = 2, 11
    table, n_pages = workloads.block_table(B, nb, seed=166)
    a, h = workloads.flash_prefill(seed=167, B=B, T=256, n0=1024, H=64, c=512, H_I=64, d_I=128, k=128)
    for g, P, label in ((a, 32, "paged-prefill-csa"), (h, 1, "paged-prefill-hca")):
        gp = workloads.with_pages(g, P, table, n_pages)
        paged, flat = PrefillSession(gp), PrefillSession(g)
        paged.run()
        flat.run()
        torch.cuda.synchronize()
        _check_prefill(gp, paged, label)
        _same_io(paged.io, flat.io, label)
        _same_entries(paged.state, flat.state, flat.state.n_entries.cpu().numpy(), label)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_prefill_then_decode_paged(gpu_lib, kind):
    """A chunk, then 40 decode steps on the library's own paged state (the
    fold kernel appends entries through the table, later steps read them):
    every step against the oracle, and bit for bit against the same steps
    on the per-sequence layout."""
    from sparse_attention_csa_amd.harness import PrefillSession
    from tests.test_gpu_continuation import _stack_steps
    B, n0, T0, steps = 2, 2048, 128, 40
    a, h = workloads.flash_prefill(seed=168, B=B, T=T0 + steps, n0=n0, H=64, c=512, H_I=64, d_I=128, k=128)
    full = a if kind == "csa" else h
    pre = prefix_case(full, T0)
    table, n_pages = workloads.block_table(B, -(-(n0 + T0 + steps) // 128) + 1, seed=169)
    prep = workloads.with_pages(pre, 32 if kind == "csa" else 1, table, n_pages)
    paged, flat = PrefillSession(prep), PrefillSession(pre)
    paged.run()
    flat.run()
    torch.cuda.synchronize()
    _same_io(paged.io, flat.io, f"paged-cont-{kind} prefill")
    kv_new, idx_new = zip(*[OL.prefill_entries(pre, b) for b in range(B)])
    extra_kv = [[] for _ in range(B)]
    extra_idx = [[] for _ in range(B)]
    for j in range(steps):
        t = n0 + T0 + j
        gs = [decode_from_prefill(full, T0, kv_new[b], idx_new[b] if kind == "csa" else (), t, extra_kv[b],
                                  extra_idx[b], b=b) for b in range(B)]
        step = _stack_steps(gs)
        io = paged.decode(step)
        io_flat = flat.decode(step)
        torch.cuda.synchronize()
        _same_io(io, io_flat, f"paged-cont-{kind} t={t}")
        o = f64(io["out"])
        for b in range(B):
            ref = OL.decode_step(gs[b], 0)
            if ref["folded_kv"]:
                extra_kv[b] += ref["folded_kv"]
                extra_idx[b] += ref["folded_idx"]
            if kind == "csa":
                ids = io["topk_idx"][b].cpu().numpy()
                cnt = int(io["topk_cnt"][b])
                ok, swaps, msg = check_selection(ids, cnt, full["k"], ref, decode_err(gs[b], 0, ref))
                assert ok, f"paged-cont t={t} b={b}: {msg}"
                if swaps:
                    ref = OL.decode_step(gs[b], 0, selected=ids[:cnt])
            assert_close(o[b], ref["o"], "bf16", f"paged-cont-{kind} t={t} out b={b}")
    n_ent = flat.state.n_entries.cpu().numpy()
    assert np.array_equal(n_ent, paged.state.n_entries.cpu().numpy())
    _same_entries(paged.state, flat.state, n_ent, f"paged-cont-{kind} entries")
    print(f"[paged-cont-{kind}] {steps} steps ok, entries {n_ent.tolist()}", flush=True)


def test_full_size_decode_paged_matches_per_sequence_layout(gpu_lib):
    """The bench's decode step at full size (Pro-shaped CSA: 4 x 262,144
    entries, e4m3 keys, k = 1024; Flash-shaped HCA: 8 x 8,192 entries), paged
    in 128-token units: bit for bit the per-sequence layout's results."""
    from sparse_attention_csa_amd.harness import DecodeSession
    for g, P, label in ((workloads.pro_csa_decode(), 32, "full-csa"), (workloads.flash_hca_decode(), 1, "full-hca")):
        print(f"[{label}] build", flush=True)
        gp = workloads.with_pages(g, P, seed=170)
        paged, flat = DecodeSession(gp), DecodeSession(g)
        paged.run()
        flat.run()
        torch.cuda.synchronize()
        _same_io(paged.io, flat.io, label)
        _same_entries(paged.state, flat.state, flat.state.n_entries.cpu().numpy(), label)
        print(f"[{label}] paged = per-sequence layout", flush=True)
        del paged, flat
        torch.cuda.empty_cache()


def test_full_size_prefill_paged_matches_per_sequence_layout(gpu_lib):
    """The 4096-token prefill chunk over a 262,144-token context (both
    layers) with its caches in 128-token pages: bit for bit the per-sequence
    layout's outputs, selections and produced entries; and a second run of
    the paged chunk on a fresh state gives the same bits (run-to-run
    determinism of the paged forms)."""
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill()
    for g, P, label in ((a, 32, "full-prefill-csa"), (h, 1, "full-prefill-hca")):
        print(f"[{label}] build", flush=True)
        gp = workloads.with_pages(g, P, seed=174)
        paged, flat = PrefillSession(gp), PrefillSession(g)
        paged.run()
        flat.run()
        torch.cuda.synchronize()
        _same_io(paged.io, flat.io, label)
        _same_entries(paged.state, flat.state, flat.state.n_entries.cpu().numpy(), label)
        again = PrefillSession(gp)
        again.run()
        torch.cuda.synchronize()
        _same_io(paged.io, again.io, label + " rerun")
        print(f"[{label}] paged = per-sequence layout, rerun identical", flush=True)
        del paged, flat, again
        torch.cuda.empty_cache()

