"""GPU parity of variable-length prefill batches ("DeepSeek-V4" book ch. 11
"Packing and attention boundaries": compression blocks never span two
samples, and a trailing fragment shorter than the compression rate makes no
entry; ch. 13 "What to measure in a server": exact-prefix continuation).

Each sequence of a batch takes its own chunk start and length: two
variable-length chunks (lengths that are not multiples of m, one empty, one
of a single token, chunks that start inside a block), then decode steps from
each sequence's own position, all on the library's state.  The oracle
answers the same token data as one aligned chunk: a query's answer depends
only on the tokens up to it, so chunking must not change it.  Checked:
every produced entry (the chunks' blocks that end inside them, built from
tail and chunk tokens), every query's top-k set and output, the entry
counts, and the decode steps after."""

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as OL
from tests.cases import decode_from_prefill, varlen_chunk
from tests.compare import assert_close, check_selection, decode_err, prefill_err
from tests.test_gpu_parity import f64

pytestmark = pytest.mark.gpu


def _pad4(n):
    return max(4, -(-int(n) // 4) * 4)


@pytest.mark.parametrize("kind,variant", [("csa", None), ("hca", None), ("csa", "norm_rope"), ("hca", "norm_rope"),
                                          ("csa", "paged"), ("hca", "paged")])
def test_two_varlen_chunks_then_decode(gpu_lib, kind, variant):
    """variant: norm_rope (queries, window rows and entries prepared at
    each sequence's own positions) or paged (the state's caches in pages of
    one 128-token unit)."""
    from sparse_attention_csa_amd.harness import PrefillSession
    from tests.test_gpu_continuation import _stack_steps
    B, n0, steps = 3, 1024, 12
    if kind == "csa":
        L1, L2 = [5, 128, 0], [130, 3, 67]      # m = 4: fragments of 1, 3 and 3 tokens
    else:
        L1, L2 = [100, 256, 0], [190, 2, 300]   # m = 128: chunks inside blocks
    Ttot = -(-(max(a + b for a, b in zip(L1, L2)) + steps) // 128) * 128  # (the aligned chunk: whole blocks)
    a, h = workloads.flash_prefill(seed=171, B=B, T=Ttot, n0=n0, H=64, c=512, H_I=64, d_I=128, k=128)
    full = a if kind == "csa" else h
    if variant == "norm_rope":
        full = workloads.with_norm_rope(full, seed=172)
    m = full["m"]
    label = f"varlen-{kind}-{variant}"
    kv_full, idx_full = zip(*[OL.prefill_entries(full, b) for b in range(B)])
    E0 = int(full["n_entries"][0])

    c1 = varlen_chunk(full, [0] * B, L1, _pad4(max(L1)))
    if variant == "paged":
        c1 = workloads.with_pages(c1, 32 if kind == "csa" else 1, seed=173)
    sess = PrefillSession(c1)
    sess.run()
    io1 = sess.io
    io2 = sess.prefill(varlen_chunk(full, L1, L2, _pad4(max(L2))))
    torch.cuda.synchronize()
    print(f"[{label}] chunks {L1} + {L2} done", flush=True)

    Ls = [x + y for x, y in zip(L1, L2)]
    n_ent = sess.state.n_entries.cpu().numpy()
    for b in range(B):
        n_b = (n0 + Ls[b]) // m
        assert n_ent[b] == n_b, f"{label} b={b}: {n_ent[b]} entries, want {n_b}"
        got = f64(sess.state.kv_cache[b, E0:n_b])
        assert_close(got, kv_full[b][:n_b - E0], "bf16", f"{label} entries b={b}")
        if kind == "csa":
            assert_close(f64(sess.state.idx_cache[b, E0:n_b]), np.asarray(idx_full[b][:n_b - E0]), "bf16",
                         f"{label} keys b={b}")
    # every query of both chunks against the oracle's answer for its position
    n_q = 0
    for io, offs, lens in ((io1, [0] * B, L1), (io2, L1, L2)):
        out = f64(io["out"])
        lse = f64(io["lse"])
        for b in range(B):
            for r in range(lens[b]):
                i = offs[b] + r  # the token's index in the aligned chunk
                ref = OL.prefill_query(full, b, i, kv_full[b], idx_full[b] if kind == "csa" else None)
                if kind == "csa":
                    ids = io["topk_idx"][b, r].cpu().numpy()
                    cnt = int(io["topk_cnt"][b, r])
                    ok, swaps, msg = check_selection(ids, cnt, full["k"], ref,
                                                     prefill_err(full, b, i, idx_full[b], len(ref["scores"])))
                    assert ok, f"{label} b={b} token {i}: {msg}"
                    if swaps:
                        ref = OL.prefill_query(full, b, i, kv_full[b], idx_full[b], selected=ids[:cnt])
                assert_close(out[b, r], ref["o"], "bf16", f"{label} b={b} token {i} out")
                assert np.abs(lse[b, r] - ref["lse"]).max() < 1e-3, f"{label} b={b} token {i} lse"
                n_q += 1
    print(f"[{label}] {n_q} chunk queries ok", flush=True)

    # decode steps from each sequence's own position
    extra_kv = [[] for _ in range(B)]
    extra_idx = [[] for _ in range(B)]
    for j in range(steps):
        gs = []
        for b in range(B):
            t = n0 + Ls[b] + j
            n_pre = (n0 + Ls[b]) // m - E0
            gs.append(decode_from_prefill(full, None, kv_full[b][:n_pre],
                                          idx_full[b][:n_pre] if kind == "csa" else (), t,
                                          extra_kv[b], extra_idx[b], b=b))
        io = sess.decode(_stack_steps(gs))
        torch.cuda.synchronize()
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
                assert ok, f"{label} decode j={j} b={b}: {msg}"
                if swaps:
                    ref = OL.decode_step(gs[b], 0, selected=ids[:cnt])
            assert_close(o[b], ref["o"], "bf16", f"{label} decode j={j} b={b}")
    n_ent = sess.state.n_entries.cpu().numpy()
    for b in range(B):
        assert n_ent[b] == (n0 + Ls[b] + steps - 1) // m, f"{label} entries after decode b={b}"
    print(f"[{label}] {steps} decode steps ok", flush=True)
