"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (DecodeSession / PrefillSession through the C ABI).

Decode workloads are checked on every sequence (the oracle scores all visible
entries of a sequence in float64 in a few seconds); the prefill workload is
checked on sampled queries (first, last and spread between, including block
boundaries), with the chunk's compressed entries checked in full."""

import numpy as np
import pytest
import torch

import workloads
from tests.test_gpu_parity import _check_decode, _check_prefill

pytestmark = pytest.mark.gpu


def _run_decode(g, label):
    from sparse_attention_csa_amd.harness import DecodeSession
    print(f"[{label}] upload", flush=True)
    sess = DecodeSession(g)
    sess.run()
    torch.cuda.synchronize()
    print(f"[{label}] compare", flush=True)
    swaps = _check_decode(g, sess, label)
    print(f"[{label}] ok, tie swaps: {swaps}", flush=True)


def test_flash_csa_decode_128k(gpu_lib):
    _run_decode(workloads.flash_csa_decode(), "flash-csa-128k")


def test_flash_hca_decode_1m(gpu_lib):
    _run_decode(workloads.flash_hca_decode(), "flash-hca-1m")


def test_pro_csa_decode_1m_fp8_indexer(gpu_lib):
    _run_decode(workloads.pro_csa_decode(), "pro-csa-1m")


def test_flash_prefill_4096_on_256k(gpu_lib):
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill()
    T = a["T"]
    sample = sorted(set([0, 1, 3, 4, 127, 128, 1000, 2047, 2048, T - 129, T - 128, T - 2, T - 1]))
    for g, label in ((a, "prefill-csa"), (h, "prefill-hca")):
        print(f"[{label}] upload", flush=True)
        sess = PrefillSession(g)
        sess.run()
        torch.cuda.synchronize()
        print(f"[{label}] compare {len(sample)} queries", flush=True)
        _check_prefill(g, sess, label, queries=sample)
        del sess
        torch.cuda.empty_cache()
