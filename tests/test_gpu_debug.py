"""Parity cases through libcsa_debug.so, the CSA_DEBUG build (through the C ABI).

That build fills the scratch part of every workspace, and every kernel's LDS,
with all-ones words (NaN as fp32 and as bf16) before the kernels run, and
checks the launch plans on the host.  A kernel that read scratch or LDS that
nothing had written would carry NaN (or a wild value) into its results, so
these cases, which pass the same criteria as the release build's, show that
every kernel writes such memory before reading it.  Every loop is bounded by
sizes alone, so poisoned values cannot change how long a kernel runs.  The
cases cover each kernel: compressor and append, decode and prefill indexer
(bf16, e4m3, f32 keys, fp8 query, bf16 scores), split and unsplit attention,
the multi-token HCA kernel, fp8 caches.
"""
import os
import subprocess
import sys

import pytest
import torch

import compressed_attention_csa_amd as csa
import test_gpu_parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def debug_library():
    with csa.use_library(csa.DEBUG_LIB_PATH):
        yield
    torch.cuda.synchronize()


def test_the_debug_build_is_in_use():
    # Both libraries export the same ABI; the debug one is a separate file.
    assert csa.lib()._name == csa.DEBUG_LIB_PATH
    assert csa.lib().csa_abi_version() == csa.load(csa.LIB_PATH).csa_abi_version()


@pytest.mark.parametrize("case", [P.COMPRESS_CASES[i] for i in (0, 2, 4, 6)], ids=lambda c: f"{c[0]}-{c[1]}-m{c[2]}")
def test_compress(case):
    P.test_compress(case)


@pytest.mark.parametrize("case", P.OVERLAP_CASES[:2], ids=lambda c: f"m{c[2]}-o{c[3]}")
def test_compress_with_overlapping_blocks(case):
    P.test_compress_with_overlapping_blocks(case)


@pytest.mark.parametrize("case", P.APPEND_CASES[:2], ids=lambda c: str(c[:3]))
def test_append(case):
    P.test_append_builds_the_caches_of_the_full_history(case)


INDEX = [P.INDEX_CASES[i] for i in (0, 1, 3, 5, 8, 9, 10, 11, 13, 15)]


@pytest.mark.parametrize("case", INDEX, ids=lambda c: f"{c[0]}-B{c[1]}T{c[2]}-N{c[5]}-k{c[8]}")
def test_index_topk(case):
    P.test_index_topk(case)


@pytest.mark.parametrize("case", [P.FP8Q_CASES[i] for i in (0, 3)], ids=lambda c: f"T{c[2]}-N{c[5]}")
def test_index_topk_fp8_query(case):
    P.test_index_topk_fp8_query(case)


@pytest.mark.parametrize("case", [P.BF16_SEL_CASES[i] for i in (0, 3)], ids=lambda c: f"T{c[2]}-N{c[5]}")
def test_index_topk_bf16_selector(case):
    P.test_index_topk_bf16_selector(case)


def test_index_topk_winners_concentrated_in_few_slices():
    P.test_index_topk_winners_concentrated_in_few_slices("e4m3")


def test_index_topk_prefill_sampled_threshold_falls_back():
    P.test_index_topk_prefill_sampled_threshold_falls_back()


ATTEND = [c for c in P.ATTEND_CASES if c[0] in (
    "csa-decode", "csa-prefill", "csa-empty-rows", "csa-f32", "csa-f32-decode", "hca-f32-h13-decode",
    "csa-f32-h2-d32", "hca-decode-b16",
    "hca-prefill", "hca-prefill-multi", "hca-prefill-multi-h128-d64", "csa-max-k-window")]


@pytest.mark.parametrize("case", ATTEND, ids=lambda c: c[0])
def test_attend(case):
    P.test_attend(case)


@pytest.mark.parametrize("case", [c for c in P.FP8_KV_CASES if c[0] in ("csa-decode", "hca-prefill-multi")],
                         ids=lambda c: c[0])
def test_attend_with_fp8_compressed_caches(case):
    P.test_attend_with_fp8_compressed_caches(case)


def test_tiny_prefill_f32_end_to_end():
    P.test_tiny_prefill_f32_end_to_end()


LOG_SCRIPT = """
import torch, compressed_attention_csa_amd as csa
q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
k = torch.zeros((1, 5000, 64), dtype=torch.bfloat16, device="cuda")
out = torch.empty((1, 1, 16), dtype=torch.int32, device="cuda")
csa.csa_index_topk(q, None, k, None, 4 * 5000 - 1, 4, 16, out)
torch.cuda.synchronize()
"""


def test_dispatch_log():
    """CSA_LOG=1 prints every launch decision to stderr (a child process, so that
    the setting does not reach the rest of the session)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, CSA_LOG="1", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", LOG_SCRIPT], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "[csa] index_topk: B=1 T=1 H_I=8 d_I=64 N=5000 k=16 keys=bf16 -> rows x slices path" in r.stderr
    assert "slices of" in r.stderr
