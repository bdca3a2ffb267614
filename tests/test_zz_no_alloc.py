"""csa_attend_noalloc (the entry point that brings its own static scratch)
against csa_attend with a caller workspace, through the C ABI.

Calls in a row on one GPU share the library's scratch: a CSA decode shape
with split partials (bf16 kernel and merge), then a smaller one, then fp32
rows whose splits are merged by the last arriving workgroup (which uses the
scratch's arrival counters), then a smaller fp32 call.  Each output must
equal csa_attend's bit for bit: the same kernels run on the same inputs with
the same plan.
"""
import math

import numpy as np
import pytest
import torch

import compressed_attention_csa_amd as csa
import inputgen

pytestmark = pytest.mark.gpu
DEV = "cuda"

# name, dtype, B, T, H, d, N, k, W
CASES = [
    ("bf16-decode-large", "bf16", 4, 1, 128, 128, 3000, 1024, 128),
    ("bf16-decode-small", "bf16", 2, 1, 64, 128, 700, 256, 64),
    ("f32-decode-large", "f32", 3, 1, 8, 64, 3000, 1024, 128),
    ("f32-decode-small", "f32", 1, 1, 4, 64, 900, 100, 16),
]


def make(case, seed):
    name, dt, B, T, H, d, N, k, W = case
    m = 4
    t0 = m * N - 1
    n_raw = W + T
    g = lambda nm, shape, std=1.0: inputgen.normal(nm, shape, seed, dt, std=std, device=DEV)
    q = g("na_q", (B, T, H, d))
    kc, vc = g("na_kc", (B, N, d), 0.6), g("na_vc", (B, N, d), 0.6)
    kr, vr = g("na_kr", (B, n_raw, d)), g("na_vr", (B, n_raw, d))
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(B * T)]).reshape(B, T, k).astype(np.int32)
    idx[:, :, :5] = -1  # some skipped slots
    return dict(q=q, kc=kc, vc=vc, kr=kr, vr=vr, idx=torch.from_numpy(idx).to(DEV), m=m, t0=t0, W=W,
                raw_base=t0 - W + 1, scale=1.0 / math.sqrt(d))


def run(x, noalloc):
    B, T, H, d = x["q"].shape
    out = torch.full((B, T, H, d), 7.0, dtype=torch.float32, device=DEV)
    lse = torch.full((B, T, H), 7.0, dtype=torch.float32, device=DEV)
    args = (x["q"], x["kc"], x["vc"], x["m"], x["idx"], x["kr"], x["vr"], x["t0"], x["W"], x["scale"], out, lse)
    if noalloc:
        csa.csa_attend_noalloc(*args, raw_base=x["raw_base"])
    else:
        csa.csa_attend(*args, raw_base=x["raw_base"])
    return out, lse


def test_noalloc_matches_workspace_entry_point_over_consecutive_calls():
    for i, case in enumerate(CASES):
        print("csa_attend_noalloc", case, flush=True)
        x = make(case, seed=40 + i)
        o_na, l_na = run(x, True)
        o_ws, l_ws = run(x, False)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), f"{case[0]}: outputs differ"
        assert torch.equal(l_na, l_ws), f"{case[0]}: lse differ"
        assert torch.isfinite(o_na).all()


def test_noalloc_rejects_shapes_beyond_its_scratch():
    B = 200  # decode rows whose split partials exceed the scratch
    assert csa.lib().csa_attend_workspace(B, 1, 128, 128, 1024, 128) > (16 << 20)
    x = make(("big", "bf16", B, 1, 128, 128, 2000, 1024, 128), seed=9)
    with pytest.raises(csa.CsaError, match="CSA_E_WORKSPACE"):
        run(x, True)
