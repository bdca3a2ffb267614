"""Closed forms of the method, run through the GPU path (through the C ABI).

Each case is a configuration in which the method reduces to something with a
plain definition, computed here on the CPU with torch's attention routine or
NumPy, independently of the oracle:

* m = 1, k at least every visible entry, no window: each compressed entry is its
  token, so CSA (compress, index + top-k, attend) is causal softmax attention;
* k at least every visible entry: CSA with block m attends every visible
  compressed entry plus the window, which is HCA with heavy block m;
* equal compressor logits: every entry is the mean of its block;
* every index -1: CSA is sliding-window attention over the raw rows.

Tolerances are the bf16 attention criterion (2e-3 of the row's largest output,
see parity_util) and, for the compressor, one bf16 step.
"""
import math

import numpy as np
import pytest
import torch

import compressed_attention_csa_amd as csa
import inputgen
from oracle import formats
from parity_util import TOL, f64, ulp_diff_bf16, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gen(name, shape, dtype, seed=0, std=1.0):
    return inputgen.normal(name, shape, seed, dtype, std=std)


def say(*a):
    print(*a, flush=True)


def sdpa(q, k, v, scale, mask):
    """torch's attention on the CPU in float64: q [T, H, d], k / v [S, d] (one KV
    head), mask [T, S] boolean (True = attend)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                       # [1, H, T, d]
    H = q.shape[1]
    kt = torch.from_numpy(k)[None, None].expand(1, H, -1, -1).contiguous()  # [1, H, S, d]
    vt = torch.from_numpy(v)[None, None].expand(1, H, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                                         scale=scale)
    return o[0].permute(1, 0, 2).numpy()                                  # [T, H, d]


def close_rows(o_gpu, o_ref, tol, what):
    err = np.abs(o_gpu - o_ref).max(axis=-1)
    ref = np.abs(o_ref).max(axis=-1)
    worst = float(np.max(err / np.maximum(ref, 1e-30)))
    say(f"  {what}: worst row error {worst:.2e} of the row maximum")
    assert np.all(err <= tol * np.maximum(ref, 1e-30)), f"{what}: {worst:.2e}"


def test_m1_full_selection_no_window_is_causal_attention():
    B, T, H, d, HI, dI = 1, 300, 16, 64, 8, 32
    say("closed form: m = 1, k >= visible, W = 0 -> causal attention")
    x_k = gen("cf1_k", (B, T, d), "bf16", seed=1).to(DEV)
    x_v = gen("cf1_v", (B, T, d), "bf16", seed=2).to(DEV)
    q = gen("cf1_q", (B, T, H, d), "bf16", seed=3).to(DEV)
    q_idx = gen("cf1_qi", (B, T, HI, dI), "bf16", seed=4).to(DEV)
    k_idx = gen("cf1_ki", (B, T, dI), "bf16", seed=5).to(DEV)
    z = torch.zeros(1, device=DEV)
    kc = torch.empty_like(x_k)
    vc = torch.empty_like(x_v)
    csa.csa_compress(x_k, z, 1, kc)
    csa.csa_compress(x_v, z, 1, vc)
    k = 512
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(q_idx, None, k_idx, None, 0, 1, k, idx)
    out = torch.empty((B, T, H, d), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    csa.csa_attend(q, kc, vc, 1, idx, x_k, x_v, 0, 0, scale, out)
    torch.cuda.synchronize()
    assert torch.equal(kc, x_k) and torch.equal(vc, x_v), "m = 1 entries are their tokens"
    sel = idx[0].cpu().numpy()
    for i in range(T):
        assert np.array_equal(np.sort(sel[i, : i + 1]), np.arange(i + 1)) and np.all(sel[i, i + 1:] == -1)
    mask = np.tril(np.ones((T, T), dtype=bool))
    ref = sdpa(f64(q[0]), f64(x_k[0]), f64(x_v[0]), scale, mask)
    close_rows(f64(out[0]), ref, TOL["bf16"], "causal attention")


def test_full_selection_csa_equals_hca_with_the_same_block():
    B, T, H, d, m, W, HI, dI = 2, 40, 64, 128, 4, 128, 8, 64
    t0 = 4000
    n = t0 + T
    N = n // m
    k = 1024  # at least every visible entry: c(t) <= (t0 + T) / 4 = 1010
    say("closed form: k >= visible -> CSA(m) = HCA(m)")
    x_k = gen("cf2_k", (B, n, d), "bf16", seed=11).to(DEV)
    x_v = gen("cf2_v", (B, n, d), "bf16", seed=12).to(DEV)
    q = gen("cf2_q", (B, T, H, d), "bf16", seed=13).to(DEV)
    q_idx = gen("cf2_qi", (B, T, HI, dI), "bf16", seed=14).to(DEV)
    k_idx = gen("cf2_ki", (B, N, dI), "bf16", seed=15).to(DEV)
    z = gen("cf2_z", (m,), "f32", seed=16, std=0.5).to(DEV)
    kc = torch.empty((B, N, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    csa.csa_compress(x_k, z, m, kc)
    csa.csa_compress(x_v, z, m, vc)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(q_idx, None, k_idx, None, t0, m, k, idx)
    scale = 1.0 / math.sqrt(d)
    o_csa = torch.empty((B, T, H, d), dtype=torch.float32, device=DEV)
    o_hca = torch.empty_like(o_csa)
    csa.csa_attend(q, kc, vc, m, idx, x_k, x_v, t0, W, scale, o_csa)
    csa.hca_attend(q, kc, vc, m, x_k, x_v, t0, W, scale, o_hca)
    torch.cuda.synchronize()
    # Both against one softmax over the visible compressed entries and the window.
    vmax = max(float(np.abs(f64(vc)).max()), float(np.abs(f64(x_v)).max()))
    for b in range(B):
        K, V = f64(kc[b]), f64(vc[b])
        xr_k, xr_v = f64(x_k[b]), f64(x_v[b])
        keys = np.concatenate([K, xr_k])
        vals = np.concatenate([V, xr_v])
        mask = np.zeros((T, N + n), dtype=bool)
        for i in range(T):
            t = t0 + i
            mask[i, : min(N, (t + 1) // m)] = True
            mask[i, N + max(0, t - W + 1): N + t + 1] = True
        ref = sdpa(f64(q[b]), keys, vals, scale, mask)
        close_rows(f64(o_csa[b]), ref, TOL["bf16"], f"CSA b={b}")
        close_rows(f64(o_hca[b]), ref, TOL["bf16"], f"HCA b={b}")
    # And against each other: summation order, plus the multi-token HCA kernel's binary16
    # weights (at most 2^-11 relative each, so 2^-11 of the largest |V| per output).
    err = np.abs(f64(o_csa) - f64(o_hca)).max(axis=-1)
    ref = np.abs(f64(o_csa)).max(axis=-1)
    assert np.all(err <= 1e-4 * ref + 2.0 ** -11 * vmax)


def test_equal_logits_give_block_means():
    B, n, d, m = 2, 1000, 128, 4
    say("closed form: equal logits -> block means")
    x = gen("cf3_x", (B, n, d), "bf16", seed=21).to(DEV)
    out = torch.empty((B, n // m, d), dtype=torch.bfloat16, device=DEV)
    csa.csa_compress(x, torch.full((m,), 0.7, device=DEV), m, out)
    torch.cuda.synchronize()
    mean = f64(x).reshape(B, n // m, m, d).mean(axis=2)
    diff = ulp_diff_bf16(bf16_bits(out), bf16_bits(torch.from_numpy(formats.round_to_bf16(mean)).to(torch.bfloat16)))
    say(f"  largest difference {int(diff.max())} bf16 steps, {float((diff == 0).mean()):.5f} identical")
    assert diff.max() <= 1


def test_no_selected_entry_is_sliding_window_attention():
    B, T, H, d, W, m = 1, 70, 32, 128, 100, 4
    t0 = 500
    n = t0 + T
    say("closed form: every index -1 -> sliding-window attention")
    x_k = gen("cf4_k", (B, n, d), "bf16", seed=31).to(DEV)
    x_v = gen("cf4_v", (B, n, d), "bf16", seed=32).to(DEV)
    q = gen("cf4_q", (B, T, H, d), "bf16", seed=33).to(DEV)
    kc = gen("cf4_kc", (B, n // m, d), "bf16", seed=34).to(DEV)
    idx = torch.full((B, T, 16), -1, dtype=torch.int32, device=DEV)
    out = torch.empty((B, T, H, d), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    csa.csa_attend(q, kc, kc, m, idx, x_k, x_v, t0, W, scale, out)
    torch.cuda.synchronize()
    mask = np.zeros((T, n), dtype=bool)
    for i in range(T):
        t = t0 + i
        mask[i, max(0, t - W + 1): t + 1] = True
    ref = sdpa(f64(q[0]), f64(x_k[0]), f64(x_v[0]), scale, mask)
    close_rows(f64(out[0]), ref, TOL["bf16"], "window attention")
