"""GPU parity of every kernel stage against the fp64 CPU oracle (through the C ABI).

Each stage receives the same inputs on both sides; inputs of a later stage are
the oracle's stored outputs of the earlier one (never a GPU result), so every
comparison is stage-local.  Shapes span several tiles and slices with ragged
tails, and the edge cases of the method: rows that see nothing, k above the
visible count, invalid / invisible / repeated indices, window off, HCA blocks
longer than the context seen so far.
"""
import math

import numpy as np
import pytest
import torch

import compressed_attention_csa_amd as csa
import inputgen
from oracle import formats, method
from parity_util import (check_attention, check_bf16_selection_row, check_e4m3, check_topk_rows,
                         check_topk_rows_fp8, fp8_score_error_bound, f64, bf16_bits,
                         to_dev_bf16, to_dev_f32, ulp_diff_bf16)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gen(name, shape, dtype, seed=0, std=1.0):
    return inputgen.normal(name, shape, seed, dtype, std=std)


def say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------------------- compressor

COMPRESS_CASES = [
    # x_dt, out_dt, m, d, n_raw, raw_base, entry_begin, entry_end, N_alloc
    ("bf16", "bf16", 4, 128, 1003, 0, 0, 250, 250),
    ("bf16", "f32", 4, 64, 517, 0, 0, 129, 129),
    ("bf16", "e4m3", 4, 64, 1000, 0, 0, 250, 250),
    ("bf16", "e4m3", 4, 32, 999, 0, 0, 249, 260),
    ("f32", "f32", 4, 32, 4096, 0, 0, 1024, 1024),
    ("f32", "bf16", 128, 64, 1000, 0, 0, 7, 7),
    ("bf16", "bf16", 128, 128, 4096, 0, 0, 32, 32),
    ("bf16", "bf16", 4, 128, 300, 100, 25, 100, 120),  # sub-range after raw_base
    ("bf16", "bf16", 1, 64, 77, 0, 0, 77, 77),         # m = 1 copies
    ("bf16", "bf16", 5, 16, 103, 0, 3, 20, 20),        # odd block, narrow rows
    # long blocks split over slot groups: 4 groups of 32 slots (wide rows cap the
    # groups), 8 groups of 13 slots with a short last one, 3 groups on 3-thread rows
    ("bf16", "e4m3", 128, 512, 1024, 0, 0, 8, 8),
    ("f32", "f32", 100, 256, 1000, 0, 0, 10, 10),
    ("bf16", "bf16", 17, 24, 200, 0, 0, 11, 11),
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=[f"{c[0]}-{c[1]}-m{c[2]}-d{c[3]}-n{c[4]}" for c in COMPRESS_CASES])
def test_compress(case):
    x_dt, out_dt, m, d, n_raw, raw_base, eb, ee, N = case
    say("compress", case)
    B = 2
    x = gen("cmp_x", (B, n_raw, d), x_dt, seed=n_raw + d)
    z = gen("cmp_z", (m,), "f32", seed=m, std=0.5)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.uint8}[out_dt]
    sentinel = 0x55 if out_dt == "e4m3" else 7.0
    out = torch.full((B, N, d), sentinel, dtype=tdt, device=DEV)
    scale = torch.full((B, N), 7.0, device=DEV) if out_dt == "e4m3" else None
    csa.csa_compress(x.to(DEV), z.to(DEV), m, out, scale, raw_base=raw_base, entry_begin=eb,
                     entry_end=ee)
    torch.cuda.synchronize()
    z64 = f64(z)
    for b in range(B):
        sums = method.compress_exact(f64(x[b]), z64, m, eb, ee, raw_base)
        if out_dt == "bf16":
            got = bf16_bits(out[b, eb:ee])
            exp = formats.f64_to_bf16_bits(sums)
            diff = ulp_diff_bf16(got, exp)
            assert diff.max() <= 1
            assert (diff == 0).mean() >= 0.9999, f"exact-match rate {(diff == 0).mean()}"
        elif out_dt == "f32":
            got = f64(out[b, eb:ee])
            exp = formats.round_to_f32(sums)
            np.testing.assert_allclose(got, exp, rtol=1e-6, atol=0)
        else:
            n_bad = check_e4m3(out[b, eb:ee].cpu().numpy(), scale[b, eb:ee].cpu().numpy(),
                               sums.astype(np.float32))
            assert n_bad <= max(2, sums.size // 10000)
        # entries outside the range are untouched
        if out_dt == "e4m3":
            assert (out[b, :eb] == 0x55).all() and (out[b, ee:] == 0x55).all()
            assert (scale[b, :eb] == 7.0).all() and (scale[b, ee:] == 7.0).all()
        else:
            assert (out[b, :eb] == 7.0).all() and (out[b, ee:] == 7.0).all()


OVERLAP_CASES = [
    # x_dt, out_dt, m, overlap, d, n_raw, raw_base, entry_begin, entry_end, N
    ("bf16", "bf16", 4, 2, 128, 400, 0, 0, 100, 100),
    ("bf16", "e4m3", 4, 4, 64, 300, 40, 11, 70, 80),
    ("f32", "f32", 5, 3, 32, 203, 0, 0, 40, 41),
    ("bf16", "bf16", 64, 64, 128, 1024, 0, 0, 16, 16),
    ("f32", "f32", 12, 5, 64, 300, 0, 0, 24, 24),  # 17 slots in 3 groups; the first entry renormalised
]


@pytest.mark.parametrize("case", OVERLAP_CASES, ids=[f"{c[0]}-{c[1]}-m{c[2]}-o{c[3]}" for c in OVERLAP_CASES])
def test_compress_with_overlapping_blocks(case):
    """The overlapping variant (m + o slots per entry, first entries renormalised)
    against the oracle's compress_overlap, with the csa_compress criteria."""
    x_dt, out_dt, m, o, d, n_raw, raw_base, eb, ee, N = case
    say("compress overlap", case)
    B = 2
    x = gen("ov_x", (B, n_raw, d), x_dt, seed=n_raw + d + o)
    z = gen("ov_z", (m + o,), "f32", seed=m + o, std=0.5)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.uint8}[out_dt]
    sentinel = 0x55 if out_dt == "e4m3" else 7.0
    out = torch.full((B, N, d), sentinel, dtype=tdt, device=DEV)
    scale = torch.full((B, N), 7.0, device=DEV) if out_dt == "e4m3" else None
    csa.csa_compress(x.to(DEV), z.to(DEV), m, out, scale, raw_base=raw_base, entry_begin=eb, entry_end=ee,
                     overlap=o)
    torch.cuda.synchronize()
    for b in range(B):
        sums = method.compress_overlap(f64(x[b]), f64(z), m, o, eb, ee, raw_base)
        if out_dt == "bf16":
            diff = ulp_diff_bf16(bf16_bits(out[b, eb:ee]), formats.f64_to_bf16_bits(sums))
            assert diff.max() <= 1
            assert (diff == 0).mean() >= 0.999
        elif out_dt == "f32":
            np.testing.assert_allclose(f64(out[b, eb:ee]), formats.round_to_f32(sums), rtol=1e-6, atol=0)
        else:
            n_bad = check_e4m3(out[b, eb:ee].cpu().numpy(), scale[b, eb:ee].cpu().numpy(), sums.astype(np.float32))
            assert n_bad <= max(2, sums.size // 10000)
        assert (out[b, :eb] == sentinel).all() and (out[b, ee:] == sentinel).all()


# ----------------------------------------------------------------------------- state cache (append)

APPEND_CASES = [
    # x_dt, out_dt, B, d, m, R, positions, pattern of rows per call, overlap
    ("bf16", "bf16", 2, 128, 4, 132, 701, [1], 0),
    ("bf16", "e4m3", 3, 64, 4, 132, 530, [1, 1, 3, 1, 2, 7, 1], 0),
    ("bf16", "bf16", 2, 128, 128, 256, 1100, [1] * 9 + [100], 0),
    ("f32", "f32", 1, 32, 5, 12, 301, [1, 2, 8, 1], 0),
    ("bf16", "bf16", 2, 64, 4, 134, 403, [1, 1, 5, 1, 3], 2),
    ("f32", "f32", 1, 32, 5, 17, 120, [1, 2, 8, 1], 3),
]


@pytest.mark.parametrize("case", APPEND_CASES,
                         ids=[f"{c[0]}-{c[1]}-m{c[4]}-R{c[5]}-o{c[8]}" for c in APPEND_CASES])
def test_append_builds_the_caches_of_the_full_history(case):
    """Rows appended token by token (and in small chunks) leave the ring holding
    the newest R positions bit-exactly, and the compressed cache equal to the
    oracle's compression of the whole history (same criteria as csa_compress)."""
    x_dt, out_dt, B, d, m, R, n, pattern, o = case
    say("append", case)
    hist = gen("app_x", (B, n, d), x_dt, seed=n + d)
    z = gen("app_z", (m + o,), "f32", seed=m, std=0.5).to(DEV)
    N = n // m + 3  # a few entries past the history stay untouched
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.uint8}[out_dt]
    sentinel = 0x55 if out_dt == "e4m3" else 7.0
    out = torch.full((B, N, d), sentinel, dtype=tdt, device=DEV)
    scale = torch.full((B, N), 7.0, device=DEV) if out_dt == "e4m3" else None
    ring = torch.zeros((B, 2 * R, d), dtype=hist.dtype, device=DEV)
    hd = hist.to(DEV)
    t, k = 0, 0
    while t < n:
        T_new = min(pattern[k % len(pattern)], n - t)
        k += 1
        csa.csa_append(hd[:, t:t + T_new].contiguous(), ring, t, z, m, out, scale, overlap=o)
        t += T_new
    torch.cuda.synchronize()
    z64 = f64(z)
    n_ent = n // m
    for b in range(B):
        # the ring rows the oracle's state cache holds (the newest R positions), bit-exact
        exp_ring = method.state_ring(f64(hist[b]), n - 1, R)
        held = ~np.isnan(exp_ring).any(axis=1)
        assert held.sum() == 2 * min(R, n)
        got_ring = f64(ring[b])
        np.testing.assert_array_equal(got_ring[held], exp_ring[held])
        sums = method.compress_overlap(f64(hist[b]), z64, m, o, 0, n_ent) if o else \
            method.compress_exact(f64(hist[b]), z64, m, 0, n_ent)
        if out_dt == "bf16":
            diff = ulp_diff_bf16(bf16_bits(out[b, :n_ent]), formats.f64_to_bf16_bits(sums))
            assert diff.max() <= 1
            assert (diff == 0).mean() >= 0.9999
        elif out_dt == "f32":
            np.testing.assert_allclose(f64(out[b, :n_ent]), formats.round_to_f32(sums), rtol=1e-6, atol=0)
        else:
            n_bad = check_e4m3(out[b, :n_ent].cpu().numpy(), scale[b, :n_ent].cpu().numpy(),
                               sums.astype(np.float32))
            assert n_bad <= max(2, sums.size // 10000)
            assert (scale[b, n_ent:] == 7.0).all()
        rest = out[b, n_ent:]
        assert (rest == sentinel).all(), "entries of incomplete blocks must stay untouched"


def test_decode_reads_its_window_from_the_ring():
    """A CSA and an HCA decode step whose window comes from the state ring equal
    the oracle over the full history."""
    B, d, H, W, n = 2, 128, 64, 128, 4099
    say("append+decode", B, n)
    hist_k = gen("ad_k", (B, n, d), "bf16", seed=1)
    hist_v = gen("ad_v", (B, n, d), "bf16", seed=2)
    q = gen("ad_q", (B, 1, H, d), "bf16", seed=3)
    scale = 1.0 / math.sqrt(d)
    t0 = n - 1
    for m, k in ((4, 256), (128, 0)):
        R = W + m
        z = gen("ad_z", (m,), "f32", seed=m, std=0.5).to(DEV)
        N = n // m
        kc = torch.empty((B, N, d), dtype=torch.bfloat16, device=DEV)
        vc = torch.empty_like(kc)
        rk = torch.zeros((B, 2 * R, d), dtype=torch.bfloat16, device=DEV)
        rv = torch.zeros_like(rk)
        hk, hv = hist_k.to(DEV), hist_v.to(DEV)
        for t in range(n):  # one token per decode step
            csa.csa_append(hk[:, t:t + 1].contiguous(), rk, t, z, m, kc)
            csa.csa_append(hv[:, t:t + 1].contiguous(), rv, t, z, m, vc)
        s = t0 - W + 1
        raw, base = csa.ring_window(rk, s)
        out = torch.empty((B, 1, H, d), dtype=torch.float32, device=DEV)
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
        z64 = f64(z)
        ek = [method.store(method.compress_exact(f64(hist_k[b]), z64, m), "bf16")["values"] for b in range(B)]
        ev = [method.store(method.compress_exact(f64(hist_v[b]), z64, m), "bf16")["values"] for b in range(B)]
        if m == 4:
            idx = np.stack([np.random.default_rng(b).choice(N, k, replace=False) for b in range(B)])
            idx = idx.astype(np.int32).reshape(B, 1, k)
            csa.csa_attend(q.to(DEV), kc, vc, m, torch.from_numpy(idx).to(DEV), raw, rv, t0, W, scale, out,
                           lse, raw_base=base)
        else:
            csa.hca_attend(q.to(DEV), kc, vc, m, raw, rv, t0, W, scale, out, lse, raw_base=base)
        torch.cuda.synchronize()
        for b in range(B):
            if m == 4:
                o_ref, l_ref = method.csa_attend(f64(q[b]), ek[b], ev[b], idx[b], f64(hist_k[b]), f64(hist_v[b]),
                                                 0, t0, W, m, scale)
            else:
                o_ref, l_ref = method.hca_attend(f64(q[b]), ek[b], ev[b], m, f64(hist_k[b]), f64(hist_v[b]),
                                                 0, t0, W, scale)
            check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, "bf16", what=f"ring m={m} b={b}")


# ----------------------------------------------------------------------------- indexer + top-k


def make_keys(kind, B, N, d_I, seed):
    """Stored indexer keys: (device tensor, device scale or None, float64 values)."""
    if kind == "e4m3":
        r = gen("idx_k", (B, N, d_I), "f32", seed=seed).numpy()
        codes, scale, stored = formats.e4m3_quantize_rows(r)
        return (torch.from_numpy(codes).to(DEV), torch.from_numpy(scale).to(DEV), stored)
    k = gen("idx_k", (B, N, d_I), kind, seed=seed)
    return k.to(DEV), None, f64(k)


INDEX_CASES = [
    # kind, B, T, H_I, d_I, N, t0, m, k, with_w
    ("bf16", 3, 1, 8, 64, 20000, 4 * 20000 - 1, 4, 512, True),     # decode, many slices
    ("e4m3", 2, 1, 8, 64, 33000, 4 * 33000 - 1, 4, 1024, True),    # decode, fp8 keys
    ("bf16", 2, 1, 8, 64, 20000, 4 * 15000 + 1, 4, 300, True),     # only 15000 visible
    ("e4m3", 2, 3, 8, 32, 9000, 4 * 9000 - 3, 4, 100, False),      # T=3 rows, w = 1
    ("bf16", 2, 37, 8, 64, 300, 1100, 4, 64, True),                # prefill-like, one slice
    ("bf16", 1, 9, 4, 32, 100, 0, 4, 16, True),                    # rows with 0..2 visible
    ("bf16", 1, 2, 8, 64, 1500, 4 * 1500 - 1, 4, 2048, True),      # k above visible count
    ("bf16", 2, 1, 16, 64, 12000, 4 * 12000 - 1, 4, 1, True),      # k = 1, 16 heads
    ("bf16", 2, 100, 8, 64, 3000, 11900, 4, 256, True),            # prefill path (T >= 64)
    ("e4m3", 1, 70, 8, 64, 40000, 4 * 40000 - 70, 4, 64, True),    # prefill, many compactions
    ("bf16", 1, 130, 4, 32, 9000, 30000, 4, 512, False),           # prefill, d_I 32, ragged T
    ("e4m3", 2, 64, 8, 32, 500, 0, 4, 100, True),                  # prefill, rows see 0..16
    ("bf16", 1, 96, 8, 64, 20000, 4 * 20000 - 96, 4, 2048, True),  # prefill, k = 2048
    ("f32", 1, 40, 4, 32, 1024, 4000, 4, 64, True),                # fp32 path
    ("f32", 2, 1, 4, 64, 6000, 4 * 6000 - 1, 4, 200, True),        # fp32, many slices
    # 256 rows of 4097 entries: slices of 4096, so each row's second slice holds
    # one entry and the first must list almost all of the 1024 winners
    ("bf16", 256, 1, 8, 64, 4097, 4 * 4097 - 1, 4, 1024, True),
]


@pytest.mark.parametrize("case", INDEX_CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}-N{c[5]}-k{c[8]}" for c in INDEX_CASES])
def test_index_topk(case):
    kind, B, T, H_I, d_I, N, t0, m, k, with_w = case
    say("index_topk", case)
    qdt = "f32" if kind == "f32" else "bf16"
    q = gen("idx_q", (B, T, H_I, d_I), qdt, seed=N + T)
    w = gen("idx_w", (B, T, H_I), "f32", seed=N + 1) if with_w else None
    kd, ks, k64 = make_keys(kind, B, N, d_I, seed=N)
    out_idx = torch.full((B, T, k), 12345, dtype=torch.int32, device=DEV)
    out_score = torch.full((B, T, k), 5.0, dtype=torch.float32, device=DEV)
    qd, wd = q.to(DEV), (None if w is None else w.to(DEV))
    csa.csa_index_topk(qd, wd, kd, ks, t0, m, k, out_idx, out_score)
    again = torch.full_like(out_idx, 777)
    csa.csa_index_topk(qd, wd, kd, ks, t0, m, k, again)
    torch.cuda.synchronize()
    assert torch.equal(out_idx, again), "selection order is not deterministic"
    idx = out_idx.cpu().numpy()
    sc = out_score.cpu().numpy()
    swaps = 0
    for b in range(B):
        scores, vis = method.index_scores(f64(q[b]), None if w is None else f64(w[b]), k64[b], t0, m)
        swaps += check_topk_rows(idx[b], sc[b], scores, vis, k)
    say("  in-band swaps:", swaps)


BF16_SEL_CASES = [INDEX_CASES[i] for i in (0, 1, 3, 8, 9, 13)]


FP8Q_CASES = [c for c in INDEX_CASES if c[0] == "e4m3"] + [
    # kind, B, T, H_I, d_I, N, t0, m, k, with_w
    ("e4m3", 2, 1, 16, 64, 12000, 4 * 12000 - 1, 4, 1, True),      # decode, 16 heads, k = 1
    ("e4m3", 2, 100, 8, 64, 3000, 11900, 4, 256, True),            # prefill path
    ("e4m3", 1, 130, 4, 32, 9000, 30000, 4, 512, False),           # prefill, 4 heads, d_I 32, ragged T
    ("e4m3", 1, 96, 8, 64, 20000, 4 * 20000 - 96, 4, 2048, True),  # prefill, k = 2048
]


@pytest.mark.parametrize("case", FP8Q_CASES, ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}d{c[4]}-N{c[5]}-k{c[8]}"
                                                  for c in FP8Q_CASES])
def test_index_topk_fp8_query(case):
    """The fp8 x fp8 indexer (csa_index_topk_fp8): the query quantised to e4m3
    per (token, head) row in the kernel; selection and scores against the
    oracle's index_scores_fp8q, through the decode and prefill paths."""
    kind, B, T, H_I, d_I, N, t0, m, k, with_w = case
    say("index_topk fp8 query", case)
    q = gen("idx_q", (B, T, H_I, d_I), "bf16", seed=N + T)
    w = gen("idx_w", (B, T, H_I), "f32", seed=N + 1) if with_w else None
    kd, ks, k64 = make_keys(kind, B, N, d_I, seed=N)
    out_idx = torch.full((B, T, k), 12345, dtype=torch.int32, device=DEV)
    out_score = torch.full((B, T, k), 5.0, dtype=torch.float32, device=DEV)
    qd, wd = q.to(DEV), (None if w is None else w.to(DEV))
    csa.csa_index_topk_fp8(qd, wd, kd, ks, t0, m, k, out_idx, out_score)
    again = torch.full_like(out_idx, 777)
    csa.csa_index_topk_fp8(qd, wd, kd, ks, t0, m, k, again)
    torch.cuda.synchronize()
    assert torch.equal(out_idx, again), "selection order is not deterministic"
    idx, sc = out_idx.cpu().numpy(), out_score.cpu().numpy()
    differ = 0
    for b in range(B):
        wb = None if w is None else f64(w[b])
        scores, vis = method.index_scores_fp8q(f64(q[b]), wb, k64[b], t0, m)
        E = fp8_score_error_bound(method.quantize_query_e4m3(f64(q[b])), wb, k64[b])
        check_topk_rows_fp8(idx[b], sc[b], scores, vis, k, E)
        exact, _ = method.index_scores(f64(q[b]), wb, k64[b], t0, m)
        fin = np.isfinite(exact) & np.isfinite(scores)
        differ += int(np.sum(np.abs(exact - scores)[fin] > E[fin]))
        rel = E[fin] / np.maximum(np.abs(scores[fin]), 1e-30)
        say(f"  b={b}: median error bound / |score| {np.median(rel):.2e}")
    assert differ > 0, "no score moved beyond the bound by quantising the query: the case does not test it"



@pytest.mark.parametrize("case", BF16_SEL_CASES,
                         ids=[f"{c[0]}-B{c[1]}T{c[2]}-N{c[5]}-k{c[8]}" for c in BF16_SEL_CASES])
def test_index_topk_bf16_selector(case):
    """The approximate selector (csa_index_topk_bf16): the exact top-k of the
    bf16-rounded scores, ties to the lower index, through the decode, prefill
    and fp32 paths; its recall against the exact top-k is reported."""
    kind, B, T, H_I, d_I, N, t0, m, k, with_w = case
    say("index_topk bf16 selector", case)
    qdt = "f32" if kind == "f32" else "bf16"
    q = gen("idx_q", (B, T, H_I, d_I), qdt, seed=N + T)
    w = gen("idx_w", (B, T, H_I), "f32", seed=N + 1) if with_w else None
    kd, ks, k64 = make_keys(kind, B, N, d_I, seed=N)
    out_idx = torch.full((B, T, k), 12345, dtype=torch.int32, device=DEV)
    out_score = torch.full((B, T, k), 5.0, dtype=torch.float32, device=DEV)
    csa.csa_index_topk(q.to(DEV), None if w is None else w.to(DEV), kd, ks, t0, m, k, out_idx, out_score,
                       bf16_scores=True)
    torch.cuda.synchronize()
    idx, sc = out_idx.cpu().numpy(), out_score.cpu().numpy()
    total = hits = 0
    for b in range(B):
        scores, vis = method.index_scores(f64(q[b]), None if w is None else f64(w[b]), k64[b], t0, m)
        for i in range(T):
            kk, h = check_bf16_selection_row(idx[b, i], sc[b, i], scores[i], vis[i], k)
            total, hits = total + kk, hits + h
    say(f"  recall against the exact top-k: {hits / max(total, 1):.4f}")
    assert hits >= 0.95 * total


def test_index_topk_bf16_selector_edges():
    """The approximate selector where rounding decides everything: identical
    keys (every score ties: the lowest indices win), k above the visible count
    (everything visible is listed, then -1), and scores that differ only below
    bf16 resolution (ties again, so the lowest indices win where the exact
    selection would take the highest scores)."""
    B, N, d_I = 1, 20000, 64
    q = gen("bsel_q", (B, 1, 8, d_I), "bf16", seed=31)
    same = gen("bsel_k", (1, 1, d_I), "bf16", seed=32).expand(B, N, d_I).contiguous()
    out = torch.empty((B, 1, 700), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(q.to(DEV), None, same.to(DEV), None, 4 * N - 1, 4, 700, out, bf16_scores=True)
    few = torch.empty((B, 1, 2048), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(q.to(DEV), None, same.to(DEV), None, 4 * 1500 - 1, 4, 2048, few, bf16_scores=True)
    # scores 8 * (1 + (j % 64) * 2^-16): distinct in binary32, all 8.0 in bf16
    k64 = np.zeros((3000, d_I))
    k64[:, 0] = 1.0
    k64[:, 1] = (np.arange(3000) % 64) * 2.0 ** -16
    qq = np.zeros((1, 1, 8, d_I))
    qq[..., :2] = 1.0
    near = torch.empty((1, 1, 64), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(to_dev_bf16(qq), None, to_dev_bf16(k64[None]), None, 4 * 3000 - 1, 4, 64, near,
                       bf16_scores=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.sort(out[0, 0].cpu().numpy()), np.arange(700))
    got = few[0, 0].cpu().numpy()
    np.testing.assert_array_equal(np.sort(got[:1500]), np.arange(1500))
    assert (got[1500:] == -1).all()
    np.testing.assert_array_equal(np.sort(near[0, 0].cpu().numpy()), np.arange(64))
    scores, vis = method.index_scores(qq[0], None, k64, 4 * 3000 - 1, 4)
    check_bf16_selection_row(near[0, 0].cpu().numpy(), None, scores[0], vis[0], 64)


def test_index_topk_exact_ties_go_to_lower_index():
    B, N, d_I, k = 1, 2000, 64, 100
    base = gen("tie_k", (1, 50, d_I), "bf16", seed=3)
    keys = base.repeat(1, 40, 1)  # row j equals row j % 50
    q = gen("tie_q", (B, 1, 8, d_I), "bf16", seed=4)
    out = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(q.to(DEV), None, keys.to(DEV).contiguous(), None, 4 * N - 1, 4, k, out)
    torch.cuda.synchronize()
    scores, vis = method.index_scores(f64(q[0]), None, f64(keys[0]), 4 * N - 1, 4)
    exp = np.sort(method.select_topk(scores, vis, k)[0])
    np.testing.assert_array_equal(np.sort(out[0, 0].cpu().numpy()), exp)


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
def test_index_topk_winners_concentrated_in_few_slices(kind):
    """Entries 5000..5599 score far above the rest, so a few slices hold every
    winner: their local candidate lists cannot cover them and the exact
    fallback (rescoring those slices) must produce the true top-k."""
    B, N, d_I, k = 2, 24000, 64, 512
    r = gen("conc_k", (B, N, d_I), "f32", seed=11).numpy()
    r[:, 5000:5600] *= 4.0
    q = gen("conc_q", (B, 1, 8, d_I), "bf16", seed=12)
    w = gen("conc_w", (B, 1, 8), "f32", seed=13).abs()
    if kind == "e4m3":
        codes, scale, k64 = formats.e4m3_quantize_rows(r)
        kd, ks = torch.from_numpy(codes).to(DEV), torch.from_numpy(scale).to(DEV)
    else:
        k64 = formats.round_to_bf16(r.astype(np.float64))
        kd, ks = to_dev_bf16(k64), None
    out = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, 1, k), device=DEV)
    csa.csa_index_topk(q.to(DEV), w.to(DEV), kd, ks, 4 * N - 1, 4, k, out, sc)
    torch.cuda.synchronize()
    for b in range(B):
        scores, vis = method.index_scores(f64(q[b]), f64(w[b]), k64[b], 4 * N - 1, 4)
        check_topk_rows(out[b].cpu().numpy(), sc[b].cpu().numpy(), scores, vis, k)
        assert (out[b, 0].cpu().numpy() >= 5000).mean() > 0.9


def test_index_topk_all_scores_equal():
    """Identical keys: every score ties, the winners are the lowest indices, all
    inside the first slice."""
    B, N, d_I, k = 1, 20000, 64, 700
    keys = gen("eq_k", (1, 1, d_I), "bf16", seed=5).expand(B, N, d_I).contiguous()
    q = gen("eq_q", (B, 1, 8, d_I), "bf16", seed=6)
    out = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(q.to(DEV), None, keys.to(DEV), None, 4 * N - 1, 4, k, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.sort(out[0, 0].cpu().numpy()), np.arange(k))


def test_index_topk_prefill_sampled_threshold_falls_back():
    """Prefill rows whose best entries all sit at multiples of 32 (the sample
    stride of a 40000-entry sweep): the threshold taken from the sampled
    entries then prunes away most of the true top-k, and the kernel must notice
    and sweep those queries again without a threshold."""
    B, T, H_I, d_I, N, m, k = 1, 70, 8, 64, 40000, 4, 64
    t0 = 4 * N - T
    q = gen("smp_q", (B, T, H_I, d_I), "f32", seed=3).abs().to(torch.bfloat16)
    keys = gen("smp_k", (B, N, d_I), "f32", seed=4)
    keys[:, ::32, :] = 3.0 + 0.3 * keys[:, ::32, :]
    keys = keys.to(torch.bfloat16)
    out_idx = torch.full((B, T, k), 12345, dtype=torch.int32, device=DEV)
    out_score = torch.empty((B, T, k), dtype=torch.float32, device=DEV)
    say("index_topk prefill, winners on the sample grid")
    csa.csa_index_topk(q.to(DEV), None, keys.to(DEV), None, t0, m, k, out_idx, out_score)
    torch.cuda.synchronize()
    scores, vis = method.index_scores(f64(q[0]), None, f64(keys[0]), t0, m)
    idx = out_idx[0].cpu().numpy()
    check_topk_rows(idx, out_score[0].cpu().numpy(), scores, vis, k)
    assert np.all(idx % 32 == 0), "winners are the entries on the sample grid"


@pytest.mark.parametrize("d_I", [64, 32])
def test_index_topk_every_e4m3_code_scores_exactly(d_I):
    """Entry j of the fp8 key cache holds code j in one dimension and +0 in the
    others (NaN codes replaced by +0); every head's query picks that dimension
    with +1 (sequence 0) or -1 (sequence 1), so the score is 8 * ReLU(+-value),
    exact in binary32.  With k = 256 every entry is selected and every score
    must equal the oracle's bit for bit: a code the kernel widens wrongly
    (subnormals, the sign, the largest exponents) shows up here."""
    N, H_I, m = 256, 8, 4
    code = np.arange(256, dtype=np.uint8)
    code[(code & 0x7F) == 0x7F] = 0
    codes = np.zeros((2, N, d_I), dtype=np.uint8)
    codes[:, :, 5] = code
    scale = np.ones((2, N), dtype=np.float32)
    q = torch.zeros((2, 1, H_I, d_I), dtype=torch.bfloat16)
    q[0, 0, :, 5] = 1.0
    q[1, 0, :, 5] = -1.0
    out_idx = torch.empty((2, 1, N), dtype=torch.int32, device=DEV)
    out_score = torch.empty((2, 1, N), dtype=torch.float32, device=DEV)
    say("index_topk every e4m3 code, d_I", d_I)
    csa.csa_index_topk(q.to(DEV), None, torch.from_numpy(codes).to(DEV), torch.from_numpy(scale).to(DEV),
                       4 * N - 1, m, N, out_idx, out_score)
    torch.cuda.synchronize()
    stored = formats.e4m3_decode(codes) * scale[:, :, None]
    for b in range(2):
        ref = method.index_scores(f64(q[b]), None, stored[b], 4 * N - 1, m)[0][0]
        idx = out_idx[b, 0].cpu().numpy()
        np.testing.assert_array_equal(np.sort(idx), np.arange(N))
        np.testing.assert_array_equal(out_score[b, 0].cpu().numpy().astype(np.float64), ref[idx])


# ----------------------------------------------------------------------------- attention


def make_idx(B, T, k, t0, m, N, seed, bad_frac=0.1):
    """Random selections of distinct visible entries, with some slots set to -1, to
    entries not yet visible, to entries past the cache, and one repeated entry."""
    rng = np.random.default_rng(seed)
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(T):
            c = min(N, (t0 + i + 1) // m)
            n = min(k, c)
            if n:
                idx[b, i, :n] = rng.choice(c, n, replace=False)
            nbad = int(bad_frac * k)
            pos = rng.choice(k, nbad, replace=False)
            p1, p2, p3 = pos[: nbad // 3], pos[nbad // 3: 2 * nbad // 3], pos[2 * nbad // 3:]
            idx[b, i, p1] = -1
            idx[b, i, p2] = c + rng.integers(0, 5, len(p2))  # not yet visible
            idx[b, i, p3] = N + 7                             # past the cache
            if n >= 2 and nbad and 0 not in pos and 1 not in pos:
                idx[b, i, 1] = idx[b, i, 0]                   # counted twice
    return idx


ATTEND_CASES = [
    # name, dt, B, T, H, d, N, m, k, W, t0, out_dt
    ("csa-decode", "bf16", 2, 1, 128, 128, 3000, 4, 1024, 128, 4 * 3000 - 1, "f32"),
    ("csa-decode-h64", "bf16", 3, 1, 64, 128, 3000, 4, 512, 128, 4 * 3000 - 1, "bf16"),
    ("csa-prefill", "bf16", 1, 37, 64, 128, 300, 4, 64, 128, 1100, "f32"),
    ("csa-nowin-d64", "bf16", 2, 20, 16, 64, 100, 4, 40, 0, 60, "f32"),
    ("csa-empty-rows", "bf16", 1, 12, 32, 128, 50, 4, 8, 0, 0, "f32"),
    ("csa-f32", "f32", 1, 50, 8, 64, 1024, 4, 64, 128, 3000, "f32"),
    ("csa-f32-d32", "f32", 2, 9, 3, 32, 200, 4, 100, 7, 700, "f32"),
    ("csa-f32-decode", "f32", 2, 1, 8, 128, 3000, 4, 1024, 128, 4 * 3000 - 1, "f32"),
    ("csa-f32-h32", "f32", 1, 20, 32, 64, 300, 4, 64, 128, 1200, "f32"),     # 8 heads per wave
    ("hca-f32-h13-decode", "f32", 2, 1, 13, 128, 400, 128, 0, 128, 128 * 400 - 1, "f32"),  # split, merged
    ("csa-f32-h2-d32", "f32", 1, 70, 2, 32, 90, 4, 16, 5, 300, "f32"),
    ("csa-decode-h80", "bf16", 3, 1, 80, 128, 3000, 4, 1024, 128, 4 * 3000 - 1, "f32"),
    ("hca-decode", "bf16", 2, 1, 128, 128, 2000, 128, 0, 128, 128 * 2000 - 1, "f32"),
    ("hca-decode-b16", "bf16", 16, 1, 128, 128, 700, 128, 0, 128, 128 * 700 - 1, "f32"),
    ("hca-short", "bf16", 3, 1, 64, 128, 200, 128, 0, 128, 128 * 200 - 1, "bf16"),
    ("hca-prefill", "bf16", 1, 40, 64, 128, 10, 128, 0, 128, 300, "f32"),
    ("hca-f32", "f32", 1, 33, 8, 64, 32, 128, 0, 128, 4000, "f32"),
    # many consecutive query tokens per sequence (multi-token HCA kernel): heavy
    # blocks completing inside the chunk, ragged token counts, capped entries
    ("hca-prefill-multi", "bf16", 2, 301, 64, 128, 40, 128, 0, 128, 4000, "f32"),
    ("hca-prefill-multi-h128-d64", "bf16", 1, 263, 128, 64, 30, 128, 0, 100, 3700, "bf16"),
    ("hca-prefill-multi-h16", "bf16", 1, 259, 16, 128, 64, 128, 0, 128, 100, "f32"),
    ("hca-prefill-multi-h32-nowin", "bf16", 1, 300, 32, 128, 20, 128, 0, 0, 2000, "f32"),
    ("hca-prefill-multi-empty-rows", "bf16", 1, 300, 64, 128, 8, 128, 0, 0, 0, "f32"),
    ("hca-prefill-multi-w1", "bf16", 1, 290, 48, 128, 16, 128, 0, 1, 1000, "f32"),
    # the limits: top_k 2048 and a 1024-token window
    ("csa-max-k-window", "bf16", 1, 1, 64, 128, 4000, 4, 2048, 1024, 4 * 4000 - 1, "f32"),
    ("hca-prefill-multi-w1024", "bf16", 1, 260, 64, 128, 40, 128, 0, 1024, 4000, "f32"),
]


@pytest.mark.parametrize("case", ATTEND_CASES, ids=[c[0] for c in ATTEND_CASES])
def test_attend(case):
    name, dt, B, T, H, d, N, m, k, W, t0, out_dt = case
    say("attend", case)
    hca = name.startswith("hca")
    n_raw = t0 + T + 3
    q = gen("att_q", (B, T, H, d), dt, seed=H + T)
    kc = gen("att_kc", (B, N, d), dt, seed=N, std=0.6)
    vc = gen("att_vc", (B, N, d), dt, seed=N + 1, std=0.6)
    kr = gen("att_kr", (B, n_raw, d), dt, seed=7)
    vr = gen("att_vr", (B, n_raw, d), dt, seed=8)
    scale = 1.0 / math.sqrt(d)
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    out = torch.full((B, T, H, d), 9.0, dtype=odt, device=DEV)
    lse = torch.full((B, T, H), 9.0, device=DEV)
    out_nolse = None
    if hca:
        csa.hca_attend(q.to(DEV), kc.to(DEV), vc.to(DEV), m, kr.to(DEV), vr.to(DEV), t0, W, scale,
                       out, lse)
        # without an lse output the multi-token kernel sums its binary16 weights on
        # the matrix cores: the output alone is held to the same criterion
        out_nolse = torch.full_like(out, 9.0)
        csa.hca_attend(q.to(DEV), kc.to(DEV), vc.to(DEV), m, kr.to(DEV), vr.to(DEV), t0, W, scale,
                       out_nolse)
    else:
        idx = make_idx(B, T, k, t0, m, N, seed=N + k)
        csa.csa_attend(q.to(DEV), kc.to(DEV), vc.to(DEV), m, torch.from_numpy(idx).to(DEV),
                       kr.to(DEV), vr.to(DEV), t0, W, scale, out, lse)
    torch.cuda.synchronize()
    for b in range(B):
        if hca:
            o_ref, l_ref = method.hca_attend(f64(q[b]), f64(kc[b]), f64(vc[b]), m, f64(kr[b]),
                                             f64(vr[b]), 0, t0, W, scale)
        else:
            o_ref, l_ref = method.csa_attend(f64(q[b]), f64(kc[b]), f64(vc[b]), idx[b], f64(kr[b]),
                                             f64(vr[b]), 0, t0, W, m, scale)
        check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, dt, what=f"{name} b={b}",
                        out_bf16=(out_dt == "bf16"))
        if out_nolse is not None:
            check_attention(f64(out_nolse[b]), None, o_ref, l_ref, dt, what=f"{name} b={b}, no lse",
                            out_bf16=(out_dt == "bf16"))


@pytest.mark.parametrize("T", [64, 1], ids=["prefill-multi", "decode"])
def test_hca_many_tiny_weights(T):
    """HCA prefill (multi-token kernel) and decode where one entry dominates and
    thousands of others carry weights 2^-15 .. 2^-23 of it, all with the same V
    row: their sum moves the output by several percent, so weights lost in
    rounding (the binary16 weights of bf16 tiles fall below the binary16 normal
    range here) would show.  Scores follow from one nonzero coordinate:
    q = (8, 0, ...), k_j = (c_j, 0, ...)."""
    B, H, d, m, N, W = 1, 64, 128, 4, 4000, 128
    t0 = m * N - T - 1
    say("hca, many tiny weights", (B, T, H, d, m, N, W, t0))
    n_raw = t0 + T + 3
    scale = 1.0 / math.sqrt(d)
    gamma = 8.0
    rng = np.random.default_rng(5)
    # natural-log score gaps of -e*ln2 below the dominant entry, e in 15..23
    gaps = rng.integers(15, 24, size=N).astype(np.float64)
    c = formats.bf16_bits_to_f64(formats.f64_to_bf16_bits(-gaps * math.log(2) / (gamma * scale)))
    c[0] = 0.0
    q = np.zeros((B, T, H, d))
    q[..., 0] = gamma
    kc = np.zeros((B, N, d))
    kc[0, :, 0] = c
    vc = np.ones((B, N, d))
    vc[0, 0] = formats.bf16_bits_to_f64(formats.f64_to_bf16_bits(rng.standard_normal(d)))
    kr = np.zeros((B, n_raw, d))
    kr[0, :, 0] = c[1 + np.arange(n_raw) % (N - 1)]
    vr = np.ones((B, n_raw, d))
    out = torch.full((B, T, H, d), 9.0, device=DEV)
    lse = torch.full((B, T, H), 9.0, device=DEV)
    csa.hca_attend(to_dev_bf16(q), to_dev_bf16(kc), to_dev_bf16(vc), m, to_dev_bf16(kr), to_dev_bf16(vr),
                   t0, W, scale, out, lse)
    out2 = torch.full((B, T, H, d), 9.0, device=DEV)  # no lse: weight sums on the matrix cores
    csa.hca_attend(to_dev_bf16(q), to_dev_bf16(kc), to_dev_bf16(vc), m, to_dev_bf16(kr), to_dev_bf16(vr),
                   t0, W, scale, out2)
    torch.cuda.synchronize()
    o_ref, l_ref = method.hca_attend(q[0], kc[0], vc[0], m, kr[0], vr[0], 0, t0, W, scale)
    shift = np.abs(o_ref - vc[0, 0]).max()
    assert shift > 0.02, shift  # the tiny weights matter
    check_attention(f64(out[0]), f64(lse[0]), o_ref, l_ref, "bf16", what="tiny weights")
    check_attention(f64(out2[0]), None, o_ref, l_ref, "bf16", what="tiny weights, no lse")


@pytest.mark.parametrize("T", [301, 1], ids=["prefill-multi", "decode"])
def test_hca_v_outside_binary16_range(T):
    """HCA prefill (multi-token kernel) and decode with V values the binary16
    weight path of the multi-token kernel cannot take: in sequence 0 the raw V
    rows of positions 4100..4109 (and, in decode, the heavy entries 10..12) are
    scaled by 2^17 (|V| past 65280), so the prefill sweeps that meet them switch
    paths part-way and the others stay binary16; sequence 1 has every V value
    scaled by 2^-12 (largest |V| below 2^-10), so it never takes the binary16
    path.  (Decode uses bf16 hi + lo weights throughout; the cases check it on
    the same extremes.)"""
    B, H, d, m, N, W = 2, 64, 128, 128, 40, 128
    t0 = 4000 if T > 1 else 4105
    say("hca, V outside the binary16 range", (B, T, H, d, m, N, W, t0))
    n_raw = t0 + T + 3
    q = gen("rng_q", (B, T, H, d), "bf16", seed=11)
    kc = gen("rng_kc", (B, N, d), "bf16", seed=12, std=0.6)
    vc = f64(gen("rng_vc", (B, N, d), "bf16", seed=13, std=0.6))
    kr = gen("rng_kr", (B, n_raw, d), "bf16", seed=14)
    vr = f64(gen("rng_vr", (B, n_raw, d), "bf16", seed=15))
    vr[0, 4100:4110] *= 2.0 ** 17
    if T == 1:  # (in prefill this would end every sweep's binary16 run at its first tile)
        vc[0, 10:13] *= 2.0 ** 17
    vc[1] *= 2.0 ** -12
    vr[1] *= 2.0 ** -12
    scale = 1.0 / math.sqrt(d)
    out = torch.full((B, T, H, d), 9.0, device=DEV)
    lse = torch.full((B, T, H), 9.0, device=DEV)
    csa.hca_attend(q.to(DEV), kc.to(DEV), to_dev_bf16(vc), m, kr.to(DEV), to_dev_bf16(vr), t0, W, scale,
                   out, lse)
    out2 = torch.full((B, T, H, d), 9.0, device=DEV)  # no lse: weight sums on the matrix cores
    csa.hca_attend(q.to(DEV), kc.to(DEV), to_dev_bf16(vc), m, kr.to(DEV), to_dev_bf16(vr), t0, W, scale,
                   out2)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, l_ref = method.hca_attend(f64(q[b]), f64(kc[b]), vc[b], m, f64(kr[b]), vr[b], 0, t0, W, scale)
        check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, "bf16", what=f"v range b={b}")
        check_attention(f64(out2[b]), None, o_ref, l_ref, "bf16", what=f"v range b={b}, no lse")


FP8_KV_CASES = [
    # name, B, T, H, d, N, m, k, W, t0
    ("csa-decode", 2, 1, 128, 128, 3000, 4, 1024, 128, 4 * 3000 - 1),
    ("csa-prefill", 1, 37, 64, 128, 300, 4, 64, 128, 1100),
    ("csa-d64", 2, 20, 16, 64, 100, 4, 40, 0, 60),
    ("hca-decode", 2, 1, 128, 128, 2000, 128, 0, 128, 128 * 2000 - 1),
    ("hca-prefill-multi", 2, 301, 64, 128, 40, 128, 0, 128, 4000),
    ("hca-prefill-multi-d64", 1, 263, 32, 64, 30, 128, 0, 100, 3700),
]


@pytest.mark.parametrize("case", FP8_KV_CASES, ids=[c[0] for c in FP8_KV_CASES])
def test_attend_with_fp8_compressed_caches(case):
    """Compressed K and V stored as e4m3 codes with one fp32 scale per entry (the
    oracle's quantiser); the oracle attends over the stored values code * scale."""
    name, B, T, H, d, N, m, k, W, t0 = case
    say("attend fp8 kv", case)
    hca = name.startswith("hca")
    n_raw = t0 + T + 3
    q = gen("f8_q", (B, T, H, d), "bf16", seed=H + T)
    kq = formats.e4m3_quantize_rows(gen("f8_kc", (B, N, d), "f32", seed=N, std=0.6).numpy())
    vq = formats.e4m3_quantize_rows(gen("f8_vc", (B, N, d), "f32", seed=N + 1, std=0.6).numpy())
    kc, ks, kv64 = torch.from_numpy(kq[0]).to(DEV), torch.from_numpy(kq[1]).to(DEV), kq[2]
    vc, vs, vv64 = torch.from_numpy(vq[0]).to(DEV), torch.from_numpy(vq[1]).to(DEV), vq[2]
    kr = gen("f8_kr", (B, n_raw, d), "bf16", seed=7)
    vr = gen("f8_vr", (B, n_raw, d), "bf16", seed=8)
    scale = 1.0 / math.sqrt(d)
    out = torch.full((B, T, H, d), 9.0, device=DEV)
    lse = torch.full((B, T, H), 9.0, device=DEV)
    if hca:
        csa.hca_attend(q.to(DEV), kc, vc, m, kr.to(DEV), vr.to(DEV), t0, W, scale, out, lse,
                       k_scale=ks, v_scale=vs)
    else:
        idx = make_idx(B, T, k, t0, m, N, seed=N + k)
        csa.csa_attend(q.to(DEV), kc, vc, m, torch.from_numpy(idx).to(DEV), kr.to(DEV), vr.to(DEV), t0, W,
                       scale, out, lse, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    for b in range(B):
        if hca:
            o_ref, l_ref = method.hca_attend(f64(q[b]), kv64[b], vv64[b], m, f64(kr[b]), f64(vr[b]), 0, t0, W,
                                             scale)
        else:
            o_ref, l_ref = method.csa_attend(f64(q[b]), kv64[b], vv64[b], idx[b], f64(kr[b]), f64(vr[b]), 0,
                                             t0, W, m, scale)
        check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, "bf16", what=f"fp8 kv {name} b={b}")


def test_empty_calls_enqueue_nothing():
    """T = 0 queries, an empty entry range and T_new = 0 rows succeed and leave
    every output untouched.  (Zero-length views keep a valid base pointer.)"""
    say("empty calls")
    B, H, d, N = 2, 64, 128, 64
    empty = lambda shape, dt: torch.zeros((shape[0], 1) + tuple(shape[2:]), dtype=dt, device=DEV)[:, :0]
    q = empty((B, 0, H, d), torch.bfloat16)
    kc = torch.zeros((B, N, d), dtype=torch.bfloat16, device=DEV)
    raw = torch.zeros((B, 300, d), dtype=torch.bfloat16, device=DEV)
    out = empty((B, 0, H, d), torch.float32)
    csa.hca_attend(q, kc, kc, 4, raw, raw, 10, 128, 0.1, out)
    csa.csa_attend(q, kc, kc, 4, empty((B, 0, 8), torch.int32), raw, raw, 10, 128, 0.1, out)
    csa.csa_index_topk(empty((B, 0, 8, 64), torch.bfloat16), None,
                       torch.zeros((B, N, 64), dtype=torch.bfloat16, device=DEV), None, 10, 4, 8,
                       empty((B, 0, 8), torch.int32))
    cache = torch.full((B, N, d), 7.0, device=DEV)
    z = torch.zeros(4, device=DEV)
    csa.csa_compress(raw.float(), z, 4, cache, entry_begin=5, entry_end=5)
    ring = torch.full((B, 2 * 8, d), 3.0, device=DEV)
    csa.csa_append(empty((B, 0, d), torch.float32), ring, 17, z, 4, cache)
    torch.cuda.synchronize()
    assert (cache == 7.0).all() and (ring == 3.0).all()


def test_append_of_the_largest_chunk():
    """4096 rows in one call (the limit): ring and compressed entries as from the
    full history, with the blocks before the chunk completed by an earlier call."""
    B, d, m, R = 2, 64, 4, 4096 + 4 - 1 + 5
    say("append max chunk", R)
    n = 4096 + 6
    hist = gen("app_big", (B, n, d), "bf16", seed=5)
    z = gen("app_big_z", (m,), "f32", seed=6, std=0.5).to(DEV)
    out = torch.full((B, n // m + 1, d), 7.0, dtype=torch.bfloat16, device=DEV)
    ring = torch.zeros((B, 2 * R, d), dtype=torch.bfloat16, device=DEV)
    hd = hist.to(DEV)
    csa.csa_append(hd[:, :6].contiguous(), ring, 0, z, m, out)
    csa.csa_append(hd[:, 6:].contiguous(), ring, 6, z, m, out)
    torch.cuda.synchronize()
    z64 = f64(z)
    for b in range(B):
        exp_ring = method.state_ring(f64(hist[b]), n - 1, R)
        held = ~np.isnan(exp_ring).any(axis=1)
        np.testing.assert_array_equal(f64(ring[b])[held], exp_ring[held])
        sums = method.compress_exact(f64(hist[b]), z64, m, 0, n // m)
        diff = ulp_diff_bf16(bf16_bits(out[b, :n // m]), formats.f64_to_bf16_bits(sums))
        assert diff.max() <= 1
        assert (f64(out[b, n // m:]) == 7.0).all()


def test_attend_is_deterministic_and_consistent_across_splits():
    """Same call twice: identical bits.  Decode rows (split) equal the same rows
    computed inside a prefill call (unsplit), within tolerance."""
    B, H, d, N, m, k, W = 2, 64, 128, 2000, 4, 1024, 128
    t_last = 4 * N - 1
    T = 6
    t0 = t_last - T + 1
    q = gen("det_q", (B, T, H, d), "bf16", seed=1).to(DEV)
    kc = gen("det_kc", (B, N, d), "bf16", seed=2, std=0.6).to(DEV)
    vc = gen("det_vc", (B, N, d), "bf16", seed=3, std=0.6).to(DEV)
    kr = gen("det_kr", (B, t_last + 1, d), "bf16", seed=4).to(DEV)
    vr = gen("det_vr", (B, t_last + 1, d), "bf16", seed=5).to(DEV)
    idx = torch.from_numpy(make_idx(B, T, k, t0, m, N, seed=9, bad_frac=0.0)).to(DEV)
    outs = []
    for _ in range(2):
        o = torch.empty((B, T, H, d), device=DEV)
        csa.csa_attend(q, kc, vc, m, idx, kr, vr, t0, W, 0.088, o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    last = torch.empty((B, 1, H, d), device=DEV)
    csa.csa_attend(q[:, -1:].contiguous(), kc, vc, m, idx[:, -1:].contiguous(), kr, vr, t_last, W,
                   0.088, last)
    torch.cuda.synchronize()
    ref = f64(outs[0][:, -1])
    diff = np.abs(f64(last[:, 0]) - ref).max(axis=-1)
    assert np.all(diff <= 1e-5 * np.abs(ref).max(axis=-1))


# ----------------------------------------------------------------------------- end to end, fp32


def test_chunked_prefill_rows_equal_full_prefill():
    """A prefill processed in chunks, each call continuing at t0 plus the rows
    already done, gives the rows of one call over the whole prefill.  Indexer:
    every chunk takes the prefill path, where a query's scores and selection do
    not depend on the other rows of the call, so lists and scores agree bit for
    bit.  Attention: the chunks run as split rows (three to four splits and a
    merge) where the whole prefill runs unsplit, so CSA rows agree to fp32
    summation order, 1e-4 of the row's largest output.  The whole HCA prefill
    runs on the multi-token kernel, whose softmax weights enter the value product
    as binary16 (relative error at most 2^-11 each) where V is in the binary16
    range, so there a row may move by up to 2^-11 of the largest |V| on top."""
    B, T, H, d, HI, dI, m, mh, k, W = 1, 320, 64, 128, 8, 64, 4, 128, 256, 128
    t0 = 20000
    n_raw = t0 + T
    N, Nh = n_raw // m, n_raw // mh
    chunks = [100, 64, 156]
    say("chunked vs full prefill", chunks)
    q_idx = gen("ch_qi", (B, T, HI, dI), "bf16", seed=1).to(DEV)
    w = gen("ch_w", (B, T, HI), "f32", seed=2).to(DEV)
    keys = gen("ch_ki", (B, N, dI), "bf16", seed=3).to(DEV)
    q = gen("ch_q", (B, T, H, d), "bf16", seed=4).to(DEV)
    kc, vc = gen("ch_kc", (B, N, d), "bf16", seed=5).to(DEV), gen("ch_vc", (B, N, d), "bf16", seed=6).to(DEV)
    kh, vh = gen("ch_kh", (B, Nh, d), "bf16", seed=7).to(DEV), gen("ch_vh", (B, Nh, d), "bf16", seed=8).to(DEV)
    kr, vr = gen("ch_kr", (B, n_raw, d), "bf16", seed=9).to(DEV), gen("ch_vr", (B, n_raw, d), "bf16", seed=10).to(DEV)
    scale = 1.0 / math.sqrt(d)

    def run(lo, hi, idx, sc, o_csa, l_csa, o_hca, l_hca):
        csa.csa_index_topk(q_idx[:, lo:hi], w[:, lo:hi], keys, None, t0 + lo, m, k, idx[:, lo:hi], sc[:, lo:hi])
        csa.csa_attend(q[:, lo:hi], kc, vc, m, idx[:, lo:hi], kr, vr, t0 + lo, W, scale, o_csa[:, lo:hi],
                       l_csa[:, lo:hi])
        csa.hca_attend(q[:, lo:hi], kh, vh, mh, kr, vr, t0 + lo, W, scale, o_hca[:, lo:hi], l_hca[:, lo:hi])

    def buffers():
        return (torch.full((B, T, k), -7, dtype=torch.int32, device=DEV),
                torch.full((B, T, k), 7.0, device=DEV),
                torch.full((B, T, H, d), 7.0, device=DEV), torch.full((B, T, H), 7.0, device=DEV),
                torch.full((B, T, H, d), 7.0, device=DEV), torch.full((B, T, H), 7.0, device=DEV))

    full, part = buffers(), buffers()
    run(0, T, *full)
    lo = 0
    for c in chunks:
        run(lo, lo + c, *part)
        lo += c
    torch.cuda.synchronize()
    assert torch.equal(full[0], part[0]), "indexer lists differ between chunked and whole prefill"
    assert torch.equal(full[1], part[1]), "indexer scores differ between chunked and whole prefill"
    vmax = max(float(f64(vh).__abs__().max()), float(f64(vr).__abs__().max()))
    for name, o_f, o_p, l_f, l_p, extra in (("csa", full[2], part[2], full[3], part[3], 0.0),
                                            ("hca", full[4], part[4], full[5], part[5], 2.0 ** -11 * vmax)):
        of, op = f64(o_f), f64(o_p)
        row_max = np.abs(of).max(axis=-1, keepdims=True)
        err = np.abs(of - op).max(axis=-1, keepdims=True)
        assert np.all(err <= 1e-4 * np.maximum(row_max, 1e-30) + extra), f"{name}: worst {np.max(err / row_max):.2e}"
        assert np.allclose(f64(l_f), f64(l_p), rtol=1e-6, atol=1e-5), f"{name}: lse"
        say(f"  {name}: worst row difference {np.max(err / np.maximum(row_max, 1e-30)):.2e} of the row maximum")


def test_decode_row_equals_the_last_prefill_row():
    """A decode call for the token at t = n - 1 (the rows x slices indexer, split
    attention with a merge) gives the last row of a prefill call ending at that
    token (the streaming prefill indexer, unsplit attention; HCA: the multi-token
    kernel): both selections are valid top-k sets of the oracle's scores, the
    decode scores of the shared winners agree with the prefill ones to fp32
    rounding, and, given the same selection, the attention rows agree to
    summation order (HCA also to its multi-token kernel's binary16 weights,
    2^-11 of the largest |V|)."""
    B, T, H, d, HI, dI, m, mh, k, W = 2, 128, 128, 128, 8, 64, 4, 128, 512, 128
    n = 24000
    t0 = n - T
    N, Nh = n // m, n // mh
    say("decode row vs last prefill row")
    q_idx = gen("dp_qi", (B, T, HI, dI), "bf16", seed=1)
    w = gen("dp_w", (B, T, HI), "f32", seed=2)
    keys = gen("dp_ki", (B, N, dI), "bf16", seed=3)
    q = gen("dp_q", (B, T, H, d), "bf16", seed=4).to(DEV)
    kc, vc = gen("dp_kc", (B, N, d), "bf16", seed=5).to(DEV), gen("dp_vc", (B, N, d), "bf16", seed=6).to(DEV)
    kh, vh = gen("dp_kh", (B, Nh, d), "bf16", seed=7).to(DEV), gen("dp_vh", (B, Nh, d), "bf16", seed=8).to(DEV)
    kr, vr = gen("dp_kr", (B, n, d), "bf16", seed=9).to(DEV), gen("dp_vr", (B, n, d), "bf16", seed=10).to(DEV)
    scale = 1.0 / math.sqrt(d)
    qd_idx, wd, kd = q_idx.to(DEV), w.to(DEV), keys.to(DEV)
    idx_p = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    sc_p = torch.full((B, T, k), 7.0, device=DEV)
    csa.csa_index_topk(qd_idx, wd, kd, None, t0, m, k, idx_p, sc_p)
    idx_d = torch.full((B, 1, k), -7, dtype=torch.int32, device=DEV)
    sc_d = torch.full((B, 1, k), 7.0, device=DEV)
    csa.csa_index_topk(qd_idx[:, T - 1:].contiguous(), wd[:, T - 1:].contiguous(), kd, None, n - 1, m, k, idx_d, sc_d)
    o_p = torch.empty((B, T, H, d), device=DEV)
    o_d = torch.empty((B, 1, H, d), device=DEV)
    csa.csa_attend(q, kc, vc, m, idx_p, kr, vr, t0, W, scale, o_p)
    last = idx_p[:, T - 1:].contiguous()
    csa.csa_attend(q[:, T - 1:].contiguous(), kc, vc, m, last, kr, vr, n - 1, W, scale, o_d)
    h_p = torch.empty((B, T, H, d), device=DEV)
    h_d = torch.empty((B, 1, H, d), device=DEV)
    csa.hca_attend(q, kh, vh, mh, kr, vr, t0, W, scale, h_p)
    csa.hca_attend(q[:, T - 1:].contiguous(), kh, vh, mh, kr, vr, n - 1, W, scale, h_d)
    torch.cuda.synchronize()
    ip, idd = idx_p.cpu().numpy(), idx_d.cpu().numpy()
    sp, sd = sc_p.cpu().numpy(), sc_d.cpu().numpy()
    for b in range(B):
        scores, vis = method.index_scores(f64(q_idx[b, T - 1:]), f64(w[b, T - 1:]), f64(keys[b]), n - 1, m)
        check_topk_rows(ip[b, T - 1:], sp[b, T - 1:], scores, vis, k)
        check_topk_rows(idd[b], sd[b], scores, vis, k)
        common = np.intersect1d(ip[b, T - 1], idd[b, 0])
        assert common.size >= k - 2, "the two selections differ beyond ties"
        a = dict(zip(ip[b, T - 1].tolist(), sp[b, T - 1].tolist()))
        c = dict(zip(idd[b, 0].tolist(), sd[b, 0].tolist()))
        rel = max(abs(a[j] - c[j]) / max(abs(a[j]), 1e-30) for j in common.tolist())
        assert rel <= 1e-5, rel
    vmax = max(float(f64(vh).__abs__().max()), float(f64(vr).__abs__().max()))
    for name, full, one, extra in (("csa", o_p, o_d, 0.0), ("hca", h_p, h_d, 2.0 ** -11 * vmax)):
        a, b_ = f64(full[:, T - 1]), f64(one[:, 0])
        err = np.abs(a - b_).max(axis=-1)
        ref = np.abs(a).max(axis=-1)
        say(f"  {name}: worst row difference {np.max(err / ref):.2e} of the row maximum")
        assert np.all(err <= 1e-4 * ref + extra), name


def test_tiny_prefill_f32_end_to_end():
    """Tiny CSA + HCA prefill in fp32, fully independent: the GPU runs compress ->
    index/top-k -> attend on its own outputs; the oracle runs its own pipeline.
    Rows whose selected set differs (only possible inside the tie band) are
    validated as sets and excluded from the output comparison."""
    wl = inputgen.WORKLOADS["tiny_prefill_f32"]
    say("end-to-end", wl)
    x = inputgen.make_inputs(wl, seed=0)
    dev = {k: v.to(DEV) for k, v in x.items()}
    n, N, Nh = wl.n, wl.N_c, wl.N_h
    kc = torch.empty((1, N, wl.d), device=DEV)
    vc = torch.empty((1, N, wl.d), device=DEV)
    kic = torch.empty((1, N, wl.d_I), device=DEV)
    csa.csa_compress(dev["k_raw"], dev["z_csa"], wl.m, kc)
    csa.csa_compress(dev["v_raw"], dev["z_csa"], wl.m, vc)
    csa.csa_compress(dev["k_idx_raw"], dev["z_csa"], wl.m, kic)
    idx = torch.empty((1, wl.T, wl.k), dtype=torch.int32, device=DEV)
    csa.csa_index_topk(dev["q_idx"], dev["w"], kic, None, wl.t0, wl.m, wl.k, idx)
    o = torch.empty((1, wl.T, wl.H, wl.d), device=DEV)
    lse = torch.empty((1, wl.T, wl.H), device=DEV)
    csa.csa_attend(dev["q"], kc, vc, wl.m, idx, dev["k_raw"], dev["v_raw"], wl.t0, wl.W, wl.scale,
                   o, lse)
    hk = torch.empty((1, Nh, wl.d), device=DEV)
    hv = torch.empty((1, Nh, wl.d), device=DEV)
    csa.csa_compress(dev["k_raw"], dev["z_hca"], wl.m_heavy, hk)
    csa.csa_compress(dev["v_raw"], dev["z_hca"], wl.m_heavy, hv)
    ho = torch.empty_like(o)
    hl = torch.empty_like(lse)
    csa.hca_attend(dev["q"], hk, hv, wl.m_heavy, dev["k_raw"], dev["v_raw"], wl.t0, wl.W, wl.scale,
                   ho, hl)
    torch.cuda.synchronize()

    ref = method.csa_layer(f64(x["q"][0]), f64(x["k_raw"][0]), f64(x["v_raw"][0]),
                           f64(x["q_idx"][0]), f64(x["k_idx_raw"][0]), f64(x["w"][0]),
                           f64(x["z_csa"]), wl.m, wl.k, wl.W, wl.scale, wl.t0)
    np.testing.assert_array_equal(f64(kc[0]), ref["k_cmp"]["values"])
    np.testing.assert_array_equal(f64(kic[0]), ref["k_idx"]["values"])
    g = idx[0].cpu().numpy()
    same = np.array([set(g[i][g[i] >= 0]) == set(ref["idx"][i][ref["idx"][i] >= 0])
                     for i in range(wl.T)])
    mism = np.nonzero(~same)[0]
    for i in mism:
        ok, why, _ = method.topk_is_valid(g[i], ref["scores"][i], ref["visible"][i], wl.k)
        assert ok, f"row {i}: {why}"
    say("  rows with an in-band set difference:", len(mism))
    assert len(mism) <= wl.T // 100
    check_attention(f64(o[0])[same], f64(lse[0])[same], ref["o"][same], ref["lse"][same], "f32", "csa e2e")
    href = method.hca_layer(f64(x["q"][0]), f64(x["k_raw"][0]), f64(x["v_raw"][0]),
                            f64(x["z_hca"]), wl.m_heavy, wl.W, wl.scale, wl.t0)
    np.testing.assert_array_equal(f64(hk[0]), href["k_cmp"]["values"])
    check_attention(f64(ho[0]), f64(hl[0]), href["o"], href["lse"], "f32", "hca e2e")


def test_gather_diagnostic_runs_in_bounds():
    """csa_diag_gather_read (the benchmark's gather-rate legs) on a small buffer with
    indices outside [0, n_rows) (clamped) and a ragged last round: it returns OK and the
    checksum sink is untouched (the buffers hold a constant, so it cannot hit the key)."""
    n_rows, per, groups = 1000, 77, 5
    k = torch.full((n_rows, 128), 1.0, dtype=torch.bfloat16, device=DEV)
    v = torch.full((n_rows, 128), 2.0, dtype=torch.bfloat16, device=DEV)
    idx = torch.randint(-50, n_rows + 50, (groups * per,), dtype=torch.int32, device=DEV)
    sink = torch.full((groups,), 7, dtype=torch.int32, device=DEV)
    csa.diag_gather_read(k, v, idx, per, sink)
    torch.cuda.synchronize()
    assert (sink == 7).all()
