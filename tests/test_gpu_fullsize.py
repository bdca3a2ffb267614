"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The benchmark's own step objects draw the seeded inputs on the GPU and run one
whole step (the compressed caches it builds are checked on sampled entries).
Then every later stage is run again, through the C ABI with the same shapes
and therefore the same launch plan, on inputs the oracle produced itself
(oracle-compressed keys and values, the oracle's own top-k), and compared:

* compressor: sampled entries of every cache against the oracle's fp64 block
  sum rounded once (bf16 bits within one step, e4m3 via the midpoint rule);
* indexer: every decode row (sampled query rows in prefill) must be a valid
  top-k of the oracle's fp64 scores over all visible entries;
* attention: sampled rows against the oracle's fp64 attention, 2e-3 of the
  row's largest magnitude.

Nothing the oracle consumes comes from the GPU: raw rows are regenerated from
their seeds (on the GPU, then copied), and the GPU gets the oracle's results.
"""
import numpy as np
import pytest
import torch

import bench
import compressed_attention_csa_amd as csa
import inputgen
from oracle import formats, method
from parity_util import (bf16_bits, check_attention, check_bf16_selection_row, check_e4m3, check_topk_rows,
                         check_topk_rows_fp8, f64, fp8_score_error_bound, ulp_diff_bf16)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 0
CHUNK = 1 << 17  # raw rows per host chunk


def say(*a):
    print(*a, flush=True)


def bf16_dev(x64: np.ndarray) -> torch.Tensor:
    bits = formats.f64_to_bf16_bits(x64)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def oracle_compress(raw_dev_row: torch.Tensor, z64, m: int, dtype: str, e0: int = 0, e1=None):
    """Oracle entries [e0, e1) of one sequence from its raw rows (device tensor [n, d]),
    computed chunk by chunk on the host.  Returns the oracle's store() dict."""
    n = raw_dev_row.shape[0]
    e1 = n // m if e1 is None else e1
    parts = {"values": [], "codes": [], "scale": []}
    step = CHUNK // m
    for a in range(e0, e1, step):
        b = min(e1, a + step)
        x = f64(raw_dev_row[a * m:b * m])
        st = method.store(method.compress_exact(x, z64, m, a, b, raw_base=a * m), dtype)
        for k in parts:
            if k in st:
                parts[k].append(st[k])
    return {k: np.concatenate(v) for k, v in parts.items() if v}


def check_cache_samples(cache, raw_dev, z64, m, dtype, scale=None, count=256, seed=1):
    """Sampled entries of a GPU-built cache [B, N, d] against the oracle."""
    B, N = cache.shape[0], cache.shape[1]
    rng = np.random.default_rng(seed)
    bs = rng.integers(0, B, count)
    js = rng.integers(0, N, count)
    rows = torch.stack([raw_dev[int(b), int(j) * m:(int(j) + 1) * m] for b, j in zip(bs, js)])
    x = f64(rows)  # [count, m, d]
    sums = np.einsum("s,csd->cd", method.compressor_weights(z64), x)
    if dtype == "e4m3":
        codes = cache[torch.from_numpy(bs).to(DEV), torch.from_numpy(js).to(DEV)].cpu().numpy()
        sc = scale[torch.from_numpy(bs).to(DEV), torch.from_numpy(js).to(DEV)].cpu().numpy()
        check_e4m3(codes, sc, sums.astype(np.float32))
    else:
        got = bf16_bits(cache[torch.from_numpy(bs).to(DEV), torch.from_numpy(js).to(DEV)])
        want = formats.f64_to_bf16_bits(sums)
        assert ulp_diff_bf16(got, want).max() <= 1, "compressed entry differs from the oracle"


def window_dev(raw_dev, n, W):
    return raw_dev[:, n - W:].contiguous()


# ----------------------------------------------------------------------------- CSA decode


@pytest.mark.parametrize("name", ["csa_decode_flash_128k", "csa_decode_pro_1m"])
def test_csa_decode_full_size(name):
    wl = inputgen.WORKLOADS[name]
    say("full-size", name)
    B, n, N, d, dI, m, k, W = wl.B, wl.n, wl.N_c, wl.d, wl.d_I, wl.m, wl.k, wl.W
    e4m3 = wl.idx_key_dtype == "e4m3"
    P = bench.DecodeCSA(wl, SEED, 1)
    P.step(0)
    torch.cuda.synchronize()
    c = P.reps[0]
    z64 = f64(inputgen.normal("z_csa", (m,), SEED, "f32", std=0.5, device=DEV))

    # compressor: sampled entries of the three caches the step used
    raw = {nm: inputgen.normal(nm, (B, n, dim), SEED, "bf16", device=DEV)
           for nm, dim in (("k_raw", d), ("v_raw", d), ("k_idx_raw", dI))}
    check_cache_samples(c["k_cmp"], raw["k_raw"], z64, m, "bf16")
    check_cache_samples(c["v_cmp"], raw["v_raw"], z64, m, "bf16", seed=2)
    check_cache_samples(c["k_idx"], raw["k_idx_raw"], z64, m, "e4m3" if e4m3 else "bf16",
                        scale=c["k_scale"], seed=3)
    say("  compressor samples ok")

    # indexer on oracle-compressed keys, same call as the step
    keys64 = []
    if e4m3:
        codes = torch.empty((B, N, dI), dtype=torch.uint8, device=DEV)
        scales = torch.empty((B, N), dtype=torch.float32, device=DEV)
    else:
        kbf = torch.empty((B, N, dI), dtype=torch.bfloat16, device=DEV)
    for b in range(B):
        st = oracle_compress(raw["k_idx_raw"][b], z64, m, "e4m3" if e4m3 else "bf16")
        keys64.append(st["values"])
        if e4m3:
            codes[b] = torch.from_numpy(st["codes"]).to(DEV)
            scales[b] = torch.from_numpy(st["scale"]).to(DEV)
        else:
            kbf[b] = bf16_dev(st["values"])
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    score = torch.empty((B, 1, k), dtype=torch.float32, device=DEV)
    csa.csa_index_topk(P.q_idx, P.w, codes if e4m3 else kbf, scales if e4m3 else None, wl.t0, m, k,
                       idx, score)
    torch.cuda.synchronize()
    q_idx64, w64 = f64(P.q_idx), f64(P.w)
    sel = []
    for b in range(B):
        s64, vis = method.index_scores(q_idx64[b], w64[b], keys64[b], wl.t0, m)
        check_topk_rows(idx[b].cpu().numpy(), score[b].cpu().numpy(), s64, vis, k)
        sel.append(method.select_topk(s64, vis, k)[0])
    del keys64
    say("  indexer rows ok")

    # attention on the oracle's selection and oracle-compressed entries
    kc = torch.zeros((B, N, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((B, N, d), dtype=torch.bfloat16, device=DEV)
    kc64, vc64 = [], []
    for b in range(B):
        js = sel[b][sel[b] >= 0]
        rows_k = f64(raw["k_raw"][b].view(N, m, d)[torch.from_numpy(js).to(DEV)])
        rows_v = f64(raw["v_raw"][b].view(N, m, d)[torch.from_numpy(js).to(DEV)])
        alpha = method.compressor_weights(z64)
        ek = formats.round_to_bf16(np.einsum("s,jsd->jd", alpha, rows_k))
        ev = formats.round_to_bf16(np.einsum("s,jsd->jd", alpha, rows_v))
        kc[b, torch.from_numpy(js).to(DEV)] = bf16_dev(ek)
        vc[b, torch.from_numpy(js).to(DEV)] = bf16_dev(ev)
        kc64.append((js, ek))
        vc64.append((js, ev))
    idx_o = torch.from_numpy(np.stack(sel)[:, None, :].astype(np.int32)).to(DEV)
    kw, vw = window_dev(raw["k_raw"], n, W), window_dev(raw["v_raw"], n, W)
    out = torch.empty((B, 1, wl.H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, wl.H), dtype=torch.float32, device=DEV)
    csa.csa_attend(P.q, kc, vc, m, idx_o, kw, vw, wl.t0, W, wl.scale, out, lse, raw_base=n - W)
    torch.cuda.synchronize()
    q64 = f64(P.q)
    for b in range(B):
        K = np.zeros((N, d))
        V = np.zeros((N, d))
        K[kc64[b][0]] = kc64[b][1]
        V[vc64[b][0]] = vc64[b][1]
        o_ref, l_ref = method.csa_attend(q64[b], K, V, sel[b][None, :], f64(kw[b]), f64(vw[b]), n - W,
                                         wl.t0, W, m, wl.scale)
        check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, "bf16", what=f"{name} b={b}")
    say("  attention rows ok")


def test_csa_decode_selector_variants_full_size():
    """The two selector variants the benchmark times beside the Pro-like decode
    (1M context, e4m3 keys), at that size and launch plan: the bf16 selector
    must be exactly the top-k of the oracle's scores rounded to binary32 and
    then bf16, and the fp8 x fp8 indexer a top-k of scores within the fp8 bound
    of the oracle's index_scores_fp8q.  Keys come from the oracle's compression."""
    name = "csa_decode_pro_1m"
    wl = inputgen.WORKLOADS[name]
    say("full-size selector variants", name)
    B, n, N, dI, m, k = wl.B, wl.n, wl.N_c, wl.d_I, wl.m, wl.k
    z64 = f64(inputgen.normal("z_csa", (m,), SEED, "f32", std=0.5, device=DEV))
    q_idx = inputgen.normal("q_idx", (B, 1, wl.H_I, dI), SEED, "bf16", device=DEV)
    w = inputgen.normal("w", (B, 1, wl.H_I), SEED, "f32", device=DEV)
    raw = inputgen.normal("k_idx_raw", (B, n, dI), SEED, "bf16", device=DEV)
    codes = torch.empty((B, N, dI), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, N), dtype=torch.float32, device=DEV)
    keys64 = []
    for b in range(B):
        st = oracle_compress(raw[b], z64, m, "e4m3")
        keys64.append(st["values"])
        codes[b] = torch.from_numpy(st["codes"]).to(DEV)
        scales[b] = torch.from_numpy(st["scale"]).to(DEV)
    del raw
    sel_b = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    sc_b = torch.empty((B, 1, k), dtype=torch.float32, device=DEV)
    csa.csa_index_topk(q_idx, w, codes, scales, wl.t0, m, k, sel_b, sc_b, bf16_scores=True)
    sel_q = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    sc_q = torch.empty((B, 1, k), dtype=torch.float32, device=DEV)
    csa.csa_index_topk_fp8(q_idx, w, codes, scales, wl.t0, m, k, sel_q, sc_q)
    torch.cuda.synchronize()
    q64, w64 = f64(q_idx), f64(w)
    total = hits = 0
    for b in range(B):
        s64, vis = method.index_scores(q64[b], w64[b], keys64[b], wl.t0, m)
        kk, h = check_bf16_selection_row(sel_b[b, 0].cpu().numpy(), sc_b[b, 0].cpu().numpy(), s64[0], vis[0], k)
        total, hits = total + kk, hits + h
        s8, vis8 = method.index_scores_fp8q(q64[b], w64[b], keys64[b], wl.t0, m)
        E = fp8_score_error_bound(method.quantize_query_e4m3(q64[b]), w64[b], keys64[b])
        check_topk_rows_fp8(sel_q[b].cpu().numpy(), sc_q[b].cpu().numpy(), s8, vis8, k, E)
    say(f"  bf16 selector recall against the exact top-k: {hits / total:.4f}; fp8 x fp8 rows ok")
    assert hits >= 0.95 * total


# ----------------------------------------------------------------------------- HCA decode


def test_hca_decode_full_size():
    name = "hca_decode_1m"
    wl = inputgen.WORKLOADS[name]
    say("full-size", name)
    B, n, Nh, d, mh, W = wl.B, wl.n, wl.N_h, wl.d, wl.m_heavy, wl.W
    P = bench.DecodeHCA(wl, SEED, 1)
    P.step(0)
    torch.cuda.synchronize()
    c = P.reps[0]
    z64 = f64(inputgen.normal("z_hca", (mh,), SEED, "f32", std=0.5, device=DEV))
    raw = {nm: inputgen.normal(nm, (B, n, d), SEED, "bf16", device=DEV) for nm in ("k_raw", "v_raw")}
    check_cache_samples(c["k_cmp"], raw["k_raw"], z64, mh, "bf16", count=64)
    check_cache_samples(c["v_cmp"], raw["v_raw"], z64, mh, "bf16", count=64, seed=2)
    say("  compressor samples ok")

    # Two sequences get oracle-compressed heavy entries; the rest attend zeros.
    checked = [0, B - 1]
    kc = torch.zeros((B, Nh, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((B, Nh, d), dtype=torch.bfloat16, device=DEV)
    ref = {}
    for b in checked:
        ek = oracle_compress(raw["k_raw"][b], z64, mh, "bf16")["values"]
        ev = oracle_compress(raw["v_raw"][b], z64, mh, "bf16")["values"]
        kc[b] = bf16_dev(ek)
        vc[b] = bf16_dev(ev)
        ref[b] = (ek, ev)
    kw, vw = window_dev(raw["k_raw"], n, W), window_dev(raw["v_raw"], n, W)
    out = torch.empty((B, 1, wl.H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, wl.H), dtype=torch.float32, device=DEV)
    csa.hca_attend(P.q, kc, vc, mh, kw, vw, wl.t0, W, wl.scale, out, lse, raw_base=n - W)
    torch.cuda.synchronize()
    q64 = f64(P.q)
    for b in checked:
        o_ref, l_ref = method.hca_attend(q64[b], ref[b][0], ref[b][1], mh, f64(kw[b]), f64(vw[b]),
                                         n - W, wl.t0, W, wl.scale)
        check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, "bf16", what=f"{name} b={b}")
    say("  attention rows ok")


def test_hca_decode_fp8_caches_full_size():
    """The fp8 variant of the HCA decode leg: e4m3 heavy caches as the bench builds
    them (sampled entries against the oracle's quantiser), then whole decode rows of
    two sequences on oracle-quantised caches against the oracle over code * scale."""
    name = "hca_decode_1m"
    wl = inputgen.WORKLOADS[name]
    say("full-size fp8 caches", name)
    B, n, Nh, d, mh, W = wl.B, wl.n, wl.N_h, wl.d, wl.m_heavy, wl.W
    P = bench.DecodeHCA(wl, SEED, 1, variant="fp8kv")
    P.step(0)
    torch.cuda.synchronize()
    c = P.reps[0]
    z64 = f64(inputgen.normal("z_hca", (mh,), SEED, "f32", std=0.5, device=DEV))
    raw = {nm: inputgen.normal(nm, (B, n, d), SEED, "bf16", device=DEV) for nm in ("k_raw", "v_raw")}
    check_cache_samples(c["k_cmp"], raw["k_raw"], z64, mh, "e4m3", scale=c["k_scale"], count=64)
    check_cache_samples(c["v_cmp"], raw["v_raw"], z64, mh, "e4m3", scale=c["v_scale"], count=64, seed=2)
    say("  compressor samples ok")
    checked = [0, B - 1]
    kc = torch.zeros((B, Nh, d), dtype=torch.uint8, device=DEV)
    vc = torch.zeros((B, Nh, d), dtype=torch.uint8, device=DEV)
    ks = torch.ones((B, Nh), device=DEV)
    vs = torch.ones((B, Nh), device=DEV)
    ref = {}
    for b in checked:
        sk = oracle_compress(raw["k_raw"][b], z64, mh, "e4m3")
        sv = oracle_compress(raw["v_raw"][b], z64, mh, "e4m3")
        kc[b], ks[b] = torch.from_numpy(sk["codes"]).to(DEV), torch.from_numpy(sk["scale"]).to(DEV)
        vc[b], vs[b] = torch.from_numpy(sv["codes"]).to(DEV), torch.from_numpy(sv["scale"]).to(DEV)
        ref[b] = (sk["values"], sv["values"])
    kw, vw = window_dev(raw["k_raw"], n, W), window_dev(raw["v_raw"], n, W)
    out = torch.empty((B, 1, wl.H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, wl.H), dtype=torch.float32, device=DEV)
    csa.hca_attend(P.q, kc, vc, mh, kw, vw, wl.t0, W, wl.scale, out, lse, raw_base=n - W, k_scale=ks,
                   v_scale=vs)
    torch.cuda.synchronize()
    q64 = f64(P.q)
    for b in checked:
        o_ref, l_ref = method.hca_attend(q64[b], ref[b][0], ref[b][1], mh, f64(kw[b]), f64(vw[b]),
                                         n - W, wl.t0, W, wl.scale)
        check_attention(f64(out[b]), f64(lse[b]), o_ref, l_ref, "bf16", what=f"{name} fp8 b={b}")
    say("  attention rows ok")


# ----------------------------------------------------------------------------- CSA prefill


def sample_rows(T, fixed, seed, count=64):
    """count query rows of a prefill chunk: the fixed ones (chunk edges, workgroup
    boundaries) and seeded random ones spread over every part of the chunk."""
    rng = np.random.default_rng(seed)
    rows = set(fixed)
    while len(rows) < count:
        rows.add(int(rng.integers(0, T)))
    return sorted(rows)


def test_csa_prefill_chunk_full_size():
    name = "csa_prefill_chunk_1m"
    wl = inputgen.WORKLOADS[name]
    say("full-size", name)
    n, N, d, dI, m, k, W, T = wl.n, wl.N_c, wl.d, wl.d_I, wl.m, wl.k, wl.W, wl.T
    P = bench.PrefillCSA(wl, SEED, 1)
    P.step(0)
    torch.cuda.synchronize()
    z64 = f64(inputgen.normal("z_csa", (m,), SEED, "f32", std=0.5, device=DEV))
    # caches: entries of the prior context and of the chunk compressed in the step
    for nm, key, sd in (("k_raw", "k_raw", 1), ("v_raw", "v_raw", 2), ("k_idx_raw", "k_idx_raw", 3)):
        check_cache_samples(P.cmp[key], P.raw[nm], z64, m, "bf16", seed=sd)
        tail = P.cmp[key][:, wl.cmp_begin:]
        check_cache_samples(tail, P.raw[nm][:, wl.cmp_begin * m:], z64, m, "bf16", seed=sd + 10)
    say("  compressor samples ok")

    # indexer for every query on oracle-compressed keys; sampled rows checked
    keys64 = oracle_compress(P.raw["k_idx_raw"][0], z64, m, "bf16")["values"]
    kbf = bf16_dev(keys64)[None]
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    score = torch.empty((1, T, k), dtype=torch.float32, device=DEV)
    csa.csa_index_topk(P.q_idx, P.w, kbf, None, wl.t0, m, k, idx, score)
    torch.cuda.synchronize()
    rows = sample_rows(T, [0, 1, 2047, 4096, 5000, T - 2, T - 1], seed=21)
    q_idx64, w64 = f64(P.q_idx[0]), f64(P.w[0])
    idx_h, score_h = idx[0].cpu().numpy(), score[0].cpu().numpy()
    sel = {}
    for i in rows:
        s64, vis = method.index_scores(q_idx64[i:i + 1], w64[i:i + 1], keys64, wl.t0 + i, m)
        check_topk_rows(idx_h[i:i + 1], score_h[i:i + 1], s64, vis, k)
        sel[i] = method.select_topk(s64, vis, k)[0]
    say("  indexer rows ok")

    # attention: sampled rows carry the oracle's selection, the others none
    idx_o = np.full((1, T, k), -1, dtype=np.int32)
    for i in rows:
        idx_o[0, i] = sel[i]
    used = np.unique(np.concatenate([sel[i][sel[i] >= 0] for i in rows]))
    used_d = torch.from_numpy(used).to(DEV)
    alpha = method.compressor_weights(z64)
    ek = formats.round_to_bf16(np.einsum("s,jsd->jd", alpha, f64(P.raw["k_raw"][0].view(N, m, d)[used_d])))
    ev = formats.round_to_bf16(np.einsum("s,jsd->jd", alpha, f64(P.raw["v_raw"][0].view(N, m, d)[used_d])))
    kc = torch.zeros((1, N, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((1, N, d), dtype=torch.bfloat16, device=DEV)
    kc[0, used_d] = bf16_dev(ek)
    vc[0, used_d] = bf16_dev(ev)
    out = torch.empty((1, T, wl.H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, T, wl.H), dtype=torch.float32, device=DEV)
    csa.csa_attend(P.q, kc, vc, m, torch.from_numpy(idx_o).to(DEV), P.raw["k_raw"], P.raw["v_raw"],
                   wl.t0, W, wl.scale, out, lse)
    torch.cuda.synchronize()
    K = np.zeros((N, d))
    V = np.zeros((N, d))
    K[used], V[used] = ek, ev
    q64 = f64(P.q[0])
    for i in rows:
        t = wl.t0 + i
        win = method.window_positions(t, W)
        kr = f64(P.raw["k_raw"][0, int(win[0]):int(win[-1]) + 1])
        vr = f64(P.raw["v_raw"][0, int(win[0]):int(win[-1]) + 1])
        o_ref, l_ref = method.csa_attend(q64[i:i + 1], K, V, sel[i][None, :], kr, vr, int(win[0]), t, W, m,
                                         wl.scale)
        check_attention(f64(out[0, i:i + 1]), f64(lse[0, i:i + 1]), o_ref, l_ref, "bf16", what=f"{name} row {i}")
    say("  attention rows ok")


# ----------------------------------------------------------------------------- HCA prefill


def test_hca_prefill_chunk_full_size():
    name = "hca_prefill_chunk_1m"
    wl = inputgen.WORKLOADS[name]
    say("full-size", name)
    n, Nh, d, mh, W, T = wl.n, wl.N_h, wl.d, wl.m_heavy, wl.W, wl.T
    P = bench.PrefillHCA(wl, SEED, 1)
    P.step(0)
    torch.cuda.synchronize()
    z64 = f64(inputgen.normal("z_hca", (mh,), SEED, "f32", std=0.5, device=DEV))
    for nm, sd in (("k_raw", 1), ("v_raw", 2)):
        check_cache_samples(P.cmp[nm], P.raw[nm], z64, mh, "bf16", count=64, seed=sd)
        tail = P.cmp[nm][:, wl.cmp_begin:]
        check_cache_samples(tail, P.raw[nm][:, wl.cmp_begin * mh:], z64, mh, "bf16", count=64, seed=sd + 10)
    say("  compressor samples ok")

    # every query of the chunk on oracle-compressed heavy entries; sampled rows checked
    ek = oracle_compress(P.raw["k_raw"][0], z64, mh, "bf16")["values"]
    ev = oracle_compress(P.raw["v_raw"][0], z64, mh, "bf16")["values"]
    out = torch.empty((1, T, wl.H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, T, wl.H), dtype=torch.float32, device=DEV)
    csa.hca_attend(P.q, bf16_dev(ek)[None], bf16_dev(ev)[None], mh, P.raw["k_raw"], P.raw["v_raw"],
                   wl.t0, W, wl.scale, out, lse)
    torch.cuda.synchronize()
    q64 = f64(P.q[0])
    for i in sample_rows(T, [0, 1, 127, 128, 4095, 5000, T - 2, T - 1], seed=22):
        t = wl.t0 + i
        win = method.window_positions(t, W)
        kr = f64(P.raw["k_raw"][0, int(win[0]):int(win[-1]) + 1])
        vr = f64(P.raw["v_raw"][0, int(win[0]):int(win[-1]) + 1])
        o_ref, l_ref = method.hca_attend(q64[i:i + 1], ek, ev, mh, kr, vr, int(win[0]), t, W, wl.scale)
        check_attention(f64(out[0, i:i + 1]), f64(lse[0, i:i + 1]), o_ref, l_ref, "bf16",
                        what=f"{name} row {i}")
    say("  attention rows ok")
