#!/usr/bin/env python
"""Benchmark of the compressed-attention hot path on one MI355X.

Prints ONE JSON line.  The headline is the Pro-like CSA decode step at 1M
context (4 sequences, 128 query heads, e4m3 indexer keys, top-1024 + 128-token
window): one step = csa_index_topk + csa_attend for one new query token per
sequence, with every input already resident in HBM.  ``value`` is decode
query-tokens/s.  The same line carries "legs" for the HCA dense decode at 1M,
the CSA chunked prefill at 1M (which also compresses the chunk's new blocks),
the Flash-like CSA decode at 128K, the HCA chunked prefill at 1M and the
Pro-like decode with state-cache maintenance (csa_append of the new token's
K, V and indexer-key rows before the step) and the HCA decode over fp8-e4m3
heavy caches, so that every step of the path is measured.

Decode steps are measured cache-cold: each step reads its own replica of the
caches, and the replicas together are at least twice the 256 MB Infinity
Cache.  Steps are captured in a HIP graph (torch.cuda.CUDAGraph) and replayed;
the timed region is bracketed by device synchronisation.  The dominant kernel
is also timed on its own with HIP events recorded by the library around each
launch (csa_profile_enable), which gives the roofline figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "decode query-tokens/s + HBM GB/s at 1M ctx; prefill TFLOP/s (frac. of peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- workloads


class DecodeCSA:
    """CSA decode step: index + top-k over all compressed entries, then attention.

    With ``state`` the step first appends the new token's K, V and indexer-key
    rows to the state-cache rings (compressing the block the token completes)
    and the attention reads its window from the K / V rings.  With ``bf16sel``
    the selection is the approximate one (top-k of bf16-rounded scores); its
    recall against the exact selection is reported beside the timing."""

    dominant = "index_topk"

    def __init__(self, wl, seed, replicas, variant=""):
        assert variant in ("", "state", "bf16sel"), variant
        state = variant == "state"
        self.bf16sel = variant == "bf16sel"
        import torch
        import compressed_attention_csa_amd as csa
        import inputgen
        self.wl, self.csa, self.torch = wl, csa, torch
        dev = "cuda"
        B, n, d, dI, N, W = wl.B, wl.n, wl.d, wl.d_I, wl.N_c, wl.W
        e4m3 = wl.idx_key_dtype == "e4m3"
        self.q = inputgen.normal("q", (B, 1, wl.H, d), seed, "bf16", device=dev)
        self.q_idx = inputgen.normal("q_idx", (B, 1, wl.H_I, dI), seed, "bf16", device=dev)
        self.w = inputgen.normal("w", (B, 1, wl.H_I), seed, "f32", device=dev)
        z = inputgen.normal("z_csa", (wl.m,), seed, "f32", std=0.5, device=dev)
        self.z, self.state = z, state
        R = W + wl.m  # state-cache ring rows
        caches, self.new = {}, {}
        for name, dim in (("k_raw", d), ("v_raw", d), ("k_idx_raw", dI)):
            raw = inputgen.normal(name, (B, n, dim), seed, "bf16", device=dev)
            if state:  # the newest R positions, as the appends of earlier steps left them
                ring = torch.empty((B, 2 * R, dim), dtype=torch.bfloat16, device=dev)
                rows = torch.arange(n - R, n, device=dev) % R
                ring[:, rows] = raw[:, n - R:]
                ring[:, rows + R] = raw[:, n - R:]
                caches["ring_" + name] = ring
                self.new[name] = raw[:, n - 1:].contiguous()
            if name == "k_idx_raw":
                if e4m3:
                    out = torch.empty((B, N, dI), dtype=torch.uint8, device=dev)
                    sc = torch.empty((B, N), device=dev)
                    csa.csa_compress(raw, z, wl.m, out, sc)
                    caches["k_idx"], caches["k_scale"] = out, sc
                else:
                    out = torch.empty((B, N, dI), dtype=torch.bfloat16, device=dev)
                    csa.csa_compress(raw, z, wl.m, out)
                    caches["k_idx"], caches["k_scale"] = out, None
            else:
                out = torch.empty((B, N, d), dtype=torch.bfloat16, device=dev)
                csa.csa_compress(raw, z, wl.m, out)
                caches[name.replace("_raw", "_cmp")] = out
                caches[name.replace("_raw", "_win")] = raw[:, n - W:].contiguous()
            del raw
        torch.cuda.synchronize()
        self.reps = [caches] + [{k: (None if v is None else v.clone()) for k, v in caches.items()}
                                for _ in range(replicas - 1)]
        self.idx = torch.empty((B, 1, wl.k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, 1, wl.H, d), dtype=torch.float32, device=dev)
        self.raw_base = n - W
        torch.cuda.synchronize()

    def step(self, r):
        wl, csa, c = self.wl, self.csa, self.reps[r % len(self.reps)]
        if self.state:
            csa.csa_append(self.new["k_raw"], c["ring_k_raw"], wl.t0, self.z, wl.m, c["k_cmp"])
            csa.csa_append(self.new["v_raw"], c["ring_v_raw"], wl.t0, self.z, wl.m, c["v_cmp"])
            csa.csa_append(self.new["k_idx_raw"], c["ring_k_idx_raw"], wl.t0, self.z, wl.m, c["k_idx"],
                           c["k_scale"])
        csa.csa_index_topk(self.q_idx, self.w, c["k_idx"], c["k_scale"], wl.t0, wl.m, wl.k, self.idx,
                           bf16_scores=self.bf16sel)
        if self.state:
            kr, base = csa.ring_window(c["ring_k_raw"], wl.t0 - wl.W + 1)
            csa.csa_attend(self.q, c["k_cmp"], c["v_cmp"], wl.m, self.idx, kr, c["ring_v_raw"], wl.t0,
                           wl.W, wl.scale, self.out, raw_base=base)
        else:
            csa.csa_attend(self.q, c["k_cmp"], c["v_cmp"], wl.m, self.idx, c["k_win"], c["v_win"], wl.t0,
                           wl.W, wl.scale, self.out, raw_base=self.raw_base)

    def quality(self):
        """Recall of the approximate selection against the exact one (replica 0)."""
        if not self.bf16sel:
            return None
        wl, csa, torch, c = self.wl, self.csa, self.torch, self.reps[0]
        sel = {}
        for approx in (False, True):
            idx = torch.empty_like(self.idx)
            csa.csa_index_topk(self.q_idx, self.w, c["k_idx"], c["k_scale"], wl.t0, wl.m, wl.k, idx,
                               bf16_scores=approx)
            sel[approx] = idx.cpu()
        hits = sum(len(set(sel[True][b, 0].tolist()) & set(sel[False][b, 0].tolist())) for b in range(wl.B))
        return {"recall_vs_exact": round(hits / (wl.B * wl.k), 5)}

    def algorithmic(self):
        wl = self.wl
        kb = 1 if wl.idx_key_dtype == "e4m3" else 2
        keys = wl.B * wl.N_c * wl.d_I * kb + (wl.B * wl.N_c * 4 if kb == 1 else 0)
        qi = wl.B * wl.H_I * wl.d_I * 2 + wl.B * wl.H_I * 4
        idx = wl.B * wl.k * 4 * 2
        gathered = wl.B * wl.k * wl.d * 2 * 2
        window = wl.B * wl.W * wl.d * 2 * 2
        q = wl.B * wl.H * wl.d * 2
        o = wl.B * wl.H * wl.d * 4
        flops = 2 * wl.B * wl.N_c * wl.H_I * wl.d_I + 4 * wl.B * wl.H * wl.d * (wl.k + wl.W)
        state = 0
        if self.state:  # new rows read, written twice; the completed block read, its entry written
            row = wl.B * (2 * wl.d + wl.d_I) * 2
            state = 3 * row + wl.m * row + wl.B * (2 * wl.d * 2 + wl.d_I * kb)
        return {"bytes": keys + qi + idx + gathered + window + q + o + state, "flops": flops,
                "dominant_bytes": keys + qi, "queries": wl.B}


class DecodeHCA:
    """HCA decode step: dense attention over every heavy entry plus the window.
    Variant ``fp8kv``: the heavy K / V caches are e4m3 codes with per-entry
    scales (as csa_compress writes them)."""

    dominant = "hca_attend"

    def __init__(self, wl, seed, replicas, variant=""):
        import torch
        import compressed_attention_csa_amd as csa
        import inputgen
        assert variant in ("", "fp8kv"), variant
        self.wl, self.csa, self.kv8 = wl, csa, variant == "fp8kv"
        dev = "cuda"
        B, n, d, Nh, W = wl.B, wl.n, wl.d, wl.N_h, wl.W
        self.q = inputgen.normal("q", (B, 1, wl.H, d), seed, "bf16", device=dev)
        z = inputgen.normal("z_hca", (wl.m_heavy,), seed, "f32", std=0.5, device=dev)
        caches = {}
        for name in ("k_raw", "v_raw"):
            raw = inputgen.normal(name, (B, n, d), seed, "bf16", device=dev)
            key = name.replace("_raw", "_cmp")
            if self.kv8:
                out = torch.empty((B, Nh, d), dtype=torch.uint8, device=dev)
                sc = torch.empty((B, Nh), device=dev)
                csa.csa_compress(raw, z, wl.m_heavy, out, sc)
                caches[key.replace("_cmp", "_scale")] = sc
            else:
                out = torch.empty((B, Nh, d), dtype=torch.bfloat16, device=dev)
                csa.csa_compress(raw, z, wl.m_heavy, out)
            caches[key] = out
            caches[name.replace("_raw", "_win")] = raw[:, n - W:].contiguous()
            del raw
        torch.cuda.synchronize()
        self.reps = [caches] + [{k: v.clone() for k, v in caches.items()} for _ in range(replicas - 1)]
        self.out = torch.empty((B, 1, wl.H, d), dtype=torch.float32, device=dev)
        self.raw_base = n - W
        torch.cuda.synchronize()

    def step(self, r):
        wl, c = self.wl, self.reps[r % len(self.reps)]
        self.csa.hca_attend(self.q, c["k_cmp"], c["v_cmp"], wl.m_heavy, c["k_win"], c["v_win"], wl.t0,
                            wl.W, wl.scale, self.out, raw_base=self.raw_base, k_scale=c.get("k_scale"),
                            v_scale=c.get("v_scale"))

    def algorithmic(self):
        wl = self.wl
        kv = wl.B * wl.N_h * (wl.d + 4) * 2 if self.kv8 else wl.B * wl.N_h * wl.d * 2 * 2
        window = wl.B * wl.W * wl.d * 2 * 2
        q = wl.B * wl.H * wl.d * 2
        o = wl.B * wl.H * wl.d * 4
        total = kv + window + q + o
        flops = 4 * wl.B * wl.H * wl.d * (wl.N_h + wl.W)
        return {"bytes": total, "flops": flops, "dominant_bytes": total, "queries": wl.B}


class PrefillCSA:
    """Chunked prefill: compress the chunk's new blocks, index + top-k for every new
    query over all visible entries, attention."""

    dominant = "index_topk"

    def __init__(self, wl, seed, replicas):
        import torch
        import compressed_attention_csa_amd as csa
        import inputgen
        self.wl, self.csa = wl, csa
        dev = "cuda"
        B, n, d, dI, N = wl.B, wl.n, wl.d, wl.d_I, wl.N_c
        self.q = inputgen.normal("q", (B, wl.T, wl.H, d), seed, "bf16", device=dev)
        self.q_idx = inputgen.normal("q_idx", (B, wl.T, wl.H_I, dI), seed, "bf16", device=dev)
        self.w = inputgen.normal("w", (B, wl.T, wl.H_I), seed, "f32", device=dev)
        self.z = inputgen.normal("z_csa", (wl.m,), seed, "f32", std=0.5, device=dev)
        self.raw = {name: inputgen.normal(name, (B, n, dim), seed, "bf16", device=dev)
                    for name, dim in (("k_raw", d), ("v_raw", d), ("k_idx_raw", dI))}
        self.cmp = {"k_raw": torch.empty((B, N, d), dtype=torch.bfloat16, device=dev),
                    "v_raw": torch.empty((B, N, d), dtype=torch.bfloat16, device=dev),
                    "k_idx_raw": torch.empty((B, N, dI), dtype=torch.bfloat16, device=dev)}
        for name, out in self.cmp.items():  # the prior context, compressed before the step
            csa.csa_compress(self.raw[name], self.z, wl.m, out, entry_begin=0, entry_end=wl.cmp_begin)
        self.idx = torch.empty((B, wl.T, wl.k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, wl.T, wl.H, d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def step(self, r):
        wl, csa = self.wl, self.csa
        for name, out in self.cmp.items():
            csa.csa_compress(self.raw[name], self.z, wl.m, out, entry_begin=wl.cmp_begin,
                             entry_end=wl.N_c)
        csa.csa_index_topk(self.q_idx, self.w, self.cmp["k_idx_raw"], None, wl.t0, wl.m, wl.k, self.idx)
        csa.csa_attend(self.q, self.cmp["k_raw"], self.cmp["v_raw"], wl.m, self.idx, self.raw["k_raw"],
                       self.raw["v_raw"], wl.t0, wl.W, wl.scale, self.out)

    def algorithmic(self):
        wl = self.wl
        sum_c = sum(min(wl.N_c, (wl.t0 + i + 1) // wl.m) for i in range(wl.T))
        idx_flops = 2 * wl.B * wl.H_I * wl.d_I * sum_c
        att_slots = sum(min(wl.k, min(wl.N_c, (wl.t0 + i + 1) // wl.m)) + min(wl.W, wl.t0 + i + 1)
                        for i in range(wl.T))
        att_flops = 4 * wl.B * wl.H * wl.d * att_slots
        return {"bytes": None, "flops": idx_flops + att_flops, "dominant_flops": idx_flops,
                "queries": wl.B * wl.T}


class PrefillHCA:
    """HCA chunked prefill: compress the chunk's new heavy blocks, then dense attention
    of every new query over the visible heavy entries and its window."""

    dominant = "hca_attend"

    def __init__(self, wl, seed, replicas):
        import torch
        import compressed_attention_csa_amd as csa
        import inputgen
        self.wl, self.csa = wl, csa
        dev = "cuda"
        B, n, d, N = wl.B, wl.n, wl.d, wl.N_h
        self.q = inputgen.normal("q", (B, wl.T, wl.H, d), seed, "bf16", device=dev)
        self.z = inputgen.normal("z_hca", (wl.m_heavy,), seed, "f32", std=0.5, device=dev)
        self.raw = {name: inputgen.normal(name, (B, n, d), seed, "bf16", device=dev)
                    for name in ("k_raw", "v_raw")}
        self.cmp = {name: torch.empty((B, N, d), dtype=torch.bfloat16, device=dev) for name in self.raw}
        for name, out in self.cmp.items():  # the prior context, compressed before the step
            csa.csa_compress(self.raw[name], self.z, wl.m_heavy, out, entry_begin=0,
                             entry_end=wl.cmp_begin)
        self.out = torch.empty((B, wl.T, wl.H, d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def step(self, r):
        wl, csa = self.wl, self.csa
        for name, out in self.cmp.items():
            csa.csa_compress(self.raw[name], self.z, wl.m_heavy, out, entry_begin=wl.cmp_begin,
                             entry_end=wl.N_h)
        csa.hca_attend(self.q, self.cmp["k_raw"], self.cmp["v_raw"], wl.m_heavy, self.raw["k_raw"],
                       self.raw["v_raw"], wl.t0, wl.W, wl.scale, self.out)

    def algorithmic(self):
        wl = self.wl
        slots = sum(min(wl.N_h, (wl.t0 + i + 1) // wl.m_heavy) + min(wl.W, wl.t0 + i + 1)
                    for i in range(wl.T))
        flops = 4 * wl.B * wl.H * wl.d * slots
        return {"bytes": None, "flops": flops, "dominant_flops": flops, "queries": wl.B * wl.T}


KINDS = {"csa_decode_pro_1m": DecodeCSA, "csa_decode_flash_128k": DecodeCSA,
         "hca_decode_1m": DecodeHCA, "csa_prefill_chunk_1m": PrefillCSA,
         "hca_prefill_chunk_1m": PrefillHCA}
REPLICAS = {"csa_decode_pro_1m": 8, "csa_decode_flash_128k": 16, "hca_decode_1m": 8,
            "csa_prefill_chunk_1m": 1, "hca_prefill_chunk_1m": 1}


# ----------------------------------------------------------------------------- timing


def time_workload(name, seed, steps, warmup, graph=True):
    import torch
    import compressed_attention_csa_amd as csa
    import inputgen
    base, _, variant = name.partition("+")  # "+state": the decode step also maintains the state cache
    wl = inputgen.WORKLOADS[base]
    R = REPLICAS[base]
    log(f"[bench] {name}: setting up ({R} replica(s))")
    t = time.time()
    w = KINDS[base](wl, seed, R, **({"variant": variant} if variant else {}))
    log(f"[bench] {name}: setup {time.time() - t:.1f}s; warmup {warmup}")
    for i in range(max(warmup, R)):
        w.step(i)
    torch.cuda.synchronize()
    # Dominant kernel, timed per launch with the library's HIP events (eager).
    csa.profile_enable(True)
    nprof = min(max(2 * R, 8), steps) if R > 1 else min(3, steps)
    for i in range(nprof):
        w.step(i)
    torch.cuda.synchronize()
    csa.profile_enable(False)
    prof = csa.profile_report()
    # Headline timing: graph replay of R steps (one per replica).
    reps = max(1, steps // R)
    g = None
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(R):
                w.step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                w.step(i)
        g.replay()
        torch.cuda.synchronize()
    log(f"[bench] {name}: timing {reps * R} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        if g is not None:
            g.replay()
        else:
            for i in range(R):
                w.step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * R)
    alg = w.algorithmic()
    res = {"workload": name, "ms_per_step": ms, "steps": reps * R, "replicas": R, "kernels": prof,
           "alg": alg, "dominant": w.dominant}
    dom = prof.get(w.dominant)
    if dom:
        res["dominant_ms"] = dom["total_ms"] / dom["launches"]
    q = w.quality() if hasattr(w, "quality") else None
    if q:
        res["quality"] = q
    del w, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def summarize(res):
    alg, ms = res["alg"], res["ms_per_step"]
    out = {"ms_per_step": round(ms, 6), "steps": res["steps"], "cache_cold_replicas": res["replicas"],
           "query_tokens_per_s": alg["queries"] / (ms * 1e-3)}
    if alg.get("bytes"):
        gbps = alg["bytes"] / (ms * 1e-3) / 1e9
        out.update({"hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "alg_bytes": alg["bytes"]})
    tf = alg["flops"] / (ms * 1e-3) / 1e12
    out.update({"tflops": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "alg_flops": alg["flops"]})
    out["kernel_ms"] = {k: round(v["total_ms"] / v["launches"], 6) for k, v in res["kernels"].items()}
    out.update(res.get("quality") or {})
    return out


def roofline(res):
    alg = res["alg"]
    dom_ms = res.get("dominant_ms")
    if dom_ms is None:
        return None
    key = f"{res['dominant']}@{res['workload']}"
    traffic = load_traffic(key)
    if "dominant_bytes" in alg:
        achieved = alg["dominant_bytes"] / (dom_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic, "kernel": res["dominant"],
                "kernel_ms": round(dom_ms, 6), "alg_bytes_per_launch": alg["dominant_bytes"]}
    achieved = alg["dominant_flops"] / (dom_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": res["dominant"],
            "kernel_ms": round(dom_ms, 6), "alg_flops_per_launch": alg["dominant_flops"]}


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_attention_csa_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources (else null)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- CPU baseline


CPU_SAMPLE_SECONDS = 12.0  # bounded oracle sample, so the default run stays within minutes


def cpu_baseline(seed):
    """The fp64 oracle on the host: one Pro-like decode step for one sequence."""
    import numpy as np
    import torch
    import inputgen
    from oracle import method
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info = None
    wl = inputgen.WORKLOADS["csa_decode_pro_1m"]
    cores = len(os.sched_getaffinity(0))
    threads = cores
    if threadpool_info is not None:
        cap = min([p.get("num_threads", cores) for p in threadpool_info() if p.get("user_api") == "blas"]
                  or [cores])
        threads = min(cores, 64, max(cap, 1))
    log(f"[bench] cpu baseline: oracle inputs for sequence 0 (untimed), {threads} BLAS threads")
    # Inputs of sequence 0 from the same generator (drawn on the GPU, copied to the host).
    dev = "cuda"
    B, n = wl.B, wl.n

    def seq0(name, shape, dt, std=1.0):
        return inputgen.normal(name, shape, seed, dt, std=std, device=dev)[0].cpu()

    q = seq0("q", (B, 1, wl.H, wl.d), "bf16").double().numpy()
    qi = seq0("q_idx", (B, 1, wl.H_I, wl.d_I), "bf16").double().numpy()
    w = seq0("w", (B, 1, wl.H_I), "f32").double().numpy()
    z = inputgen.normal("z_csa", (wl.m,), seed, "f32", std=0.5, device=dev).cpu().double().numpy()
    k_raw = seq0("k_raw", (B, n, wl.d), "bf16").double().numpy()
    v_raw = seq0("v_raw", (B, n, wl.d), "bf16").double().numpy()
    ki_raw = seq0("k_idx_raw", (B, n, wl.d_I), "bf16").double().numpy()
    kc = method.store(method.compress_exact(k_raw, z, wl.m), "bf16")["values"]
    vc = method.store(method.compress_exact(v_raw, z, wl.m), "bf16")["values"]
    ki = method.store(method.compress_exact(ki_raw, z, wl.m), "e4m3")["values"]
    del ki_raw
    import contextlib
    ctx = threadpool_limits(limits=threads, user_api="blas") if threadpool_info else contextlib.nullcontext()
    runs = 0
    with ctx:
        t0 = time.perf_counter()
        while runs < 3 or time.perf_counter() - t0 < CPU_SAMPLE_SECONDS:
            s = method.index_scores(qi, w, ki, wl.t0, wl.m)
            sel = method.select_topk(s, wl.k)
            method.csa_attend(q, kc, vc, sel, k_raw, v_raw, 0, wl.t0, wl.W, wl.m, wl.scale)
            runs += 1
        total = time.perf_counter() - t0
    t = total / runs
    cpu = platform.processor() or ""
    try:
        cpu = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        cpu = next((l.split(":", 1)[1].strip() for l in cpu.splitlines() if l.startswith("Model name")), "")
    except OSError:
        pass
    return {"value": round(1.0 / t, 4), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{runs} repeated decode steps (index + top-k + attention) of sequence 0 of the "
                      f"Pro-like 1M workload, fp64 NumPy, {total:.1f} s in all; compressed caches built untimed",
            "seconds_per_step": round(t, 4), "host_cores": cores, "cpu": cpu,
            "numpy": np.__version__}


# ----------------------------------------------------------------------------- main


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="csa_decode_pro_1m")
    ap.add_argument("--legs", default="hca_decode_1m,csa_prefill_chunk_1m,csa_decode_flash_128k,"
                    "hca_prefill_chunk_1m,csa_decode_pro_1m+state,hca_decode_1m+fp8kv,"
                    "csa_decode_pro_1m+bf16sel",
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (10 times) and exit; used to scale "
                         "the HBM byte counters of a profiler")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 10}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path would "
              "shard by sequence or by compressed-entry range, with no multi-GPU code here).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import compressed_attention_csa_amd as csa
    csa.lib()

    head = time_workload(args.workload, args.seed, args.steps, args.warmup, graph=not args.no_graph)
    legs = {}
    for name in [x for x in args.legs.split(",") if x]:
        steps = 5 if name in ("csa_prefill_chunk_1m", "hca_prefill_chunk_1m") else args.steps
        r = time_workload(name, args.seed, steps, min(args.warmup, 3) if steps < 10 else args.warmup,
                          graph=not args.no_graph)
        s = summarize(r)
        s["roofline"] = roofline(r)
        legs[name] = s
    hs = summarize(head)
    wl = __import__("inputgen").WORKLOADS[args.workload]
    line = {
        "metric": METRIC,
        "value": round(hs["query_tokens_per_s"], 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": wl.B, "context": wl.n, "H": wl.H, "d": wl.d,
                   "H_I": wl.H_I, "d_I": wl.d_I, "m": wl.m, "top_k": wl.k, "window": wl.W,
                   "indexer_keys": wl.idx_key_dtype, "cache_cold_replicas": head["replicas"]},
        "hbm_gbps": hs.get("hbm_gbps"),
        "hbm_frac": hs.get("hbm_frac"),
        "roofline": roofline(head),
        "kernel_ms": hs["kernel_ms"],
        "legs": legs,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.seed)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
