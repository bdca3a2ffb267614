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
PEAK_FP8_TFLOPS = 5000.0
COPY_CALIBRATION_BYTES = 256 << 20
METRIC = "decode query-tokens/s + HBM GB/s at 1M ctx; prefill TFLOP/s (frac. of peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- workloads


class DecodeCSA:
    """CSA decode step: index + top-k over all compressed entries, then attention.

    With ``state`` the step first appends the new token's K, V and indexer-key
    rows to the state-cache rings (compressing the block the token completes)
    and the attention reads its window from the K / V rings.  With ``bf16sel``
    the selection is the approximate one (top-k of bf16-rounded scores), with
    ``fp8q`` the fp8 x fp8 indexer (csa_index_topk_fp8: the query rows quantised to
    e4m3); the recall of either against the exact selection is reported beside
    the timing."""

    dominant = "index_topk"
    dominant_kernels = ("index_topk",)

    def __init__(self, wl, seed, replicas, variant=""):
        assert variant in ("", "state", "bf16sel", "fp8q"), variant
        state = variant == "state"
        self.bf16sel = variant == "bf16sel"
        self.fp8q = variant == "fp8q"
        assert not self.fp8q or wl.idx_key_dtype == "e4m3", "the fp8 x fp8 indexer takes e4m3 keys"
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
        if self.fp8q:
            csa.csa_index_topk_fp8(self.q_idx, self.w, c["k_idx"], c["k_scale"], wl.t0, wl.m, wl.k, self.idx)
        else:
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
        """Recall of the approximate (bf16-score or fp8 x fp8) selection against the
        exact one (replica 0)."""
        if not (self.bf16sel or self.fp8q):
            return None
        wl, csa, torch, c = self.wl, self.csa, self.torch, self.reps[0]
        sel = {}
        for approx in (False, True):
            idx = torch.empty_like(self.idx)
            if approx and self.fp8q:
                csa.csa_index_topk_fp8(self.q_idx, self.w, c["k_idx"], c["k_scale"], wl.t0, wl.m, wl.k, idx)
            else:
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
    dominant_kernels = ("hca_attend", "hca_attend_merge")  # the call: attention + split merge

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
    query over all visible entries, attention.

    Variant ``fp8k``: the indexer keys are cached as e4m3 codes with per-entry
    scales (the products stay bf16); ``fp8q``: the same keys with the fp8 x fp8
    indexer (query quantised to e4m3 in the kernel), priced against the fp8 peak."""

    dominant = "index_topk"
    dominant_kernels = ("index_topk",)

    def __init__(self, wl, seed, replicas, variant=""):
        import torch
        assert variant in ("", "fp8k", "fp8q"), variant
        self.variant = variant
        if variant == "fp8q":
            self.mfma_peak = ("fp8", PEAK_FP8_TFLOPS)
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
        self.scales = {}
        if variant:
            self.cmp["k_idx_raw"] = torch.empty((B, N, dI), dtype=torch.uint8, device=dev)
            self.scales["k_idx_raw"] = torch.empty((B, N), dtype=torch.float32, device=dev)
        for name, out in self.cmp.items():  # the prior context, compressed before the step
            csa.csa_compress(self.raw[name], self.z, wl.m, out, out_scale=self.scales.get(name),
                             entry_begin=0, entry_end=wl.cmp_begin)
        self.idx = torch.empty((B, wl.T, wl.k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, wl.T, wl.H, d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def step(self, r):
        wl, csa = self.wl, self.csa
        for name, out in self.cmp.items():
            csa.csa_compress(self.raw[name], self.z, wl.m, out, out_scale=self.scales.get(name),
                             entry_begin=wl.cmp_begin, entry_end=wl.N_c)
        index = csa.csa_index_topk_fp8 if self.variant == "fp8q" else csa.csa_index_topk
        index(self.q_idx, self.w, self.cmp["k_idx_raw"], self.scales.get("k_idx_raw"), wl.t0, wl.m, wl.k,
              self.idx)
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
    dominant_kernels = ("hca_attend",)

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


class TinyPrefill:
    """The tiny fp32 configuration, whole: compress (CSA K, V, indexer keys; HCA K, V),
    index + top-k for all 4096 positions, CSA attention, HCA attention.  A latency-bound
    correctness configuration; its rate is reported against the fp32 vector peak."""

    dominant = "csa_attend"
    dominant_kernels = ("csa_attend", "csa_attend_merge")
    peak = ("fp32", 157.3)

    def __init__(self, wl, seed, replicas):
        import torch
        import compressed_attention_csa_amd as csa
        import inputgen
        self.wl, self.csa = wl, csa
        x = inputgen.make_inputs(wl, seed=seed)
        self.x = {k: v.to("cuda") for k, v in x.items()}
        B, N, Nh, d, dI = wl.B, wl.N_c, wl.N_h, wl.d, wl.d_I
        f = dict(dtype=torch.float32, device="cuda")
        self.kc, self.vc = torch.empty((B, N, d), **f), torch.empty((B, N, d), **f)
        self.ki = torch.empty((B, N, dI), **f)
        self.hk, self.hv = torch.empty((B, Nh, d), **f), torch.empty((B, Nh, d), **f)
        self.idx = torch.empty((B, wl.T, wl.k), dtype=torch.int32, device="cuda")
        self.o = torch.empty((B, wl.T, wl.H, d), **f)
        self.ho = torch.empty_like(self.o)
        torch.cuda.synchronize()

    def step(self, r):
        wl, csa, x = self.wl, self.csa, self.x
        for src, dst in ((x["k_raw"], self.kc), (x["v_raw"], self.vc), (x["k_idx_raw"], self.ki)):
            csa.csa_compress(src, x["z_csa"], wl.m, dst)
        csa.csa_compress(x["k_raw"], x["z_hca"], wl.m_heavy, self.hk)
        csa.csa_compress(x["v_raw"], x["z_hca"], wl.m_heavy, self.hv)
        csa.csa_index_topk(x["q_idx"], x["w"], self.ki, None, wl.t0, wl.m, wl.k, self.idx)
        csa.csa_attend(x["q"], self.kc, self.vc, wl.m, self.idx, x["k_raw"], x["v_raw"], wl.t0, wl.W, wl.scale,
                       self.o)
        csa.hca_attend(x["q"], self.hk, self.hv, wl.m_heavy, x["k_raw"], x["v_raw"], wl.t0, wl.W, wl.scale,
                       self.ho)

    def algorithmic(self):
        wl = self.wl
        ts = range(wl.t0, wl.t0 + wl.T)
        sum_c = sum(min(wl.N_c, (t + 1) // wl.m) for t in ts)
        idx_flops = 2 * wl.B * wl.H_I * wl.d_I * sum_c
        csa_slots = sum(min(wl.k, min(wl.N_c, (t + 1) // wl.m)) + min(wl.W, t + 1) for t in ts)
        hca_slots = sum(min(wl.N_h, (t + 1) // wl.m_heavy) + min(wl.W, t + 1) for t in ts)
        att = 4 * wl.B * wl.H * wl.d
        return {"bytes": None, "flops": idx_flops + att * (csa_slots + hca_slots),
                "dominant_flops": att * csa_slots, "queries": wl.B * wl.T}


class CompressCache:
    """The compressor's own throughput: building the Pro-like decode caches at 1M context
    (K and V to bf16, the indexer keys to e4m3 with per-entry scales; 4 sequences,
    m = 4).  One step = the three csa_compress calls over the whole history."""

    dominant = "compress"
    dominant_kernels = ("compress",)
    calls_per_step = 3

    def __init__(self, wl, seed, replicas):
        import torch
        import compressed_attention_csa_amd as csa
        import inputgen
        self.wl, self.csa = wl, csa
        B, n, d, dI, N = wl.B, wl.n, wl.d, wl.d_I, wl.N_c
        self.z = inputgen.normal("z_csa", (wl.m,), seed, "f32", std=0.5, device="cuda")
        self.raw = {name: inputgen.normal(name, (B, n, dim), seed, "bf16", device="cuda")
                    for name, dim in (("k_raw", d), ("v_raw", d), ("k_idx_raw", dI))}
        self.kc = torch.empty((B, N, d), dtype=torch.bfloat16, device="cuda")
        self.vc = torch.empty_like(self.kc)
        self.ki = torch.empty((B, N, dI), dtype=torch.uint8, device="cuda")
        self.ks = torch.empty((B, N), device="cuda")
        torch.cuda.synchronize()

    def step(self, r):
        wl, csa = self.wl, self.csa
        csa.csa_compress(self.raw["k_raw"], self.z, wl.m, self.kc)
        csa.csa_compress(self.raw["v_raw"], self.z, wl.m, self.vc)
        csa.csa_compress(self.raw["k_idx_raw"], self.z, wl.m, self.ki, self.ks)

    def algorithmic(self):
        wl = self.wl
        read = wl.B * wl.n * (2 * wl.d + wl.d_I) * 2
        write = wl.B * wl.N_c * (2 * wl.d * 2 + wl.d_I + 4)
        return {"bytes": read + write, "flops": 0, "dominant_bytes": read + write, "queries": 0}


class StreamRead:
    """The HBM read ceiling: a plain streaming read (csa_diag_stream_read) of a buffer of
    the given size, cycling replicas so that every read is cache-cold."""

    dominant = "stream_read"
    dominant_kernels = ("stream_read",)

    def __init__(self, nbytes, replicas):
        import torch
        import compressed_attention_csa_amd as csa
        self.csa, self.nbytes = csa, nbytes
        self.bufs = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device="cuda") for i in range(replicas)]
        self.sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def step(self, r):
        self.csa.diag_stream_read(self.bufs[r % len(self.bufs)], self.sink)

    def algorithmic(self):
        return {"bytes": self.nbytes, "flops": 0, "dominant_bytes": self.nbytes, "queries": 0}


class GatherRead:
    """The rate at which workgroups gather scattered K / V rows (csa_diag_gather_read), the
    decode attention's access pattern at the Pro-like shape: four sequences of 262144 rows
    of 256 bytes per tensor, 1152 rows selected per sequence (its 1024 entries and 128
    window rows), gathered either split as the attention's plan does (per sequence 2 head
    groups x 9 splits of 128 rows: 72 workgroups) or whole (per sequence 8 head groups of 16
    heads, each gathering all 1152 rows: 32 workgroups).  Replicas are cycled so that every
    gather is cache-cold; ``bytes`` counts every workgroup's reads (the head groups of one
    split read the same rows)."""

    dominant = "gather_read"
    dominant_kernels = ("gather_read",)

    def __init__(self, split, replicas, seed=0):
        import torch
        import compressed_attention_csa_amd as csa
        self.csa = csa
        rows, N, sel = 4, 262144, 1152
        self.k = [torch.full((rows * N, 128), float(i + 1), dtype=torch.bfloat16, device="cuda")
                  for i in range(replicas)]
        self.v = [torch.full((rows * N, 128), float(i + 2), dtype=torch.bfloat16, device="cuda")
                  for i in range(replicas)]
        g = torch.Generator().manual_seed(seed)
        chosen = [torch.randint(0, N, (sel,), generator=g, dtype=torch.int64) + r * N for r in range(rows)]
        if split:
            self.per, groups = 128, 72
            parts = [chosen[w % rows][((w // rows) % 9) * 128:((w // rows) % 9 + 1) * 128] for w in range(groups)]
        else:
            self.per, groups = sel, 32
            parts = [chosen[w % rows] for w in range(groups)]
        self.idx = torch.cat(parts).to(torch.int32).to("cuda")
        self.sink = torch.zeros(groups, dtype=torch.int32, device="cuda")
        self.groups = groups
        torch.cuda.synchronize()

    def step(self, r):
        self.csa.diag_gather_read(self.k[r % len(self.k)], self.v[r % len(self.v)], self.idx, self.per, self.sink)

    def algorithmic(self):
        b = self.groups * self.per * 512
        return {"bytes": b, "flops": 0, "dominant_bytes": b, "queries": 0}


KINDS = {"csa_decode_pro_1m": DecodeCSA, "csa_decode_flash_128k": DecodeCSA,
         "hca_decode_1m": DecodeHCA, "csa_prefill_chunk_1m": PrefillCSA,
         "hca_prefill_chunk_1m": PrefillHCA, "tiny_prefill_f32": TinyPrefill}
REPLICAS = {"csa_decode_pro_1m": 8, "csa_decode_flash_128k": 16, "hca_decode_1m": 8,
            "csa_prefill_chunk_1m": 1, "hca_prefill_chunk_1m": 1, "tiny_prefill_f32": 1,
            "csa_compress_pro_1m": 1, "hbm_read_71mb": 8, "hbm_read_2gb": 1, "gather_split_72": 8,
            "gather_whole_32": 8}
# Workloads that are not a configuration of the method: the compressor's cache build at the
# Pro-like shape, the HBM read ceiling at the Pro-like step's key bytes and at 2 GB, and the
# decode attention's row gather, split and whole.
EXTRA = {"csa_compress_pro_1m": lambda seed, R: CompressCache(__import__("inputgen").WORKLOADS["csa_decode_pro_1m"],
                                                              seed, R),
         "hbm_read_71mb": lambda seed, R: StreamRead(71307392, R),
         "hbm_read_2gb": lambda seed, R: StreamRead(2 << 30, R),
         "gather_split_72": lambda seed, R: GatherRead(True, R, seed),
         "gather_whole_32": lambda seed, R: GatherRead(False, R, seed)}


# ----------------------------------------------------------------------------- timing


PROFILE_MARKER = False  # --profile-marker: a spin kernel of torch's marks where the timed launches start


def time_workload(name, seed, steps, warmup, graph=True):
    import torch
    import compressed_attention_csa_amd as csa
    import inputgen
    base, _, variant = name.partition("+")  # "+state": the decode step also maintains the state cache
    R = REPLICAS[base]
    log(f"[bench] {name}: setting up ({R} replica(s))")
    t = time.time()
    if base in EXTRA:
        w = EXTRA[base](seed, R)
    else:
        wl = inputgen.WORKLOADS[base]
        w = KINDS[base](wl, seed, R, **({"variant": variant} if variant else {}))
    log(f"[bench] {name}: setup {time.time() - t:.1f}s; warmup {warmup}")
    for i in range(max(warmup, R)):
        w.step(i)
    torch.cuda.synchronize()
    # Per-kernel durations, with the library's HIP events around each launch (eager).
    csa.profile_enable(True)
    nprof = min(max(2 * R, 8), steps) if R > 1 else min(3, steps)
    for i in range(nprof):
        w.step(i)
    torch.cuda.synchronize()
    csa.profile_enable(False)
    prof = csa.profile_report()
    # Headline timing: a graph of R steps (one per replica), replayed at least
    # ceil(steps / R) times; each replay is timed on its own.
    reps = max(1, -(-steps // R))
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
    if PROFILE_MARKER:
        torch.cuda._sleep(1000)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record()
        if g is not None:
            g.replay()
        else:
            for i in range(R):
                w.step(i)
        e1.record()
    if PROFILE_MARKER:
        torch.cuda._sleep(1000)  # end of the timed launches
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) / R for e0, e1 in ev)
    ms = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (per_step[len(per_step) // 2 - 1] +
                                                                        per_step[len(per_step) // 2])
    alg = w.algorithmic()
    res = {"workload": name, "ms_per_step": ms, "ms_min": per_step[0], "ms_max": per_step[-1],
           "steps": reps * R, "replicas": R, "kernels": prof, "alg": alg, "dominant": w.dominant,
           "dominant_kernels": list(w.dominant_kernels),
           "peak": getattr(w, "peak", None), "mfma_peak": getattr(w, "mfma_peak", None)}
    # The dominant call's time per step: its kernels' event-timed durations, summed.
    calls = prof.get(w.dominant_kernels[0], {}).get("launches", 0) / getattr(w, "calls_per_step", 1)
    if calls:
        res["dominant_ms"] = sum(prof[k]["total_ms"] for k in w.dominant_kernels if k in prof) / calls
        res["dominant_parts_ms"] = {k: round(prof[k]["total_ms"] / calls, 6) for k in w.dominant_kernels if k in prof}
    q = w.quality() if hasattr(w, "quality") else None
    if q:
        res["quality"] = q
    del w, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def summarize(res):
    alg, ms = res["alg"], res["ms_per_step"]
    out = {"ms_per_step": round(ms, 6), "ms_per_step_min": round(res["ms_min"], 6),
           "ms_per_step_max": round(res["ms_max"], 6), "steps": res["steps"],
           "cache_cold_replicas": res["replicas"]}
    if alg.get("queries"):
        out["query_tokens_per_s"] = alg["queries"] / (ms * 1e-3)
    if alg.get("bytes"):
        gbps = alg["bytes"] / (ms * 1e-3) / 1e9
        out.update({"hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "alg_bytes": alg["bytes"]})
    if alg.get("flops"):
        tf = alg["flops"] / (ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if res.get("peak") is None else res["peak"][1]
        out.update({"tflops": round(tf, 3), ("mfma_frac" if res.get("peak") is None else "fp32_frac"):
                    round(tf / peak, 4), "alg_flops": alg["flops"]})
    out["kernel_ms"] = {k: round(v["total_ms"] / v["launches"], 6) for k, v in res["kernels"].items()}
    out.update(res.get("quality") or {})
    return out


def roofline(res, ceiling_gbps=None):
    alg = res["alg"]
    dom_ms = res.get("dominant_ms")
    if dom_ms is None:
        return None
    # Counter bytes of every kernel of the dominant call (e.g. attention and its split merge).
    parts = [load_traffic(f"{k}@{res['workload']}") for k in res.get("dominant_kernels", [res["dominant"]])]
    traffic = sum(parts) if parts and all(x is not None for x in parts) else None
    common = {"traffic": traffic, "kernel": res["dominant"], "kernel_ms": round(dom_ms, 6),
              "kernel_parts_ms": res.get("dominant_parts_ms")}
    if "dominant_bytes" in alg:
        achieved = alg["dominant_bytes"] / (dom_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBPS, 4), **common, "alg_bytes_per_launch": alg["dominant_bytes"]}
        if ceiling_gbps:
            r["measured_read_ceiling_gbps"] = round(ceiling_gbps, 1)
            r["frac_of_measured_ceiling"] = round(achieved / ceiling_gbps, 4)
        return r
    achieved = alg["dominant_flops"] / (dom_ms * 1e-3) / 1e12
    if res.get("peak") is not None:
        return {"bound": "alu", "achieved": round(achieved, 3), "peak": res["peak"][1], "unit": "TFLOP/s",
                "frac": round(achieved / res["peak"][1], 4), **common,
                "alg_flops_per_launch": alg["dominant_flops"]}
    dt, peak = res.get("mfma_peak") or ("bf16", PEAK_BF16_TFLOPS)
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "peak_dtype": dt, **common,
            "alg_flops_per_launch": alg["dominant_flops"]}


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


# ----------------------------------------------------------------------------- rocprofv3 summaries
#
# One workload per profiler process: a kernel trace run, a FETCH_SIZE run, a WRITE_SIZE run and,
# optionally, one run of SQ counters, each of `bench.py --no-graph --profile-marker --workload W
# --legs ""`.  The program launches the same kernels in the same order in every run, so the
# k-th dispatch of a (kernel, grid, workgroup) in one run is the k-th in the others; only the
# dispatches after the marker (the timed steps) are summarised.


def _read_csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def _grid(row):
    """Total work-items (the kernel trace lists x, y, z; the counter runs their product)."""
    if row.get("Grid_Size"):
        return int(row["Grid_Size"])
    return int(row.get("Grid_Size_X") or 0) * int(row.get("Grid_Size_Y") or 1) * int(row.get("Grid_Size_Z") or 1)


def _wg(row):
    if row.get("Workgroup_Size"):
        return int(row["Workgroup_Size"])
    return (int(row.get("Workgroup_Size_X") or 0) * int(row.get("Workgroup_Size_Y") or 1) *
            int(row.get("Workgroup_Size_Z") or 1))


def _after_marker(rows, key="Dispatch_Id"):
    """The dispatches between the two torch spin kernels that bracket the timed steps (or
    after the only one), in dispatch order, keyed by their ordinal within (kernel, grid,
    workgroup)."""
    rows = sorted(rows, key=lambda r: int(r[key]))
    marks = [i for i, r in enumerate(rows) if "sleep" in r["Kernel_Name"] or "spin" in r["Kernel_Name"]]
    if not marks:
        raise SystemExit("no profiling marker in the dispatch list (run bench.py with --profile-marker)")
    lo, hi = (marks[-2], marks[-1]) if len(marks) >= 2 else (marks[-1], len(rows))
    out, seen = {}, {}
    for r in rows[lo + 1:hi]:
        k = (r["Kernel_Name"], _grid(r), _wg(r))
        n = seen.get(k, 0)
        seen[k] = n + 1
        out[(k, n)] = r
    return out


def _counter(directory, name):
    """Per dispatch (after the marker): the value of counter `name`, summed over its rows."""
    rows = [r for r in _read_csv_rows(directory, "counter_collection.csv") if r["Counter_Name"] == name]
    by_id = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        if d not in by_id:
            by_id[d] = dict(r, Counter_Value=0.0)
        by_id[d]["Counter_Value"] += float(r["Counter_Value"])
    return {k: v["Counter_Value"] for k, v in _after_marker(list(by_id.values())).items()}


def _role(kernel, workload):
    kernel = _short(kernel)
    att = "hca_attend" if workload.startswith("hca") else "csa_attend"
    if kernel.startswith(("idx_topk_kernel", "idx_prefill_kernel")):
        return "index_topk"
    if kernel.startswith("attend_merge_kernel"):
        return att + "_merge"
    if kernel.startswith("attend_bf16_kernel"):
        return "hca_attend" if ", true," in kernel.split("<", 1)[-1][:40] else "csa_attend"
    if kernel.startswith("hca_multi_kernel"):
        return "hca_attend"
    if kernel.startswith("attend_f32_kernel"):
        return "attend (fp32)"
    if kernel.startswith("compress_kernel"):
        # compress_kernel<input type, output kind, APPEND, SPLIT>
        args = [x.strip() for x in kernel.split("<", 1)[-1].rstrip(">").split(",")]
        return "append" if len(args) > 2 and args[2] == "true" else "compress"
    if kernel.startswith("stream_read_kernel"):
        return "stream_read"
    if kernel.startswith("gather_read_kernel"):
        return "gather_read"
    return None


def _short(kernel):
    k = kernel[5:] if kernel.startswith("void ") else kernel
    k = k.replace("(anonymous namespace)::", "").replace("csa::", "")
    return k.split("(")[0].strip()


def profile_summary(root, calib, workload, traffic_out=None, command_note="", timed_steps=0):
    trace = _after_marker(_read_csv_rows(os.path.join(root, "trace"), "kernel_trace.csv"))
    fetch = _counter(os.path.join(root, "fetch"), "FETCH_SIZE")
    write = _counter(os.path.join(root, "write"), "WRITE_SIZE")
    scale = {"FETCH_SIZE": 1.0, "WRITE_SIZE": 1.0}
    if calib:
        for cname, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            rows = [r for r in _read_csv_rows(os.path.join(calib, sub), "counter_collection.csv")
                    if r["Counter_Name"] == cname and "copy" in r["Kernel_Name"].lower()]
            per = {}
            for r in rows:
                per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
            vals = sorted(per.values())
            if vals:
                kib = vals[len(vals) // 2]
                scale[cname] = COPY_CALIBRATION_BYTES / (kib * 1024.0)
    sq_names = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAVE_CYCLES",
                "SQ_WAIT_ANY", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    sq = {}
    if os.path.isdir(os.path.join(root, "sq")):
        for n in sq_names:
            try:
                sq[n] = _counter(os.path.join(root, "sq"), n)
            except SystemExit:
                pass
    # Per (kernel, grid, workgroup): durations from the trace, bytes per dispatch from the
    # counter runs, paired dispatch by dispatch.
    groups = {}
    rejected = 0
    for (k, n), r in trace.items():
        g = groups.setdefault(k, {"us": [], "rd": [], "wr": [], "sq": {x: [] for x in sq}})
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        rd = fetch.get((k, n))
        wr = write.get((k, n))
        if rd is not None and wr is not None:
            rd_b = rd * 1024.0 * scale["FETCH_SIZE"]
            wr_b = wr * 1024.0 * scale["WRITE_SIZE"]
            if (rd_b + wr_b) / (us * 1e-6) > PEAK_HBM_GBPS * 1e9:
                rejected += 1  # more bytes than HBM can move in that time: not the same launch
            else:
                g["rd"].append(rd_b)
                g["wr"].append(wr_b)
        g["us"].append(us)
        for x in sq:
            v = sq[x].get((k, n))
            if v is not None:
                g["sq"][x].append(v)

    def med(v):
        v = sorted(v)
        return v[len(v) // 2] if v else None

    lines = [f"# Kernels of `{workload}`: durations, HBM traffic" + (" and SQ counters" if sq else ""), ""]
    lines += ["Commands (repository root on the MI355X box; each GPU step under `timeout`):", ""]
    lines += ["    " + c for c in command_note.split(" ;; ") if c]
    lines += ["", f"Kernel sources digest (bench.kernel_source_digest): `{kernel_source_digest()}`", "",
              f"Counter scale factors from the plain device copy: FETCH_SIZE x {scale['FETCH_SIZE']:.4f}, "
              f"WRITE_SIZE x {scale['WRITE_SIZE']:.4f}.", "",
              "Only dispatches after the profiling marker (the timed steps) are listed.  Durations are "
              "from the kernel trace (eager launches); bytes are medians per dispatch of the counter "
              "runs, paired with the trace dispatch by dispatch (the k-th launch of the same kernel, "
              f"grid and workgroup).  Pairs implying more than 8 TB/s are dropped: {rejected} dropped.", ""]
    hdr = "| kernel | role | grid | wg | launches | avg us | min us | max us | HBM read MB | HBM write MB | GB/s |"
    lines += [hdr, "|" + "---|" * 11]
    role_tot = {}
    n_steps = timed_steps or (min(len(g["us"]) for g in groups.values()) if groups else 1)
    for k in sorted(groups, key=lambda k: -sum(groups[k]["us"])):
        g = groups[k]
        avg = sum(g["us"]) / len(g["us"])
        rd, wr = med(g["rd"]), med(g["wr"])
        role = _role(k[0], workload) or "-"
        gbps = "-" if rd is None else f"{(rd + wr) / (avg * 1e-6) / 1e9:.1f}"
        lines.append(f"| {_short(k[0])} | {role} | {k[1]} | {k[2]} | {len(g['us'])} | {avg:.2f} | "
                     f"{min(g['us']):.2f} | {max(g['us']):.2f} | "
                     f"{'-' if rd is None else f'{rd / 1e6:.2f}'} | {'-' if wr is None else f'{wr / 1e6:.3f}'} | "
                     f"{gbps} |")
        t = role_tot.setdefault(role, {"us": 0.0, "rd": 0.0, "wr": 0.0, "n": 0, "bytes_ok": True})
        per = len(g["us"]) / n_steps  # launches of this kernel per step
        t["us"] += per * avg
        t["n"] += len(g["us"])
        if rd is None:
            t["bytes_ok"] = False
        else:
            t["rd"] += per * rd
            t["wr"] += per * wr
    extra = {}
    if os.path.isdir(os.path.join(root, "sq2")):
        rows = _read_csv_rows(os.path.join(root, "sq2"), "counter_collection.csv")
        for n in sorted({r["Counter_Name"] for r in rows}):
            extra[n] = _counter(os.path.join(root, "sq2"), n)
    if extra:
        names = list(extra)
        lines += ["", "Further SQ counters (medians per dispatch; a separate run):", "",
                  "| kernel | " + " | ".join(names) + " |", "|" + "---|" * (len(names) + 1)]
        for k in sorted(groups, key=lambda k: -sum(groups[k]["us"])):
            vals = [med([extra[n][(k, i)] for i in range(len(groups[k]["us"])) if (k, i) in extra[n]])
                    for n in names]
            if any(v is None for v in vals):
                continue
            lines.append(f"| {_short(k[0])} | " + " | ".join(f"{v:.0f}" for v in vals) + " |")
    if sq:
        lines += ["", "SQ counters (medians per dispatch).  GRBM_GUI_ACTIVE counts busy cycles per XCD, summed "
                  "over the 8 XCDs, so a kernel's cycles are C = GRBM_GUI_ACTIVE / 8 (the table's `cycles`, to be "
                  "compared with the traced duration x clock).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (C x 1024 "
                  "SIMDs); VALU busy = 4 x SQ_ACTIVE_INST_VALU / (C x 1024 SIMDs); co-issue = "
                  "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES:",
                  ""]
        lines += ["| kernel | " + " | ".join(sq_names) + " | cycles | MFMA busy | VALU busy | co-issue | waiting |",
                  "|" + "---|" * (len(sq_names) + 6)]
        for k in sorted(groups, key=lambda k: -sum(groups[k]["us"])):
            v = {x: med(groups[k]["sq"][x]) for x in sq}
            if any(x is None for x in v.values()):
                continue
            cyc = (v.get("GRBM_GUI_ACTIVE") or 0) / 8
            mf = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024) if cyc else float("nan")
            va = 4 * v["SQ_ACTIVE_INST_VALU"] / (cyc * 1024) if cyc else float("nan")
            co = v["SQ_VALU_MFMA_COEXEC_CYCLES"] / v["SQ_VALU_MFMA_BUSY_CYCLES"] if v["SQ_VALU_MFMA_BUSY_CYCLES"] else 0
            wt = v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"] if v["SQ_WAVE_CYCLES"] else 0
            lines.append(f"| {_short(k[0])} | " + " | ".join(f"{v[x]:.0f}" for x in sq_names) +
                         f" | {cyc:.0f} | {mf:.1%} | {va:.1%} | {co:.1%} | {wt:.1%} |")
    lines += ["", f"Per timed step ({n_steps} steps) of each role, all its kernels summed, and per call "
              "(the step's share divided by the role's launches per step):", ""]
    traffic = {}
    for role, t in sorted(role_tot.items()):
        if role == "-":
            continue
        calls = t["n"] / n_steps
        b = f"read {t['rd'] / 1e6:.2f} MB + write {t['wr'] / 1e6:.3f} MB" if t["bytes_ok"] else "bytes not paired"
        lines.append(f"- `{role}`: {t['us']:.2f} us per step, {b} per step; {calls:g} launch(es) per step")
        if t["bytes_ok"]:
            traffic[f"{role}@{workload}"] = {"hbm_bytes_per_launch": int((t["rd"] + t["wr"]) / calls),
                                             "hbm_bytes_per_step": int(t["rd"] + t["wr"]),
                                             "read_bytes_per_step": int(t["rd"]), "write_bytes_per_step": int(t["wr"]),
                                             "trace_us_per_step": round(t["us"], 3),
                                             "source_digest": kernel_source_digest(),
                                             "scale": {x: round(y, 4) for x, y in scale.items()}}
    if traffic_out:
        try:
            with open(traffic_out) as f:
                data = json.load(f)
        except (OSError, ValueError):
            data = {}
        data.update(traffic)
        with open(traffic_out, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
    return "\n".join(lines) + "\n"


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
            s, vis = method.index_scores(qi, w, ki, wl.t0, wl.m)
            sel = method.select_topk(s, vis, wl.k)
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
    ap.add_argument("--legs", default="hbm_read_71mb,hbm_read_2gb,gather_split_72,gather_whole_32,hca_decode_1m,csa_prefill_chunk_1m,"
                    "csa_decode_flash_128k,hca_prefill_chunk_1m,tiny_prefill_f32,csa_compress_pro_1m,"
                    "csa_decode_pro_1m+state,hca_decode_1m+fp8kv,csa_decode_pro_1m+bf16sel,csa_prefill_chunk_1m+fp8k,"
                    "csa_prefill_chunk_1m+fp8q,csa_decode_pro_1m+fp8q",
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (10 times) and exit; used to scale "
                         "the HBM byte counters of a profiler")
    ap.add_argument("--profile-marker", action="store_true",
                    help="launch one torch spin kernel right before the timed steps of each workload, so "
                         "that a profiler's dispatch list can be cut at that point")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="no GPU: summarise rocprofv3 CSV runs of one workload under DIR (trace/, fetch/, "
                         "write/, optionally sq/) with --calibration; prints markdown")
    ap.add_argument("--calibration", metavar="DIR", help="rocprofv3 runs of --copy-calibration (fetch/, write/)")
    ap.add_argument("--traffic-out", metavar="JSON", help="with --profile-summary: update this traffic file")
    ap.add_argument("--command-note", default="", help="with --profile-summary: the commands, for the summary")
    ap.add_argument("--timed-steps", type=int, default=0,
                    help="with --profile-summary: the timed steps of the profiled run (the --steps it ran with)")
    args = ap.parse_args()
    if args.profile_summary:
        print(profile_summary(args.profile_summary, args.calibration, args.workload, args.traffic_out,
                              args.command_note, args.timed_steps))
        return
    global PROFILE_MARKER
    PROFILE_MARKER = args.profile_marker
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        assert n == COPY_CALIBRATION_BYTES, "the summaries scale counters by a 256 MiB copy"
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
    legs, ceiling = {}, None
    for name in [x for x in args.legs.split(",") if x]:
        slow = name.partition("+")[0] in ("csa_prefill_chunk_1m", "hca_prefill_chunk_1m", "csa_compress_pro_1m",
                                          "hbm_read_2gb", "tiny_prefill_f32")
        steps = 5 if slow else args.steps
        r = time_workload(name, args.seed, steps, min(args.warmup, 3) if steps < 10 else args.warmup,
                          graph=not args.no_graph)
        s = summarize(r)
        if name == "hbm_read_71mb" and r.get("dominant_ms"):
            ceiling = r["alg"]["bytes"] / (r["dominant_ms"] * 1e-3) / 1e9
        s["roofline"] = roofline(r, ceiling)
        legs[name] = s
    hs = summarize(head)
    base = args.workload.partition("+")[0]
    if base not in __import__("inputgen").WORKLOADS or "query_tokens_per_s" not in hs:
        # Not a decode configuration (a profiling run of one workload): its summary only.
        print(json.dumps({"workload": args.workload, **hs, "roofline": roofline(head, ceiling)}), flush=True)
        return
    wl = __import__("inputgen").WORKLOADS[base]
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
        "ms_per_step_min": hs["ms_per_step_min"],
        "ms_per_step_max": hs["ms_per_step_max"],
        "hbm_gbps": hs.get("hbm_gbps"),
        "hbm_frac": hs.get("hbm_frac"),
        "roofline": roofline(head, ceiling),
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
