"""Seeded synthetic inputs and the workload registry.

This module is the only code shared by the GPU library's tests/benchmark and
the CPU oracle.  It holds none of the method's arithmetic: it only draws
N(0, 1) tensors (compressor logits N(0, 1) * 0.5), casts them to the storage
type with round-to-nearest-even, and lists the workload shapes.

Seeding: every tensor, sequence and 64K-row chunk gets its own generator,
seeded from a BLAKE2b hash of (master seed, tensor name, sequence, chunk).  A
slice of a tensor can therefore be regenerated without the rest, and chunks can
be drawn in parallel.  Values depend on the device the generator runs on (torch
uses different algorithms on CPU and GPU); a test draws once and hands the same
tensors to both sides.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from concurrent.futures import ThreadPoolExecutor

import torch

CHUNK_ROWS = 65536


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one workload.  Names follow the pages' notation.

    B sequences share the context length n; T query tokens sit at positions
    t0 .. t0+T-1.  H query heads of dim d share one KV head; the indexer has
    H_I heads of dim d_I.  m / m_heavy are the CSA / HCA block sizes, k the
    top-k and W the window.  ``dtype`` is the storage type of q, K, V and the
    indexer query; ``idx_key_dtype`` that of the compressed indexer keys.
    """
    name: str
    B: int
    n: int
    T: int
    t0: int
    H: int
    d: int
    H_I: int = 0
    d_I: int = 0
    m: int = 4
    k: int = 0
    m_heavy: int = 128
    W: int = 128
    dtype: str = "bf16"
    idx_key_dtype: str = "bf16"
    csa: bool = True
    hca: bool = False
    # Chunked prefill: entries [cmp_begin, n // m) are compressed as part of the step.
    cmp_begin: int = 0

    @property
    def N_c(self) -> int:
        return self.n // self.m

    @property
    def N_h(self) -> int:
        return self.n // self.m_heavy

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    # Tiny CSA + HCA prefill in fp32, every position a causal query.
    "tiny_prefill_f32": Workload("tiny_prefill_f32", B=1, n=4096, T=4096, t0=0, H=8, d=64,
                                 H_I=4, d_I=32, m=4, k=64, m_heavy=128, W=128, dtype="f32",
                                 idx_key_dtype="f32", csa=True, hca=True),
    # Flash-like CSA decode at 128K context.
    "csa_decode_flash_128k": Workload("csa_decode_flash_128k", B=8, n=131072, T=1, t0=131071,
                                      H=64, d=128, H_I=8, d_I=64, m=4, k=512, W=128),
    # Pro-like CSA decode at 1M context with fp8-e4m3 indexer keys.
    "csa_decode_pro_1m": Workload("csa_decode_pro_1m", B=4, n=1048576, T=1, t0=1048575,
                                  H=128, d=128, H_I=8, d_I=64, m=4, k=1024, W=128,
                                  idx_key_dtype="e4m3"),
    # HCA dense decode at 1M context.
    "hca_decode_1m": Workload("hca_decode_1m", B=16, n=1048576, T=1, t0=1048575, H=128, d=128,
                              m_heavy=128, W=128, csa=False, hca=True),
    # HCA chunked prefill: the same 8192-token chunk, dense over the heavy entries.
    "hca_prefill_chunk_1m": Workload("hca_prefill_chunk_1m", B=1, n=1048576, T=8192,
                                     t0=1040384, H=64, d=128, m_heavy=128, W=128, csa=False,
                                     hca=True, cmp_begin=1040384 // 128),
    # CSA chunked prefill: 8192 new tokens at the end of a 1M context.
    "csa_prefill_chunk_1m": Workload("csa_prefill_chunk_1m", B=1, n=1048576, T=8192,
                                     t0=1040384, H=64, d=128, H_I=8, d_I=64, m=4, k=1024,
                                     W=128, cmp_begin=1040384 // 4),
}


def seed_of(seed: int, name: str, b: int, chunk: int) -> int:
    h = hashlib.blake2b(f"{seed}/{name}/{b}/{chunk}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return x.to(torch.bfloat16)  # round-to-nearest-even
    raise ValueError(dtype)


def normal(name: str, shape, seed: int, dtype: str = "f32", std: float = 1.0,
           device: str = "cpu", threads: int = 8) -> torch.Tensor:
    """N(0, std^2) tensor of ``shape`` = (B, rows, ...) drawn chunk by chunk.

    A 1-D ``shape`` is one chunk of one sequence.  The float32 draw is cast to
    ``dtype`` ("f32" or "bf16") with round-to-nearest-even.
    """
    shape = tuple(int(s) for s in shape)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    if len(shape) == 1:
        g = torch.Generator(device=device).manual_seed(seed_of(seed, name, 0, 0))
        return _cast(torch.randn(shape, generator=g, device=device) * std, dtype)
    B, rows, rest = shape[0], shape[1], shape[2:]
    out = torch.empty(shape, dtype=tdt, device=device)
    jobs = [(b, c) for b in range(B) for c in range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS)]

    def draw(job):
        b, c = job
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        g = torch.Generator(device=device).manual_seed(seed_of(seed, name, b, c))
        x = torch.randn((r1 - r0,) + rest, generator=g, device=device)
        if std != 1.0:
            x = x * std
        out[b, r0:r1] = _cast(x, dtype)

    if device == "cpu" and threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(draw, jobs))
    else:
        for j in jobs:
            draw(j)
    return out


def make_inputs(wl: Workload, seed: int = 0, device: str = "cpu", threads: int = 8) -> dict:
    """All inputs of a workload.

    Returns q [B,T,H,d], k_raw / v_raw [B,n,d], and for CSA q_idx [B,T,H_I,d_I],
    k_idx_raw [B,n,d_I], w [B,T,H_I] (float32) and z_csa [m]; for HCA z_hca
    [m_heavy].
    """
    dt = wl.dtype
    out = {
        "q": normal("q", (wl.B, wl.T, wl.H, wl.d), seed, dt, device=device, threads=threads),
        "k_raw": normal("k_raw", (wl.B, wl.n, wl.d), seed, dt, device=device, threads=threads),
        "v_raw": normal("v_raw", (wl.B, wl.n, wl.d), seed, dt, device=device, threads=threads),
    }
    if wl.csa:
        out["q_idx"] = normal("q_idx", (wl.B, wl.T, wl.H_I, wl.d_I), seed, dt, device=device,
                              threads=threads)
        out["k_idx_raw"] = normal("k_idx_raw", (wl.B, wl.n, wl.d_I), seed, dt, device=device,
                                  threads=threads)
        out["w"] = normal("w", (wl.B, wl.T, wl.H_I), seed, "f32", device=device, threads=threads)
        out["z_csa"] = normal("z_csa", (wl.m,), seed, "f32", std=0.5, device=device)
    if wl.hca:
        out["z_hca"] = normal("z_hca", (wl.m_heavy,), seed, "f32", std=0.5, device=device)
    return out


def small_workload(**kw) -> Workload:
    """A workload for parity tests, defaults overridden by keyword."""
    base = dict(name="small", B=2, n=1000, T=37, t0=963, H=16, d=128, H_I=8, d_I=64, m=4,
                k=64, m_heavy=128, W=128, dtype="bf16", idx_key_dtype="bf16", csa=True,
                hca=True)
    base.update(kw)
    return Workload(**base)
