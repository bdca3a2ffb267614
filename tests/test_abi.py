"""The C ABI on the host: every declared symbol is exported and every bad argument is
rejected with its documented status before any HIP call (no GPU needed).

Pointers here are host addresses that are never dereferenced: validation runs
entirely on the host and returns before anything is enqueued.
"""
import ctypes
import os
import re
import threading

import numpy as np
import pytest

import compressed_attention_csa_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_UNSUP = 0, 1, 2, 3, 4, 5, 6
F32, BF16, FP8 = csa.CSA_F32, csa.CSA_BF16, csa.CSA_FP8_E4M3

_buf = np.zeros(1 << 16, dtype=np.uint8)
P = ctypes.c_void_p(_buf.ctypes.data + (-_buf.ctypes.data) % 256)  # 256-byte aligned
MIS = ctypes.c_void_p(P.value + 4)  # misaligned


@pytest.fixture(scope="module")
def L():
    return csa.lib()


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"^(?:csa_status_t|size_t|int|const char\*)\s+(\w+)\(", text, re.M)


def test_every_declared_symbol_is_exported_and_bound(L):
    names = declared_functions()
    assert len(names) == 18
    for n in names:
        assert hasattr(L, n), n
        assert n in csa.SIGNATURES, n
    assert L.csa_abi_version() == 7
    for s, name in enumerate(csa.STATUS):
        assert L.csa_status_string(s).decode() == name


def compress(L, x=P, x_dt=BF16, B=1, n_raw=64, d=128, raw_base=0, logits=P, m=4, eb=0, ee=16,
             N=16, out=P, out_dt=BF16, scale=None, overlap=0):
    return L.csa_compress(x, x_dt, B, n_raw, d, raw_base, logits, m, overlap, eb, ee, N, out, out_dt, scale,
                          None)


def test_compress_validation(L):
    assert compress(L, x=None) == E_NULL
    assert compress(L, logits=None) == E_NULL
    assert compress(L, x_dt=FP8) == E_DTYPE
    assert compress(L, out_dt=7) == E_DTYPE
    assert compress(L, out_dt=FP8) == E_NULL          # fp8 needs a scale buffer
    assert compress(L, scale=P) == E_DTYPE            # scale only with fp8
    assert compress(L, m=0) == E_SHAPE
    assert compress(L, m=129) == E_SHAPE
    assert compress(L, d=12) == E_SHAPE
    assert compress(L, d=8, out_dt=FP8, scale=P) == E_SHAPE  # fp8 rows need d a power of 2 >= 16
    assert compress(L, d=48, out_dt=FP8, scale=P) == E_SHAPE
    assert compress(L, ee=17) == E_SHAPE              # entry_end > N_alloc
    assert compress(L, eb=5, ee=4) == E_SHAPE
    assert compress(L, n_raw=63) == E_SHAPE           # last block not inside x
    assert compress(L, raw_base=4) == E_SHAPE         # first block before raw_base
    assert compress(L, overlap=-1) == E_SHAPE
    assert compress(L, m=100, overlap=29) == E_SHAPE  # m + overlap <= 128 logits
    assert compress(L, eb=2, raw_base=8, n_raw=56, overlap=1) == E_SHAPE  # overlap row 7 before raw_base
    assert compress(L, B=0) == E_SHAPE
    assert compress(L, x=MIS) == E_ALIGN
    assert compress(L, out=MIS) == E_ALIGN
    compress(L, x=None)
    assert L.csa_last_error() == b"x is NULL"


def append(L, x=P, dt=BF16, B=2, T_new=1, d=128, t0=100, ring=P, R=132, logits=P, m=4, N=64, out=P,
           out_dt=BF16, scale=None, overlap=0):
    return L.csa_append(x, dt, B, T_new, d, t0, ring, R, logits, m, overlap, N, out, out_dt, scale, None)


def test_append_validation(L):
    """Every check fires before any HIP call (no GPU is touched here)."""
    assert append(L, x=None) == E_NULL
    assert append(L, ring=None) == E_NULL
    assert append(L, logits=None) == E_NULL
    assert append(L, out=None) == E_NULL
    assert append(L, dt=FP8) == E_DTYPE
    assert append(L, out_dt=FP8) == E_NULL            # fp8 needs a scale buffer
    assert append(L, scale=P) == E_DTYPE
    assert append(L, B=0) == E_SHAPE
    assert append(L, T_new=-1) == E_SHAPE
    assert append(L, T_new=4097, R=5000) == E_SHAPE
    assert append(L, d=12) == E_SHAPE
    assert append(L, m=0) == E_SHAPE
    assert append(L, t0=-1) == E_SHAPE
    assert append(L, R=0) == E_SHAPE
    assert append(L, m=128, R=127) == E_SHAPE         # a block must fit in the ring
    assert append(L, m=4, T_new=10, R=12) == E_SHAPE  # R >= m + T_new - 1
    assert append(L, m=4, T_new=1, R=5, overlap=2) == E_SHAPE  # R >= m + overlap + T_new - 1
    assert append(L, ring=MIS) == E_ALIGN
    assert append(L, x=MIS) == E_ALIGN
    assert append(L, T_new=0) == OK                   # nothing to do, nothing enqueued
    append(L, R=2)
    assert b"R=2" in L.csa_last_error()


def index(L, q=P, q_dt=BF16, w=P, k=P, k_dt=BF16, ks=None, B=4, T=1, H_I=8, d_I=64, N=1024, t0=4095,
          m=4, top_k=64, out=P, score=None, ws=P, ws_bytes=None, fn="csa_index_topk"):
    if ws_bytes is None:
        ws_bytes = L.csa_index_topk_workspace(B, T, H_I, d_I, N, top_k, k_dt)
    return getattr(L, fn)(q, q_dt, w, k, k_dt, ks, B, T, H_I, d_I, N, t0, m, top_k, out, score, ws,
                          ws_bytes, None)


def test_approximate_selector_validates_like_the_exact_one(L):
    for kw in (dict(q=None), dict(out=None), dict(q_dt=F32), dict(k_dt=FP8), dict(ks=P),
               dict(top_k=0), dict(top_k=2049), dict(H_I=17), dict(d_I=48), dict(q=MIS)):
        assert index(L, fn="csa_index_topk_bf16", **kw) == index(L, **kw) != OK, kw



def index_fp8(L, q=P, w=P, k=P, ks=P, B=4, T=1, H_I=8, d_I=64, N=1024, t0=4095, m=4, top_k=64, out=P,
              score=None, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.csa_index_topk_workspace(B, T, H_I, d_I, N, top_k, FP8)
    return L.csa_index_topk_fp8(q, w, k, ks, B, T, H_I, d_I, N, t0, m, top_k, out, score, ws, ws_bytes, None)


def test_fp8_indexer_validates_like_the_exact_one(L):
    """csa_index_topk_fp8 is csa_index_topk on (bf16, e4m3) with the query quantised:
    it rejects what the exact indexer rejects for those dtypes."""
    assert index_fp8(L, ks=None) == E_NULL          # e4m3 keys need k_scale
    for kw in (dict(q=None), dict(out=None), dict(top_k=0), dict(top_k=2049), dict(H_I=17), dict(d_I=48),
               dict(q=MIS), dict(w=MIS), dict(ks=MIS), dict(m=0), dict(t0=-1), dict(T=-1)):
        ref = dict(k_dt=FP8, ks=P)
        ref.update(kw)
        assert index_fp8(L, **kw) == index(L, **ref) != OK, kw
    need = L.csa_index_topk_workspace(4, 1, 8, 64, 262144, 1024, FP8)
    assert index_fp8(L, N=262144, top_k=1024, ws_bytes=need - 1) == E_WS


def test_index_validation(L):
    assert index(L, q=None) == E_NULL
    assert index(L, out=None) == E_NULL
    assert index(L, q_dt=F32) == E_DTYPE              # f32 query with bf16 keys
    assert index(L, k_dt=FP8) == E_NULL               # e4m3 keys need k_scale
    assert index(L, ks=P) == E_DTYPE
    assert index(L, q_dt=FP8, k_dt=FP8, ks=P) == E_DTYPE
    assert index(L, top_k=0) == E_SHAPE
    assert index(L, top_k=2049) == E_SHAPE
    assert index(L, H_I=17) == E_SHAPE
    assert index(L, d_I=48) == E_SHAPE
    assert index(L, N=(1 << 22) + 1, ws_bytes=1 << 40) == E_SHAPE
    assert index(L, m=0) == E_SHAPE
    assert index(L, t0=-1) == E_SHAPE
    assert index(L, T=-1) == E_SHAPE
    need = L.csa_index_topk_workspace(4, 1, 8, 64, 262144, 1024, BF16)
    assert need > 0
    assert index(L, N=262144, top_k=1024, ws_bytes=need - 1) == E_WS
    assert index(L, N=262144, top_k=1024, ws=None) == E_WS
    assert index(L, q=MIS) == E_ALIGN
    assert index(L, w=MIS) == E_ALIGN


def attend(L, hca=False, q=P, dt=BF16, kc=P, vc=P, kv_dt=None, ks=None, vs=None, N=256, m=4, idx=P,
           top_k=64, kr=P, vr=P, raw_base=0, n_raw=1024, B=2, T=1, H=64, d=128, t0=1023, W=128, out=P,
           out_dt=F32, lse=None, ws=P, ws_bytes=None):
    kv_dt = dt if kv_dt is None else kv_dt
    if hca:
        if ws_bytes is None:
            ws_bytes = L.hca_attend_workspace(B, T, H, d, N, m, W)
        return L.hca_attend(q, dt, kc, vc, kv_dt, ks, vs, N, m, kr, vr, raw_base, n_raw, B, T, H, d, t0,
                            W, 0.1, out, out_dt, lse, ws, ws_bytes, None)
    if ws_bytes is None:
        ws_bytes = L.csa_attend_workspace(B, T, H, d, top_k, W)
    return L.csa_attend(q, dt, kc, vc, kv_dt, ks, vs, N, m, idx, top_k, kr, vr, raw_base, n_raw, B, T, H,
                        d, t0, W, 0.1, out, out_dt, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("hca", [False, True])
def test_attend_validation(L, hca):
    # fp8 compressed caches: bf16 queries only, both scales, aligned
    assert attend(L, hca, kv_dt=FP8) == E_NULL
    assert attend(L, hca, kv_dt=FP8, ks=P) == E_NULL
    assert attend(L, hca, kv_dt=FP8, ks=P, vs=MIS) == E_ALIGN
    assert attend(L, hca, dt=F32, kv_dt=FP8, ks=P, vs=P, H=8) == E_DTYPE
    assert attend(L, hca, kv_dt=F32) == E_DTYPE
    assert attend(L, hca, ks=P) == E_DTYPE            # scales only with fp8 caches
    assert attend(L, hca, q=None) == E_NULL
    assert attend(L, hca, vr=None) == E_NULL
    assert attend(L, hca, dt=FP8) == E_DTYPE
    assert attend(L, hca, out_dt=FP8) == E_DTYPE
    assert attend(L, hca, H=24) == E_UNSUP            # bf16 needs H % 16 == 0
    assert attend(L, hca, H=144) == E_UNSUP
    assert attend(L, hca, d=96) == E_UNSUP
    assert attend(L, hca, dt=F32, H=33) == E_UNSUP
    assert attend(L, hca, W=1025) == E_SHAPE
    assert attend(L, hca, W=-1) == E_SHAPE
    assert attend(L, hca, n_raw=1023) == E_SHAPE      # newest window row missing
    assert attend(L, hca, raw_base=900) == E_SHAPE    # oldest window row missing
    assert attend(L, hca, m=0) == E_SHAPE
    assert attend(L, hca, B=0) == E_SHAPE
    assert attend(L, hca, out=MIS) == E_ALIGN
    assert attend(L, hca, lse=MIS) == E_ALIGN
    if not hca:
        assert attend(L, hca, idx=None) == E_NULL
        assert attend(L, hca, top_k=2049) == E_SHAPE
        assert attend(L, hca, idx=MIS) == E_ALIGN
    # long decode rows are split, so their partials need workspace
    need = (L.hca_attend_workspace(2, 1, 64, 128, 8192, 4, 128) if hca
            else L.csa_attend_workspace(2, 1, 64, 128, 1024, 128))
    assert need > 0
    big = dict(N=8192, m=128, n_raw=1 << 20, t0=(1 << 20) - 1) if hca else dict(top_k=1024)
    assert attend(L, hca, ws_bytes=need - 1, **big) == E_WS
    assert attend(L, hca, ws=None, **big) == E_WS


def test_noalloc_attend_rejects_before_any_launch(L):
    """csa_attend_noalloc checks its arguments and its scratch limit before any
    HIP call (this runs without a GPU): a shape whose workspace exceeds the
    library's scratch, and the ordinary argument errors of csa_attend."""
    limit = (16 << 20)
    def call(B=4, T=1, H=128, d=128, k=1024, W=128, q=P, out=P, idx=P, dt=BF16):
        t0 = 4 * 300000 - 1
        return L.csa_attend_noalloc(q, dt, P, P, dt, None, None, 300000, 4, idx, k, P, P, t0 - W + 1, W + T, B, T,
                                    H, d, t0, W, 0.1, out, F32, None, None)
    big = dict(B=200, T=1)  # 200 decode rows: partials far beyond the scratch
    assert L.csa_attend_workspace(200, 1, 128, 128, 1024, 128) > limit
    assert call(**big) == E_WS
    assert b"scratch" in L.csa_last_error()
    assert L.csa_attend_workspace(4, 1, 128, 128, 1024, 128) <= limit
    assert call(q=None) == E_NULL
    assert call(q=MIS) == E_ALIGN
    assert call(d=96) == E_UNSUP
    assert call(k=4096) == E_SHAPE


def test_null_pointers_are_allowed_for_empty_arrays(L):
    """Arrays with no elements may be NULL; such calls succeed and enqueue nothing
    (no GPU is touched here)."""
    assert attend(L, False, q=None, out=None, idx=None, T=0) == OK
    assert attend(L, True, q=None, out=None, T=0) == OK
    assert index(L, q=None, out=None, T=0) == OK
    assert compress(L, x=None, n_raw=0, eb=0, ee=0) == OK
    assert append(L, x=None, T_new=0) == OK
    assert attend(L, True, q=None) == E_NULL          # but not when the array has elements


def test_last_error_is_thread_local_and_descriptive(L):
    msgs = {}

    def run(name, fn):
        fn()
        msgs[name] = L.csa_last_error().decode()

    t1 = threading.Thread(target=run, args=("a", lambda: compress(L, m=0)))
    t1.start()
    t1.join()
    t2 = threading.Thread(target=run, args=("b", lambda: index(L, d_I=48)))
    t2.start()
    t2.join()
    assert "m=0" in msgs["a"] and "d_I=48" in msgs["b"]


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 64, 128, dtype=torch.bfloat16)
    logits = torch.zeros(4)
    out = torch.zeros(1, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensors"):
        csa.csa_compress(x, logits, 4, out, entry_end=16)


def test_gather_diagnostic_validation(L):
    """csa_diag_gather_read rejects bad arguments before any launch."""
    def g(k=P, v=P, n_rows=1024, idx=P, groups=4, per=128, sink=P):
        return L.csa_diag_gather_read(k, v, n_rows, idx, groups, per, sink, None)
    assert g(k=None) == E_NULL and g(v=None) == E_NULL and g(idx=None) == E_NULL and g(sink=None) == E_NULL
    assert g(k=MIS) == E_ALIGN and g(v=MIS) == E_ALIGN
    assert g(groups=0) == E_SHAPE and g(groups=65537) == E_SHAPE
    assert g(per=0) == E_SHAPE and g(per=4097) == E_SHAPE
    assert g(n_rows=0) == E_SHAPE and g(n_rows=1 << 31) == E_SHAPE
