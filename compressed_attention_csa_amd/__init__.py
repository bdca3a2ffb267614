"""Python binding of libcsa, the gfx950 compressed-attention library.

Argument marshalling only: every step runs in the HIP kernels of ``libcsa.so``
through its C ABI (``include/csa.h``).  PyTorch provides device memory and the
current stream.  The binding raises ``CsaError`` for every non-OK status and
``ImportError``-like ``RuntimeError`` when the built library is missing; there
is no fallback path.

Functions (same names and argument order as the C ABI, tensors in place of
pointers, shapes read from the tensors):

    csa_compress(x, logits, m, out, out_scale=None, raw_base=0, entry_begin=0, entry_end=None)
    csa_index_topk(q_idx, w, k_idx, k_scale, t0, m, top_k, out_idx, out_score=None, workspace=None,
                   bf16_scores=False)
    csa_attend(q, k_cmp, v_cmp, m, idx, k_raw, v_raw, t0, window, scale, out, lse=None,
               raw_base=0, workspace=None)
    csa_attend_noalloc(q, k_cmp, v_cmp, m, idx, k_raw, v_raw, t0, window, scale, out, lse=None,
                       raw_base=0)
    hca_attend(q, k_cmp, v_cmp, m_heavy, k_raw, v_raw, t0, window, scale, out, lse=None,
               raw_base=0, workspace=None)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libcsa_debug.so")  # CSA_DEBUG build: NaN-poisoned scratch, plan checks

CSA_F32, CSA_BF16, CSA_FP8_E4M3 = 0, 1, 2
STATUS = ["CSA_OK", "CSA_E_NULL", "CSA_E_SHAPE", "CSA_E_DTYPE", "CSA_E_ALIGN",
          "CSA_E_WORKSPACE", "CSA_E_UNSUPPORTED", "CSA_E_HIP"]

# Exported symbols and their C signatures (kept in step with include/csa.h).
_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "csa_abi_version": (_i32, []),
    "csa_status_string": (ctypes.c_char_p, [_i32]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_compress": (_i32, [_vp, _i32, _i32, _i64, _i32, _i64, _vp, _i32, _i32, _i64, _i64, _i64,
                            _vp, _i32, _vp, _vp]),
    "csa_append": (_i32, [_vp, _i32, _i32, _i32, _i32, _i64, _vp, _i64, _vp, _i32, _i32, _i64, _vp,
                          _i32, _vp, _vp]),
    "csa_index_topk_workspace": (_sz, [_i32, _i64, _i32, _i32, _i64, _i32, _i32]),
    "csa_index_topk": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i64, _i32, _i32, _i64, _i64,
                              _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_bf16": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i64, _i32, _i32, _i64,
                                   _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_fp8": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _i32, _i32,
                                  _vp, _vp, _vp, _sz, _vp]),
    "csa_attend_workspace": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "csa_attend": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i64,
                          _i64, _i32, _i64, _i32, _i32, _i64, _i32, _f32, _vp, _i32, _vp, _vp, _sz,
                          _vp]),
    "csa_attend_noalloc": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp,
                                  _i64, _i64, _i32, _i64, _i32, _i32, _i64, _i32, _f32, _vp, _i32, _vp,
                                  _vp]),
    "hca_attend_workspace": (_sz, [_i32, _i64, _i32, _i32, _i64, _i32, _i32]),
    "hca_attend": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _vp, _vp, _i64, _i64,
                          _i32, _i64, _i32, _i32, _i64, _i32, _f32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "csa_diag_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
    "csa_diag_gather_read": (_i32, [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp]),
    "csa_profile_enable": (_i32, [_i32]),
    "csa_profile_report": (_i32, [ctypes.c_char_p, _sz]),
}

_lib = None


class CsaError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{fn}: {name}: {detail}")


def load(path: str) -> ctypes.CDLL:
    """The library at ``path`` with every declared signature bound."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m compressed_attention_csa_amd.build`"
                           + (" --debug" if path == DEBUG_LIB_PATH else ""))
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """The loaded libcsa.so (built by ``python -m compressed_attention_csa_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


class use_library:
    """Within the block, every call of this module goes to the library at ``path``
    (for instance DEBUG_LIB_PATH); the previous one is restored on exit."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = _lib
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def _check(fn, status):
    if status != 0:
        raise CsaError(fn, status, lib().csa_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return CSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libcsa takes device tensors; got a host tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_WS_CACHE: dict = {}


def workspace(nbytes: int, device, key: str = "default") -> torch.Tensor | None:
    """A zero-filled workspace of at least ``nbytes`` bytes, cached per (device, key).

    The library leaves a workspace zero-filled when a call finishes, so one zero
    fill at allocation is enough.  Calls sharing a key must be stream-ordered.
    """
    if nbytes == 0:
        return None
    k = (str(device), key)
    ws = _WS_CACHE.get(k)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS_CACHE[k] = ws
    return ws


def csa_compress(x, logits, m, out, out_scale=None, raw_base=0, entry_begin=0, entry_end=None,
                 overlap=0):
    """``logits`` holds m + overlap slot logits (overlap > 0: the overlapping variant)."""
    B, n_raw, d = x.shape
    N_alloc = out.shape[1]
    if entry_end is None:
        entry_end = min(N_alloc, (raw_base + n_raw) // m)
    st = lib().csa_compress(_ptr(x), _dt(x), B, n_raw, d, raw_base, _ptr(logits), m, overlap,
                            entry_begin, entry_end, N_alloc, _ptr(out), _dt(out), _ptr(out_scale),
                            _stream(x))
    _check("csa_compress", st)
    return out


def csa_append(x_new, ring, t0, logits, m, out, out_scale=None, overlap=0):
    """Append rows for positions t0 .. t0 + T_new - 1 to the mirrored ring
    [B, 2R, d] and compress the blocks they complete into ``out``."""
    B, T_new, d = x_new.shape
    R = ring.shape[1] // 2
    st = lib().csa_append(_ptr(x_new), _dt(x_new), B, T_new, d, t0, _ptr(ring), R, _ptr(logits), m,
                          overlap, out.shape[1], _ptr(out), _dt(out), _ptr(out_scale), _stream(x_new))
    _check("csa_append", st)
    return out


def ring_window(ring, s):
    """(raw rows, raw_base) that present positions s .. s + R - 1 of a mirrored ring."""
    R = ring.shape[1] // 2
    return ring, s - s % R


def index_topk_workspace_bytes(B, T, H_I, d_I, N_alloc, top_k, k_dt) -> int:
    return int(lib().csa_index_topk_workspace(B, T, H_I, d_I, N_alloc, top_k, k_dt))


def csa_index_topk(q_idx, w, k_idx, k_scale, t0, m, top_k, out_idx, out_score=None,
                   workspace_tensor=None, bf16_scores=False):
    """Exact top-k (csa_index_topk); with bf16_scores, csa_index_topk_bf16: the
    exact top-k of the scores rounded to bf16 (the approximate selector)."""
    B, T, H_I, d_I = q_idx.shape
    N_alloc = k_idx.shape[1]
    k_dt = _dt(k_idx)
    need = index_topk_workspace_bytes(B, T, H_I, d_I, N_alloc, top_k, k_dt)
    ws = workspace_tensor if workspace_tensor is not None else workspace(need, q_idx.device, "index")
    name = "csa_index_topk_bf16" if bf16_scores else "csa_index_topk"
    st = getattr(lib(), name)(_ptr(q_idx), _dt(q_idx), _ptr(w), _ptr(k_idx), k_dt, _ptr(k_scale),
                              B, T, H_I, d_I, N_alloc, t0, m, top_k, _ptr(out_idx),
                              _ptr(out_score), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(q_idx))
    _check(name, st)
    return out_idx


def csa_index_topk_fp8(q_idx, w, k_idx, k_scale, t0, m, top_k, out_idx, out_score=None,
                       workspace_tensor=None):
    """Exact top-k with fp8 x fp8 dot products (csa_index_topk_fp8): q_idx bf16,
    k_idx uint8 e4m3 codes with per-entry k_scale."""
    B, T, H_I, d_I = q_idx.shape
    N_alloc = k_idx.shape[1]
    need = index_topk_workspace_bytes(B, T, H_I, d_I, N_alloc, top_k, CSA_FP8_E4M3)
    ws = workspace_tensor if workspace_tensor is not None else workspace(need, q_idx.device, "index")
    st = lib().csa_index_topk_fp8(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), B, T, H_I, d_I, N_alloc,
                                  t0, m, top_k, _ptr(out_idx), _ptr(out_score), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(q_idx))
    _check("csa_index_topk_fp8", st)
    return out_idx


def csa_attend(q, k_cmp, v_cmp, m, idx, k_raw, v_raw, t0, window, scale, out, lse=None,
               raw_base=0, workspace_tensor=None, k_scale=None, v_scale=None):
    """k_cmp / v_cmp of dtype uint8 are e4m3 caches with per-entry k_scale / v_scale."""
    B, T, H, d = q.shape
    N_alloc = k_cmp.shape[1]
    top_k = 0 if idx is None else idx.shape[-1]
    need = int(lib().csa_attend_workspace(B, T, H, d, top_k, window))
    ws = workspace_tensor if workspace_tensor is not None else workspace(need, q.device, "attend")
    st = lib().csa_attend(_ptr(q), _dt(q), _ptr(k_cmp), _ptr(v_cmp), _dt(k_cmp), _ptr(k_scale),
                          _ptr(v_scale), N_alloc, m, _ptr(idx), top_k,
                          _ptr(k_raw), _ptr(v_raw), raw_base, k_raw.shape[1], B, T, H, d, t0,
                          window, float(scale), _ptr(out), _dt(out), _ptr(lse), _ptr(ws),
                          0 if ws is None else ws.numel(), _stream(q))
    _check("csa_attend", st)
    return out


def csa_attend_noalloc(q, k_cmp, v_cmp, m, idx, k_raw, v_raw, t0, window, scale, out, lse=None,
                       raw_base=0, k_scale=None, v_scale=None):
    """csa_attend on the library's own static scratch (no workspace argument)."""
    B, T, H, d = q.shape
    N_alloc = k_cmp.shape[1]
    top_k = 0 if idx is None else idx.shape[-1]
    st = lib().csa_attend_noalloc(_ptr(q), _dt(q), _ptr(k_cmp), _ptr(v_cmp), _dt(k_cmp), _ptr(k_scale),
                                  _ptr(v_scale), N_alloc, m, _ptr(idx), top_k,
                                  _ptr(k_raw), _ptr(v_raw), raw_base, k_raw.shape[1], B, T, H, d, t0,
                                  window, float(scale), _ptr(out), _dt(out), _ptr(lse), _stream(q))
    _check("csa_attend_noalloc", st)
    return out


def hca_attend(q, k_cmp, v_cmp, m_heavy, k_raw, v_raw, t0, window, scale, out, lse=None,
               raw_base=0, workspace_tensor=None, k_scale=None, v_scale=None):
    """k_cmp / v_cmp of dtype uint8 are e4m3 caches with per-entry k_scale / v_scale."""
    B, T, H, d = q.shape
    N_alloc = k_cmp.shape[1]
    need = int(lib().hca_attend_workspace(B, T, H, d, N_alloc, m_heavy, window))
    ws = workspace_tensor if workspace_tensor is not None else workspace(need, q.device, "attend")
    st = lib().hca_attend(_ptr(q), _dt(q), _ptr(k_cmp), _ptr(v_cmp), _dt(k_cmp), _ptr(k_scale),
                          _ptr(v_scale), N_alloc, m_heavy,
                          _ptr(k_raw), _ptr(v_raw), raw_base, k_raw.shape[1], B, T, H, d, t0,
                          window, float(scale), _ptr(out), _dt(out), _ptr(lse), _ptr(ws),
                          0 if ws is None else ws.numel(), _stream(q))
    _check("hca_attend", st)
    return out


def diag_stream_read(buf, sink):
    """Plain streaming read of the device tensor ``buf`` (diagnostics: the HBM read ceiling)."""
    st = lib().csa_diag_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf))
    _check("csa_diag_stream_read", st)


def diag_gather_read(k, v, idx, per_group, sink):
    """Row gather of 256-byte rows of the device tensors ``k`` and ``v`` at the int32
    indices ``idx`` (groups of ``per_group``; diagnostics: the gather rate)."""
    n_rows = k.numel() * k.element_size() // 256
    st = lib().csa_diag_gather_read(_ptr(k), _ptr(v), n_rows, _ptr(idx), idx.numel() // per_group, per_group,
                                    _ptr(sink), _stream(k))
    _check("csa_diag_gather_read", st)


def profile_enable(on: bool = True) -> bool:
    """Turn per-kernel event timing on or off for this thread; returns the old setting."""
    return bool(lib().csa_profile_enable(1 if on else 0))


def profile_report() -> dict:
    """Per-kernel {"launches", "total_ms"} since the last report (waits for the events)."""
    import json
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().csa_profile_report(buf, len(buf))
    if n < 0:
        raise CsaError("csa_profile_report", 7, "event query failed")
    return json.loads(buf.value.decode())
