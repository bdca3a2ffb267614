"""Shared helpers of the GPU parity tests: conversions and comparison criteria.

Criteria (each derived from the arithmetic of the two sides):
* compressor, fp32 / bf16 output: the GPU accumulates in fp64 and rounds once,
  like the oracle, so values must agree to one unit in the last place (and
  are expected to be bit-identical).
* e4m3 output: scales equal; codes equal except where the oracle's binary32
  quotient r/scale sits within binary32 rounding of a code midpoint.
* top-k: the GPU set must be a valid top-k of the oracle's fp64 scores with a
  1e-5 relative tie band at the k-th score (several sets are correct there).
* fp8 x fp8 top-k (csa_index_topk_fp8): the matrix cores sum e4m3 products in
  groups of 8 k-slots (8 consecutive dims here), aligned to the group's
  largest product, and drop the bits of every other product below 2^-13 of
  that product's power of two (measured on gfx950: a product 2^-14 times the
  largest vanishes, 2^-13 survives; the group sums then add in binary32).  So
  each dot product carries an error below 7 * 2^-13 * (largest product) per
  group plus binary32 rounding, and a score below
  E = sum_h |w_h| (sum_groups 7 * 2^-12 * max_d |q_d k_d| + 2^-21 sum_d |q_d k_d|)
  on the stored values (the bound doubled for margin; ReLU is 1-Lipschitz).
  The GPU's scores must lie within E (plus the 1e-5 relative fp32 allowance)
  of the oracle's, and its set must be a top-k of some scores within E of the
  oracle's: min over members of (s + E) >= max over visible non-members of
  (s - E), NaN scores ranking first as everywhere.
* approximate (bf16-score) top-k: the GPU set must be exactly the top-k, ties
  to the lower index, of the oracle's scores rounded to binary32 and then to
  bf16; where a binary32 score lies within 2^-20 of a bf16 rounding midpoint
  either rounding is accepted (the GPU's own binary32 sum may sit on the other
  side), taking the GPU's reported value for members and the lower one for
  non-members.
* attention: per (query, head) row, max_i |o_gpu - o_ref| <= tol * max_i |o_ref|
  with tol = 2e-3 for bf16 inputs, 1e-5 for fp32 inputs; lse to 1e-4 absolute
  plus 1e-5 relative.  A bf16 output also carries its own rounding, up to half
  a bf16 step per element (2^-8 relative), which no kernel can avoid; that
  amount is allowed on top.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats, method

TOL = {"bf16": 2e-3, "f32": 1e-5}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 image of a float32 / bf16 tensor (CPU or GPU)."""
    return t.detach().cpu().to(torch.float64).numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_dev_bf16(x64: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 device tensor holding the given (already bf16-representable) values;
    a NaN keeps its sign (quiet NaN pattern 0x7fc0 or 0xffc0)."""
    x64 = np.asarray(x64, np.float64)
    bits = formats.f64_to_bf16_bits(x64)
    nan = np.isnan(x64)
    bits = np.where(nan, np.where(np.signbit(x64), 0xFFC0, 0x7FC0), bits).astype(np.uint16)
    assert np.array_equal(formats.bf16_bits_to_f64(bits), x64, equal_nan=True), "value not bf16-representable"
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(device)


def to_dev_f32(x64: np.ndarray, device="cuda") -> torch.Tensor:
    x32 = x64.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x64), "value not binary32-representable"
    return torch.from_numpy(x32.copy()).to(device)


def ulp_diff_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16 bit patterns (finite values)."""
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def check_e4m3(codes_gpu, scale_gpu, r32_oracle):
    """Compare GPU e4m3 codes/scales with the oracle's quantiser of the same rows."""
    codes_o, scale_o, _ = formats.e4m3_quantize_rows(r32_oracle)
    np.testing.assert_array_equal(scale_gpu, scale_o)
    bad = codes_gpu != codes_o
    if bad.any():
        # only allowed where r/scale sits on a rounding midpoint (within binary32 rounding)
        y = (r32_oracle.astype(np.float32) / scale_o[..., None]).astype(np.float64)
        vals = formats.E4M3_VALUES
        dec_g = vals[codes_gpu[bad]]
        dec_o = vals[codes_o[bad]]
        mid = (dec_g + dec_o) / 2
        assert np.all(np.abs(np.abs(y[bad]) - np.abs(mid)) <= np.abs(mid) * 2.0 ** -22), \
            "e4m3 code differs away from a rounding midpoint"
    return int(bad.sum())


def bf16_half_step(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values around each (bf16-representable) value."""
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126)
    return np.where(a > 0, np.ldexp(1.0, e - 8), np.ldexp(1.0, -134))


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what="", out_bf16=False):
    """Row-relative output check and lse check; returns the worst row ratio.

    A bf16 output is the kernel's fp32 result rounded to nearest bf16, so each
    element may additionally sit half a bf16 step (up to 2^-8 relative) away.
    """
    tol = TOL[dtype]
    o_gpu = np.asarray(o_gpu, np.float64)
    err = np.abs(o_gpu - o_ref)
    if out_bf16:
        err = np.maximum(err - bf16_half_step(o_gpu), 0.0)
    d = err.max(axis=-1)
    ref = np.abs(o_ref).max(axis=-1)
    empty = np.isneginf(lse_ref)
    assert np.all(o_gpu[empty] == 0.0), f"{what}: empty rows must be zero"
    ok = d[~empty] <= tol * ref[~empty]
    worst = float((d[~empty] / np.maximum(ref[~empty], 1e-300)).max()) if (~empty).any() else 0.0
    assert ok.all(), f"{what}: {int((~ok).sum())} rows exceed tol {tol}, worst ratio {worst:.3e}"
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, np.float64)
        assert np.all(np.isneginf(lse_gpu[empty])), f"{what}: empty rows need lse = -inf"
        dl = np.abs(lse_gpu[~empty] - lse_ref[~empty])
        assert np.all(dl <= 1e-4 + 1e-5 * np.abs(lse_ref[~empty])), f"{what}: lse off by {dl.max():.3e}"
    return worst


def check_topk_rows(idx_gpu, score_gpu, scores64, visible, k):
    """Validate every row's selected set; returns the number of in-band swaps.

    visible[i] is the count of entries row i sees (a prefix of the entries)."""
    swaps = 0
    for i in range(idx_gpu.shape[0]):
        row = idx_gpu[i]
        c = int(visible[i])
        ok, why, sw = method.topk_is_valid(row, scores64[i], c, k)
        assert ok, f"row {i}: {why}"
        kk = min(k, c)
        assert np.all(row[:kk] >= 0) and np.all(row[kk:] == -1), f"row {i}: padding"
        if score_gpu is not None:
            sg = score_gpu[i, :kk].astype(np.float64)
            so = scores64[i, row[:kk]]
            fin = np.isfinite(scores64[i, :c])
            scale = np.abs(scores64[i, :c][fin]).max() if fin.any() else 1.0
            nan = np.isnan(so)
            assert np.all(np.isnan(sg[nan])), f"row {i}: a NaN score reported as a number"
            same_inf = np.isinf(so) & (sg == so)
            reg = ~nan & ~np.isinf(so)
            assert np.all(same_inf | ~np.isinf(so)), f"row {i}: infinite scores"
            err = np.abs(sg[reg] - so[reg]) / np.maximum(np.abs(so[reg]), 1e-2 * scale)
            assert np.all(err <= 1e-5), \
                f"row {i}: scores (worst relative error {err.max():.3e} at entry {row[:kk][reg][err.argmax()]}, " \
                f"{int((err > 1e-5).sum())} of {err.size} above 1e-5)"
            assert np.all(np.isneginf(score_gpu[i, kk:]))
        swaps += sw
    return swaps


def check_bf16_selection_row(row, score_row, scores64_row, visible, k):
    """Validate one row of the approximate selector; returns (kk, recall hits)
    where hits counts members of the exact fp64 top-k.  Finite scores only."""
    c = int(visible)
    vis = np.arange(c)
    assert np.isfinite(scores64_row[:c]).all(), "finite scores expected"
    kk = min(k, vis.size)
    G = row[:kk]
    assert np.all(row[kk:] == -1), "padding"
    assert np.all(G >= 0) and np.unique(G).size == kk, "members"
    assert np.all(G < c), "invisible member"
    s32 = formats.round_to_f32(scores64_row[vis])
    r_dn = formats.round_to_bf16(s32 - np.abs(s32) * 2.0 ** -20)
    r_up = formats.round_to_bf16(s32 + np.abs(s32) * 2.0 ** -20)
    R = np.full(scores64_row.shape[0], -np.inf)
    R[vis] = np.minimum(r_dn, r_up)
    lo = dict(zip(vis.tolist(), np.minimum(r_dn, r_up).tolist()))
    hi = dict(zip(vis.tolist(), np.maximum(r_dn, r_up).tolist()))
    if score_row is not None:
        sg = score_row[:kk].astype(np.float64)
        for j, v in zip(G.tolist(), sg.tolist()):
            assert lo[j] <= v <= hi[j], f"entry {j}: reported {v} outside [{lo[j]}, {hi[j]}]"
            R[j] = v
    else:
        R[G] = [hi[j] for j in G.tolist()]
    order = np.lexsort((vis, -R[vis]))
    exp = np.sort(vis[order[:kk]])
    np.testing.assert_array_equal(np.sort(G), exp, err_msg="not the top-k of the rounded scores")
    exact = set(vis[np.lexsort((vis, -scores64_row[vis]))[:kk]].tolist())
    return kk, len(exact & set(G.tolist()))


def check_attention_nonfinite(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what="", loose=None):
    """Attention outputs where some inputs are NaN or infinite.

    * every element the oracle makes non-finite is non-finite on the GPU (NaN
      or an infinity: the sides may differ in which, e.g. the GPU's weight
      w_hi + w_lo times inf with w_lo = 0 is NaN where the fp64 product is inf);
    * every element the oracle keeps finite is finite on the GPU and within
      check_attention's row criterion, relative to the largest finite
      reference element of its (query, head) row;
    * rows marked in ``loose`` ([T, H] bool) are only held to the first rule:
      they may come out non-finite where the oracle is finite (a documented
      case: a non-finite row shares a tile with a token that does not see it).
    lse: non-finite where the oracle's is; otherwise to 1e-4 + 1e-5 relative.
    """
    o_gpu = np.asarray(o_gpu, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    T, H = o_ref.shape[:2]
    loose = np.zeros((T, H), dtype=bool) if loose is None else np.asarray(loose, bool)
    bad_ref = ~np.isfinite(o_ref)
    assert np.all(~np.isfinite(o_gpu[bad_ref])), f"{what}: a non-finite reference element came out finite"
    fin = np.isfinite(o_ref) & ~loose[..., None]
    assert np.all(np.isfinite(o_gpu[fin])), f"{what}: an element the oracle keeps finite is not"
    tol = TOL[dtype]
    ref = np.abs(np.where(fin, o_ref, 0.0)).max(axis=-1, keepdims=True)
    err = np.abs(np.where(fin, o_gpu - np.where(fin, o_ref, 0.0), 0.0))
    assert np.all(err <= tol * ref), f"{what}: finite elements differ (worst {float((err / np.maximum(ref, 1e-300)).max()):.3e})"
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, np.float64)
        nf = ~np.isfinite(lse_ref)
        assert np.all(~np.isfinite(lse_gpu[nf])), f"{what}: lse of a non-finite row"
        ok = ~nf & ~loose
        dl = np.abs(lse_gpu[ok] - lse_ref[ok])
        assert np.all(dl <= 1e-4 + 1e-5 * np.abs(lse_ref[ok])), f"{what}: lse"


def fp8_score_error_bound(q_st, w, k_st):
    """E [T, N] of the fp8 x fp8 criterion above, from the stored query
    q_st [T, H, d], weights w [T, H] (None: ones) and stored keys k_st [N, d].
    Entries whose stored values are not finite get +inf."""
    T, H, d = q_st.shape
    N = k_st.shape[0]
    aq = np.abs(np.nan_to_num(q_st, nan=np.inf))
    ak = np.abs(np.nan_to_num(k_st, nan=np.inf))
    aw = np.ones((T, H)) if w is None else np.abs(np.asarray(w, dtype=np.float64))
    E = np.zeros((T, N))
    with np.errstate(invalid="ignore", over="ignore"):
        for t in range(T):
            for h in range(H):
                prod = aq[t, h][None, :] * ak  # [N, d]
                grp = prod.reshape(N, d // 8, 8).max(-1).sum(-1)
                E[t] += aw[t, h] * (7 * 2.0 ** -12 * grp + 2.0 ** -21 * prod.sum(-1))
    return np.where(np.isfinite(E), E, np.inf)


def check_topk_rows_fp8(idx_gpu, score_gpu, scores64, visible, k, E):
    """check_topk_rows under the fp8 x fp8 criterion (per-entry bound E [T, N])."""
    for i in range(idx_gpu.shape[0]):
        row = idx_gpu[i]
        c = int(visible[i])
        kk = min(k, c)
        assert np.all(row[:kk] >= 0) and np.all(row[kk:] == -1), f"row {i}: padding"
        G = row[:kk].astype(np.int64)
        assert np.unique(G).size == kk and np.all(G < c), f"row {i}: members"
        s = scores64[i, :c]
        nan = np.isnan(s)
        inG = np.zeros(c, dtype=bool)
        inG[G] = True
        nan_idx = np.nonzero(nan)[0]
        if nan_idx.size >= kk:
            assert np.array_equal(np.sort(G), nan_idx[:kk]), f"row {i}: not the lowest-indexed NaN entries"
        else:
            assert np.all(inG[nan_idx]), f"row {i}: a NaN-score entry is missing"
            mem = G[~nan[G]]
            out = np.nonzero(~nan & ~inG)[0]
            if mem.size and out.size:
                lo = np.min(s[mem] + E[i, mem])
                hi = np.max(s[out] - E[i, out])
                assert lo >= hi, f"row {i}: a member scores below a non-member beyond the bound ({lo} < {hi})"
        if score_gpu is not None:
            sg = score_gpu[i, :kk].astype(np.float64)
            so = scores64[i, G]
            fin = np.isfinite(s)
            scale = np.abs(s[fin]).max() if fin.any() else 1.0
            nn = np.isnan(so)
            assert np.all(np.isnan(sg[nn])), f"row {i}: a NaN score reported as a number"
            inf = np.isinf(so)
            assert np.all(sg[inf] == so[inf]), f"row {i}: infinite scores"
            reg = ~nn & ~inf
            tol = E[i, G][reg] + 1e-5 * np.maximum(np.abs(so[reg]), 1e-2 * scale)
            err = np.abs(sg[reg] - so[reg])
            assert np.all(err <= tol), \
                f"row {i}: scores (worst error / bound {np.max(err / tol):.3f} at entry {G[reg][np.argmax(err / tol)]})"
            assert np.all(np.isneginf(score_gpu[i, kk:]))
