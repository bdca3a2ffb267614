"""Plain fp64 CPU oracle of the compressed-attention hot path (one sequence at a time).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library and never imports it.

Sources (cited by page and section):

* [digest] V4 report digest, https://gitcode.csdn.net/69eb1ea054b52172bc6fc291.html
  - section 三: CSA folds every m KV rows into one entry, a Lightning Indexer
    scores the compressed entries and only the top-k of them take part in the
    core attention (Flash m=4, k=512; Pro m=4, k=1024); HCA folds every m'=128
    rows and attends densely, without top-k; both branches also see the newest
    n_win=128 tokens uncompressed.
  - section 七: the KV cache splits into a compressed ("classical") cache and a
    state cache holding the sliding window and the tokens whose block has not
    been folded yet.
* [book] "Evolution map" chapter, https://igloomatics.github.io/DeepSeek-V4-book/chapters/ch01.html
  - section 4: CSA turns each m=4 tokens into one super-KV and attends over the
    top-k=1024 of them (4096 fine tokens); HCA folds m'=128 tokens, giving
    n/m' = 8K dense entries at 1M context.
* [summary] structured summary, https://www.10100.com/article/149217299
  - section 2.1 / 2.2: the same constants (4:1, k=1024/512, window 128, 128:1).

Readings where the pages are silent (each is fixed here and used by the GPU
library in the same way):

* Compressor: each compressor owns one logit per slot, z in R^m, shared by the
  tensors it folds; weights alpha = softmax(z); entry j is
  sum_s alpha_s * x[j*m + s].  Blocks do not overlap; a trailing partial block
  is not emitted (its tokens are reached through the window).
* Visibility: entry j (covering positions j*m .. j*m+m-1) is visible to the
  query at position t iff its block ends at or before t, i.e. j < (t+1) // m.
* Indexer score: I(t, j) = sum_h w[t,h] * ReLU(qI[t,h] . kI[j]) with one key
  row per entry shared by all indexer heads; top-k is per query token and
  shared by all attention heads; ties go to the lower entry index.
* Attention: one KV head shared by all query heads; one softmax over the
  multiset (selected entries) + (raw window rows max(0, t-W+1) .. t), with the
  same scale for both kinds; a token may count once raw and once inside its
  block's entry.  An empty set gives o = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

from . import formats


# ----------------------------------------------------------------------------- compressor


def compressor_weights(z) -> np.ndarray:
    """Slot weights of one block compressor: softmax of its m logits, in fp64.

    [digest] section 三 and [book] section 4 give the folding of m rows into one
    entry; the weights are a softmax of learned per-slot logits (reading above).
    """
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def compress_exact(x, z, m: int, entry_begin: int = 0, entry_end: int | None = None,
                   raw_base: int = 0) -> np.ndarray:
    """Exact (fp64) block sums for entries [entry_begin, entry_end).

    ``x`` holds raw rows for positions raw_base .. raw_base + len(x) - 1.
    Entry j is sum_s alpha_s * x[position j*m + s]; every needed position must
    be present.  [digest] section 三; [book] section 4.
    """
    x = np.asarray(x, dtype=np.float64)
    alpha = compressor_weights(z)
    assert alpha.shape == (m,)
    if entry_end is None:
        entry_end = (raw_base + x.shape[0]) // m
    n_ent = entry_end - entry_begin
    if n_ent <= 0:
        return np.zeros((0, x.shape[1]), dtype=np.float64)
    lo = entry_begin * m - raw_base
    hi = entry_end * m - raw_base
    assert lo >= 0 and hi <= x.shape[0], "compressed blocks must lie inside the raw rows"
    blocks = x[lo:hi].reshape(n_ent, m, x.shape[1])
    return np.einsum("s,jsd->jd", alpha, blocks)


def compress_overlap(x, z, m: int, o: int, entry_begin: int = 0, entry_end: int | None = None,
                     raw_base: int = 0) -> np.ndarray:
    """Overlapping, position-weighted blocks (a method variant), exact in fp64.

    [summary] section 2.1 says the CSA compressor weights positions and lets
    blocks overlap so that no boundary loses context, without a formula.
    Reading taken: entry j folds the m + o rows of positions j*m - o .. j*m + m - 1
    (its own block and the last o rows of the previous one) with the weights
    softmax(z), z holding one logit per slot (m + o of them).  Slots before
    position 0 do not exist; the first entries take the softmax over the slots
    that do.  The entry still ends at position j*m + m - 1, so visibility is
    unchanged, and o = 0 is compress_exact.  ``x`` holds positions raw_base ..
    raw_base + len(x) - 1.
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    assert z.shape == (m + o,)
    if entry_end is None:
        entry_end = (raw_base + x.shape[0]) // m
    out = np.zeros((max(0, entry_end - entry_begin), x.shape[1]))
    for j in range(entry_begin, entry_end):
        pos = np.arange(j * m - o, j * m + m)
        ok = pos >= 0
        assert pos[ok][0] >= raw_base and pos[-1] < raw_base + x.shape[0], "rows outside x"
        w = compressor_weights(z[ok])
        out[j - entry_begin] = w @ x[pos[ok] - raw_base]
    return out


def state_ring(history, t_end: int, R: int) -> np.ndarray:
    """The state cache after positions 0 .. t_end were appended one by one.

    [digest] section 七 keeps the window rows and the rows of the block that is
    not complete yet in a state cache next to the compressed cache.  Reading
    taken here: a ring of R rows kept twice, position p written to rows p % R
    and p % R + R, so that the newest R positions are R consecutive rows.
    Returns [2R, d] float64; rows never written are NaN.
    """
    history = np.asarray(history, dtype=np.float64)
    ring = np.full((2 * R, history.shape[1]), np.nan)
    for p in range(t_end + 1):
        ring[p % R] = history[p]
        ring[p % R + R] = history[p]
    return ring


def completed_blocks(t0: int, T_new: int, m: int, N_alloc: int) -> range:
    """Blocks j < N_alloc whose last position (j+1) m - 1 lies in [t0, t0 + T_new - 1]."""
    return range(t0 // m, min(N_alloc, (t0 + T_new) // m))


def store(sums: np.ndarray, dtype: str):
    """Round exact entries once to the storage type.

    Returns a dict with ``values`` (float64 image of what is stored) and, for
    e4m3, ``codes`` (uint8) and ``scale`` (float32 per entry).  e4m3 follows
    ``formats.e4m3_quantize_rows``: the binary32 image of the exact sum is
    quantised with a per-entry absmax/448 scale.
    """
    if dtype == "f32":
        return {"values": formats.round_to_f32(sums)}
    if dtype == "bf16":
        return {"values": formats.round_to_bf16(sums)}
    if dtype == "e4m3":
        codes, scale, stored = formats.e4m3_quantize_rows(sums.astype(np.float32))
        return {"values": stored, "codes": codes, "scale": scale}
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- visibility


def visible_entries(t: int, m: int, n_alloc: int | None = None) -> int:
    """Number of compressed entries visible at position t: blocks ending at or before t."""
    c = (t + 1) // m
    return c if n_alloc is None else min(c, n_alloc)


def window_positions(t: int, W: int) -> np.ndarray:
    """Raw positions of the sliding window at t: the newest W tokens up to t ([digest] section 三)."""
    return np.arange(max(0, t - W + 1), t + 1, dtype=np.int64)


# ----------------------------------------------------------------------------- indexer


def index_scores(q_idx, w, k_idx, t0: int, m: int):
    """Lightning-Indexer scores in fp64 and the visible-entry count of every query.

    q_idx [T, H_I, d_I], w [T, H_I] (None means all ones), k_idx [N, d_I]
    (decoded stored values).  Query i sits at position t0 + i and sees the
    entries j < visible[i] = min(N, (t0 + i + 1) // m).  For those,
    I(t, j) = sum_h w[t,h] * max(0, q_idx[t,h] . k_idx[j]).
    [digest] sections 三 and 七; [summary] section 2.1.

    Returns (scores [T, N], visible [T]).  Visibility is carried by ``visible``
    alone: scores[i, j] for j >= visible[i] is NaN and is not a score.

    Non-finite inputs follow IEEE arithmetic: max(0, NaN) is NaN (the rectifier
    propagates NaN, of either sign), a NaN weight, query or key element makes
    the score NaN, and an infinity gives +-inf or, through inf - inf or 0 * inf,
    NaN.  The products and the head sum are written out elementwise, so that no
    library routine may skip a zero weight.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    T, H_I, _ = q_idx.shape
    N = k_idx.shape[0]
    w = np.ones((T, H_I)) if w is None else np.asarray(w, dtype=np.float64)
    out = np.full((T, N), np.nan)
    visible = np.array([visible_entries(t0 + i, m, N) for i in range(T)], dtype=np.int64)
    with np.errstate(invalid="ignore", over="ignore"):
        for i in range(T):
            c = int(visible[i])
            if c == 0:
                continue
            dots = np.einsum("hd,jd->hj", q_idx[i], k_idx[:c])  # [H_I, c]
            relu = np.maximum(dots, 0.0)  # np.maximum propagates NaN
            out[i, :c] = np.sum(w[i][:, None] * relu, axis=0)
    return out, visible


def quantize_query_e4m3(q_idx) -> np.ndarray:
    """The indexer query in fp8 e4m3: every (token, head) row quantised with the
    key rule (formats.e4m3_quantize_rows: binary32 absmax / 448 scale, 1 where
    that quotient is 0; codes rounded to nearest even).  Returns the stored
    values code * scale as float64, shape of q_idx.

    [digest] section 七: the indexer's QK path runs in low precision; with the
    keys already cached as e4m3, the plainest reading of an fp8 x fp8 product
    quantises the query the way the keys are quantised, one scale per head row.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    shape = q.shape
    _, _, stored = formats.e4m3_quantize_rows(q.reshape(-1, shape[-1]).astype(np.float32))
    return stored.reshape(shape)


def index_scores_fp8q(q_idx, w, k_idx, t0: int, m: int):
    """The fp8 x fp8 indexer variant: index_scores on the e4m3-quantised query
    (quantize_query_e4m3) against the stored keys; fp64 arithmetic on the
    stored values.  Returns (scores [T, N], visible [T]) as index_scores."""
    return index_scores(quantize_query_e4m3(q_idx), w, k_idx, t0, m)


def _rank_order(s, idx):
    """Indices ``idx`` ordered by the selection's total order on their scores s:
    NaN first, then decreasing value, then increasing index."""
    nan = np.isnan(s)
    return np.lexsort((idx, -np.where(nan, 0.0, s), ~nan))


def select_topk(scores: np.ndarray, visible, k: int) -> np.ndarray:
    """Per query, the min(k, visible) best visible entries; -1 pads the rest.

    The decision is taken on the binary32 images of the scores (the precision
    the GPU selects in), ordered by score (a NaN score ranks above every
    number, +inf included), then by lower index.  The output lists entries in
    that order.  [digest] section 三; [book] section 4.
    """
    T, N = scores.shape
    out = np.full((T, k), -1, dtype=np.int64)
    if k == 0:
        return out
    with np.errstate(over="ignore"):
        s32 = scores.astype(np.float32).astype(np.float64)
    for i in range(T):
        c = int(visible[i])
        if c == 0:
            continue
        vis = np.arange(c)
        order = _rank_order(s32[i, :c], vis)
        kk = min(k, c)
        out[i, :kk] = vis[order[:kk]]
    return out


def select_topk_bf16(scores: np.ndarray, visible, k: int) -> np.ndarray:
    """The approximate selector: select_topk on the scores rounded to bf16.

    [digest] section 七 speaks of a selector that ranks bf16 scores at a small
    loss of recall.  Reading taken: each score, in the binary32 precision the
    scores are computed in, is rounded once more to the nearest bf16 value
    (ties to even), and the exact top-k of those rounded values is selected,
    ties (now frequent) to the lower index.  NaN stays NaN (ranked first).
    """
    scores = np.asarray(scores, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        r = formats.round_to_bf16(formats.round_to_f32(scores))
    return select_topk(r, visible, k)


def topk_is_valid(G, scores_row: np.ndarray, visible: int, k: int, rel_band: float = 1e-5):
    """Check one query's selected set against exact fp64 scores.

    The query sees entries 0 .. visible-1.  With kk = min(k, visible): valid iff
    |G| = kk, the members are distinct and visible, and
      * NaN scores rank first: if there are at least kk of them, G is the kk
        lowest-indexed NaN entries; otherwise every NaN entry is in G and the
        rest of G is valid for the remaining places under the band rule;
      * band rule: every other member scores >= s_k - beta and every visible
        non-member scores <= s_k + beta, s_k being the kk-th best exact score
        and beta = rel_band * |s_k| (0 when s_k is infinite: equal infinities
        tie, and any choice among them is valid).
    Returns (ok, reason, n_in_band_swaps).
    """
    G = np.asarray(G, dtype=np.int64)
    G = G[G >= 0]
    c = int(visible)
    kk = min(k, c)
    if G.size != kk:
        return False, f"|G|={G.size} expected {kk}", 0
    if np.unique(G).size != G.size:
        return False, "duplicate members", 0
    if kk == 0:
        return True, "", 0
    if np.any(G >= c):
        return False, "invisible member", 0
    s = np.asarray(scores_row[:c], dtype=np.float64)
    nan_idx = np.nonzero(np.isnan(s))[0]
    inG = np.zeros(c, dtype=bool)
    inG[G] = True
    if nan_idx.size >= kk:
        ok = np.array_equal(np.sort(G), nan_idx[:kk])
        return (ok, "" if ok else "not the lowest-indexed NaN-score entries", 0)
    if not np.all(inG[nan_idx]):
        return False, "a NaN-score entry is missing", 0
    rest = np.nonzero(~np.isnan(s))[0]
    kr = kk - nan_idx.size
    s_sorted = np.sort(s[rest])[::-1]
    s_k = s_sorted[kr - 1]
    beta = rel_band * abs(s_k) if np.isfinite(s_k) else 0.0
    members = G[~np.isnan(s[G])]
    if np.any(s[members] < s_k - beta):
        return False, "member below the k-th score band", 0
    out_vis = rest[~inG[rest]]
    if out_vis.size and np.any(s[out_vis] > s_k + beta):
        return False, "non-member above the k-th score band", 0
    exact = set(rest[np.lexsort((rest, -s[rest]))[:kr]].tolist())
    swaps = len(exact.symmetric_difference(set(members.tolist()))) // 2
    return True, "", swaps


# ----------------------------------------------------------------------------- attention


def attend_entries(q_t, K_e, V_e, scale: float):
    """Softmax attention of H query heads over an explicit entry list (one shared KV head).

    q_t [H, d]; K_e, V_e [E, d] (E may be 0).  Returns (o [H, d], lse [H]).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    H, d = q_t.shape
    if K_e.shape[0] == 0:
        return np.zeros((H, d)), np.full(H, -np.inf)
    logits = scale * (q_t @ np.asarray(K_e, np.float64).T)  # [H, E]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    den = p.sum(axis=1, keepdims=True)
    o = (p @ np.asarray(V_e, np.float64)) / den
    lse = mx[:, 0] + np.log(den[:, 0])
    return o, lse


def _window_rows(t, W, k_raw, v_raw, raw_base):
    pos = window_positions(t, W)
    rows = pos - raw_base
    assert rows.size == 0 or (rows[0] >= 0 and rows[-1] < k_raw.shape[0]), "window not covered by raw rows"
    return k_raw[rows], v_raw[rows]


def csa_attend(q, k_cmp, v_cmp, idx, k_raw, v_raw, raw_base: int, t0: int, W: int,
               m: int, scale: float):
    """CSA core attention: selected compressed entries plus the raw window, one softmax.

    q [T, H, d]; k_cmp, v_cmp [N, d]; idx [T, k] (entries outside
    0 <= j < visible_entries(t) are skipped, so -1 pads); k_raw, v_raw hold raw
    rows for positions raw_base.. .  Returns (o [T, H, d], lse [T, H]).
    [digest] section 三 (selected entries + uncompressed window); [book] section 4.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cmp = np.asarray(k_cmp, np.float64)
    v_cmp = np.asarray(v_cmp, np.float64)
    k_raw = np.asarray(k_raw, np.float64)
    v_raw = np.asarray(v_raw, np.float64)
    T, H, d = q.shape
    o = np.zeros((T, H, d))
    lse = np.full((T, H), -np.inf)
    for i in range(T):
        t = t0 + i
        c = visible_entries(t, m, k_cmp.shape[0])
        sel = np.asarray(idx[i], dtype=np.int64)
        sel = sel[(sel >= 0) & (sel < c)]
        kw, vw = _window_rows(t, W, k_raw, v_raw, raw_base)
        K_e = np.concatenate([k_cmp[sel], kw], axis=0)
        V_e = np.concatenate([v_cmp[sel], vw], axis=0)
        o[i], lse[i] = attend_entries(q[i], K_e, V_e, scale)
    return o, lse


def hca_attend(q, k_cmp, v_cmp, m_heavy: int, k_raw, v_raw, raw_base: int, t0: int,
               W: int, scale: float):
    """HCA attention: every visible heavy entry plus the raw window, one softmax.

    Entries j < min(N, (t+1) // m_heavy) are all attended (no top-k).
    [digest] section 三; [book] section 4; [summary] section 2.2.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cmp = np.asarray(k_cmp, np.float64)
    v_cmp = np.asarray(v_cmp, np.float64)
    k_raw = np.asarray(k_raw, np.float64)
    v_raw = np.asarray(v_raw, np.float64)
    T, H, d = q.shape
    o = np.zeros((T, H, d))
    lse = np.full((T, H), -np.inf)
    for i in range(T):
        t = t0 + i
        c = visible_entries(t, m_heavy, k_cmp.shape[0])
        kw, vw = _window_rows(t, W, k_raw, v_raw, raw_base)
        K_e = np.concatenate([k_cmp[:c], kw], axis=0)
        V_e = np.concatenate([v_cmp[:c], vw], axis=0)
        o[i], lse[i] = attend_entries(q[i], K_e, V_e, scale)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint parts of one entry multiset.

    Part s has normalised output o_s and log-normaliser lse_s (-inf when
    empty).  With L = logsumexp_s(lse_s): o = sum_s exp(lse_s - L) * o_s and
    lse = L.  All parts empty gives o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)  # [S, ..., d]
    lse_parts = np.asarray(lse_parts, dtype=np.float64)  # [S, ...]
    mx = np.max(lse_parts, axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    wts = np.exp(lse_parts - safe)  # exp(-inf) = 0 for empty parts
    den = np.sum(wts, axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.sum(wts[..., None] * o_parts, axis=0) / den[..., None]
        lse = safe + np.log(den)
    empty = ~np.isfinite(mx)
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, lse)
    return o, lse


# ----------------------------------------------------------------------------- whole layers


def csa_layer(q, k_raw, v_raw, q_idx, k_idx_raw, w, z, m: int, top_k: int, W: int,
              scale: float, t0: int, cmp_dtype: str = "f32", idx_key_dtype: str = "f32"):
    """One CSA layer for one sequence whose raw rows start at position 0.

    Compress K, V and the indexer keys with the same compressor, score, select
    top-k and attend.  Returns a dict with every intermediate.
    """
    n = k_raw.shape[0]
    k_c = store(compress_exact(k_raw, z, m), cmp_dtype)
    v_c = store(compress_exact(v_raw, z, m), cmp_dtype)
    ki_c = store(compress_exact(k_idx_raw, z, m), idx_key_dtype)
    scores, visible = index_scores(q_idx, w, ki_c["values"], t0, m)
    idx = select_topk(scores, visible, top_k)
    o, lse = csa_attend(q, k_c["values"], v_c["values"], idx, k_raw, v_raw, 0, t0, W, m, scale)
    assert n >= t0 + q.shape[0]
    return {"k_cmp": k_c, "v_cmp": v_c, "k_idx": ki_c, "scores": scores, "visible": visible,
            "idx": idx, "o": o, "lse": lse}


def hca_layer(q, k_raw, v_raw, z, m_heavy: int, W: int, scale: float, t0: int,
              cmp_dtype: str = "f32"):
    """One HCA layer for one sequence whose raw rows start at position 0."""
    k_c = store(compress_exact(k_raw, z, m_heavy), cmp_dtype)
    v_c = store(compress_exact(v_raw, z, m_heavy), cmp_dtype)
    o, lse = hca_attend(q, k_c["values"], v_c["values"], m_heavy, k_raw, v_raw, 0, t0, W, scale)
    return {"k_cmp": k_c, "v_cmp": v_c, "o": o, "lse": lse}
