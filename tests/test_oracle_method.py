"""Pins of the oracle's method steps against closed forms, library routines and brute force.

Each test is chosen so that a plausible mistake in ``oracle.method`` (a dropped
term, a wrong sign or index, a transposed operand, an off-by-one block or
visibility bound) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import brute, formats, method


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- compressor


def test_weights_are_softmax_and_shift_invariant():
    z = rnd(0, 4)
    a = method.compressor_weights(z)
    assert abs(a.sum() - 1) < 1e-15 and np.all(a > 0)
    np.testing.assert_allclose(method.compressor_weights(z + 3.7), a, rtol=1e-14)
    # larger logit -> larger weight, slot order preserved
    assert np.argmax(a) == np.argmax(z)


def test_compress_m1_is_a_copy():
    x = rnd(1, 37, 8)
    np.testing.assert_array_equal(method.compress_exact(x, [0.3], 1), x)


@pytest.mark.parametrize("m", [4, 128])
def test_uniform_logits_give_mean_pooling(m):
    x = np.random.default_rng(2).integers(-1000, 1000, (m * 5 + 3, 16)).astype(np.float64)
    got = method.compress_exact(x, np.full(m, 0.25), m)
    exp = x[: m * 5].reshape(5, m, 16).mean(axis=1)
    np.testing.assert_array_equal(got, exp)  # 1/m is exact; integer sums are exact


def test_dominant_logit_picks_its_slot():
    x = rnd(3, 40, 4)
    for s in range(4):
        z = np.zeros(4)
        z[s] = 800.0  # exp(-800) underflows: alpha is one-hot
        np.testing.assert_array_equal(method.compress_exact(x, z, 4), x[s::4][:10])


def test_compress_is_linear_and_drops_partial_block():
    x, y = rnd(4, 23, 6), rnd(5, 23, 6)
    z = rnd(6, 4)
    cx, cy = method.compress_exact(x, z, 4), method.compress_exact(y, z, 4)
    assert cx.shape == (5, 6)
    np.testing.assert_allclose(method.compress_exact(2 * x - 3 * y, z, 4), 2 * cx - 3 * cy,
                               rtol=1e-13, atol=1e-13)


def test_compress_subrange_with_raw_base_matches_full():
    x = rnd(7, 64, 5)
    z = rnd(8, 4)
    full = method.compress_exact(x, z, 4)
    part = method.compress_exact(x[20:], z, 4, entry_begin=5, entry_end=16, raw_base=20)
    np.testing.assert_array_equal(part, full[5:16])


def test_compress_matches_brute_force():
    x = rnd(9, 61, 7)
    z = rnd(10, 4) * 0.5
    got = method.compress_exact(x, z, 4)
    exp = np.array(brute.compress(x.tolist(), z.tolist(), 4))
    np.testing.assert_allclose(got, exp, rtol=1e-14, atol=1e-15)


def test_overlap_zero_is_the_plain_compressor():
    x, z = rnd(31, 50, 6), rnd(32, 4) * 0.5
    np.testing.assert_allclose(method.compress_overlap(x, z, 4, 0), method.compress_exact(x, z, 4), rtol=1e-14,
                               atol=1e-15)


def test_overlap_brute_force_and_first_entries():
    """Direct fsum over the m + o rows; the first entries renormalise over the
    slots at positions >= 0."""
    m, o = 4, 3
    x, z = rnd(33, 29, 5), rnd(34, m + o) * 0.7
    got = method.compress_overlap(x, z, m, o)
    for j in range(len(got)):
        rows = [(s, j * m - o + s) for s in range(m + o) if j * m - o + s >= 0]
        e = [math.exp(z[s]) for s, _ in rows]
        tot = math.fsum(e)
        for c in range(x.shape[1]):
            exp = math.fsum(e[i] / tot * x[p, c] for i, (_, p) in enumerate(rows))
            assert abs(got[j, c] - exp) <= 1e-13 * (1 + abs(exp))


def test_overlap_slot_order_and_uniform_weights():
    """A dominant first logit picks the oldest overlapped row j*m - o (the offset
    runs backwards); uniform logits average the m + o rows."""
    m, o = 4, 2
    x = rnd(35, 40, 3)
    z = np.full(m + o, -60.0)
    z[0] = 0.0
    got = method.compress_overlap(x, z, m, o, entry_begin=1)
    np.testing.assert_allclose(got, x[[j * m - o for j in range(1, 10)]], rtol=0, atol=1e-20)
    u = method.compress_overlap(x, np.zeros(m + o), m, o, entry_begin=1)
    np.testing.assert_allclose(u, [x[j * m - o: j * m + m].mean(axis=0) for j in range(1, 10)], rtol=1e-14)


def test_overlap_subrange_with_raw_base_matches_full():
    m, o = 4, 4
    x, z = rnd(36, 64, 5), rnd(37, m + o)
    full = method.compress_overlap(x, z, m, o)
    part = method.compress_overlap(x[16:], z, m, o, entry_begin=5, entry_end=16, raw_base=16)
    np.testing.assert_array_equal(part, full[5:16])


@pytest.mark.parametrize("R", [5, 8, 13])
def test_state_ring_holds_the_newest_R_positions_as_consecutive_rows(R):
    """Every window of <= R newest positions is a contiguous row range of the
    mirrored ring, starting at row s % R; rows of older positions are gone."""
    rng = np.random.default_rng(R)
    hist = rng.standard_normal((40, 3))
    for t_end in (0, R - 2, R - 1, R, 2 * R + 3, 39):
        if t_end < 0:
            continue
        ring = method.state_ring(hist, t_end, R)
        lo = max(0, t_end - R + 1)
        for s in range(lo, t_end + 1):
            L = t_end - s + 1
            np.testing.assert_array_equal(ring[s % R: s % R + L], hist[s: t_end + 1])
        held = {tuple(r) for r in ring if not np.isnan(r).any()}
        assert held == {tuple(hist[p]) for p in range(lo, t_end + 1)}


def test_compressing_from_the_ring_equals_compressing_the_history():
    """Blocks completed by each append, compressed from the ring view, are the
    entries of the full history; the completed-block ranges tile the entries."""
    rng = np.random.default_rng(3)
    m, R, N = 4, 11, 25
    hist = rng.standard_normal((103, 6))
    z = rng.standard_normal(m) * 0.5
    full = method.compress_exact(hist, z, m, 0, N)
    seen, t = [], 0
    for T_new in [1, 1, 3, 2, 8, 1] * 20:
        if t >= len(hist):
            break
        T_new = min(T_new, len(hist) - t, R - m + 1)
        ring = method.state_ring(hist, t + T_new - 1, R)
        blocks = method.completed_blocks(t, T_new, m, N)
        if len(blocks):
            p_lo = blocks.start * m
            got = method.compress_exact(ring, z, m, blocks.start, blocks.stop, raw_base=p_lo - p_lo % R)
            np.testing.assert_allclose(got, full[blocks.start:blocks.stop], rtol=1e-15, atol=0)
            seen.extend(blocks)
        t += T_new
    assert seen == list(range(min(N, len(hist) // m)))


def test_store_rounds_once():
    s = rnd(11, 10, 64)
    np.testing.assert_array_equal(method.store(s, "bf16")["values"], formats.round_to_bf16(s))
    np.testing.assert_array_equal(method.store(s, "f32")["values"], s.astype(np.float32))
    e = method.store(s, "e4m3")
    np.testing.assert_array_equal(
        e["values"], formats.e4m3_decode(e["codes"]) * e["scale"][:, None].astype(np.float64))


# ----------------------------------------------------------------------------- visibility


def test_visibility_closed_form():
    m = 4
    assert method.visible_entries(m - 2, m) == 0
    assert method.visible_entries(m - 1, m) == 1  # block 0 ends at position m-1
    assert method.visible_entries(2 * m - 2, m) == 1
    n = 1 << 20
    assert method.visible_entries(n - 1, 4) == n // 4
    assert method.visible_entries(n - 1, 128) == 8192  # n/m' = 8K at 1M context
    assert method.visible_entries(n - 1, 4, n_alloc=1000) == 1000
    np.testing.assert_array_equal(method.window_positions(5, 128), np.arange(6))
    np.testing.assert_array_equal(method.window_positions(500, 128), np.arange(373, 501))
    assert method.window_positions(10, 0).size == 0


# ----------------------------------------------------------------------------- indexer


def test_single_head_unit_weight_positive_dots_is_a_matrix_product():
    rng = np.random.default_rng(12)
    q = np.abs(rng.standard_normal((9, 1, 16)))
    k = np.abs(rng.standard_normal((30, 16)))
    s, vis = method.index_scores(q, None, k, t0=119, m=4)  # position >= 119: all 30 visible
    assert (vis == 30).all()
    np.testing.assert_allclose(s, q[:, 0, :] @ k.T, rtol=1e-14)


def test_scores_sign_scaling_and_zero_head():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((5, 3, 8))
    k = rng.standard_normal((20, 8))
    w = rng.standard_normal((5, 3))
    s = method.index_scores(q, w, k, 100, 4)[0]
    np.testing.assert_allclose(method.index_scores(q, 2.5 * w, k, 100, 4)[0], 2.5 * s, rtol=1e-14)
    np.testing.assert_allclose(method.index_scores(0.5 * q, w, k, 100, 4)[0], 0.5 * s, rtol=1e-14)
    # one head with w = -1: score = -ReLU(q.k)
    s1 = method.index_scores(q[:, :1], -np.ones((5, 1)), k, 100, 4)[0]
    np.testing.assert_allclose(s1, -np.maximum(q[:, 0] @ k.T, 0), rtol=1e-14)
    # a head with zero weight contributes nothing
    w0 = w.copy()
    w0[:, 2] = 0
    np.testing.assert_allclose(method.index_scores(q, w0, k, 100, 4)[0],
                               method.index_scores(q[:, :2], w[:, :2], k, 100, 4)[0], rtol=1e-14)


def test_scores_visibility_mask():
    q = rnd(14, 6, 2, 4)
    k = rnd(15, 10, 4)
    s, vis = method.index_scores(q, None, k, t0=2, m=4)  # positions 2..7
    for i in range(6):
        c = (2 + i + 1) // 4
        assert vis[i] == c
        assert np.all(np.isfinite(s[i, :c])) and np.all(np.isnan(s[i, c:]))
    # the selection never reaches past the visible count, whatever the other values hold
    sel = method.select_topk(np.zeros((6, 10)), vis, 3)
    for i in range(6):
        assert list(sel[i]) == list(range(min(3, vis[i]))) + [-1] * (3 - min(3, vis[i]))


def test_scores_match_brute_force():
    q = rnd(16, 4, 3, 5)
    k = rnd(17, 12, 5)
    w = rnd(18, 4, 3)
    s, _ = method.index_scores(q, w, k, t0=47, m=4)  # (47+1)//4 = 12: all entries visible
    for i in range(4):
        for j in range(12):
            assert math.isclose(s[i, j], brute.score(q[i].tolist(), w[i].tolist(), k[j].tolist()),
                                rel_tol=1e-13, abs_tol=1e-14)


# ----------------------------------------------------------------------------- top-k


def test_topk_matches_torch_topk_on_distinct_scores():
    s = rnd(19, 7, 300)
    got = method.select_topk(s, [300] * 7, 25)
    exp = torch.topk(torch.from_numpy(s), 25, dim=1).indices.numpy()
    for i in range(7):
        assert set(got[i]) == set(exp[i])


def test_topk_short_list_pads_and_ties_go_low():
    s = np.full((2, 10), np.nan)
    s[0, :6] = [1.0, 3.0, 3.0, 2.0, 3.0, 0.5]
    s[1, :3] = [0.0, 0.0, 0.0]
    got = method.select_topk(s, [6, 3], 4)
    assert list(got[0]) == [1, 2, 4, 3]  # three-way tie at 3.0 ordered by index
    assert list(got[1]) == [0, 1, 2, -1]


def test_topk_permutation_equivariance():
    s = rnd(20, 3, 50)
    perm = np.random.default_rng(21).permutation(50)
    a = method.select_topk(s, [50] * 3, 10)
    b = method.select_topk(s[:, perm], [50] * 3, 10)
    for i in range(3):
        assert set(perm[b[i]]) == set(a[i])


def test_bf16_selector_hand_example():
    """Near 1 the bf16 spacing is 2^-7 above and 2^-8 below: 1.003 and 0.999
    round to 1.0, 1.004 and 1.006 to 1.0078125; the ties at 1.0 go to the lowest
    index, so the approximate top-4 takes entry 0 where the exact one takes 1."""
    s = np.array([[1.0, 1.003, 0.999, 2.0, 1.004, 1.006]])
    assert list(method.select_topk_bf16(s, [6], 4)[0]) == [3, 4, 5, 0]
    assert list(method.select_topk(s, [6], 4)[0]) == [3, 5, 4, 1]


def test_bf16_selector_rounds_ties_to_even():
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd last bit) and 1 + 2^-6 (even):
    # it rounds up and ties entry 1 (just below 1 + 2^-6), so index 0 wins.
    s = np.array([[1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6 - 2.0 ** -20]])
    assert list(method.select_topk_bf16(s, [2], 1)[0]) == [0]
    # 1 + 2^-8 lies halfway between 1 (even) and 1 + 2^-7: it rounds down.
    s = np.array([[1 + 2.0 ** -8, 1 + 2.0 ** -7]])
    assert list(method.select_topk_bf16(s, [2], 1)[0]) == [1]


def test_bf16_selector_equals_exact_on_bf16_values_and_keeps_invisible_out():
    s = formats.round_to_bf16(rnd(23, 4, 300))
    s[:, 250:] = np.nan  # not visible: never selected, even though NaN would rank first
    vis = [250] * 4
    np.testing.assert_array_equal(method.select_topk_bf16(s, vis, 40), method.select_topk(s, vis, 40))
    assert (method.select_topk_bf16(s, vis, 260)[:, 250:] == -1).all()


def test_topk_validity_checker_accepts_oracle_and_rejects_planted_swap():
    s = rnd(22, 1, 200)[0]
    sel = method.select_topk(s[None], [200], 20)[0]
    ok, _, swaps = method.topk_is_valid(sel, s, 200, 20)
    assert ok and swaps == 0
    order = np.argsort(-s)
    bad = sel.copy()
    bad[np.where(bad == order[19])[0][0]] = order[40]  # swap the 20th for the 41st
    assert not method.topk_is_valid(bad, s, 200, 20)[0]
    assert not method.topk_is_valid(sel[:19], s, 200, 20)[0]
    dup = sel.copy()
    dup[0] = dup[1]
    assert not method.topk_is_valid(dup, s, 200, 20)[0]
    # a member past the visible count is rejected
    assert not method.topk_is_valid(sel, s, int(sel.max()), 20)[0]
    # members inside the tie band are accepted
    s2 = s.copy()
    s2[order[20]] = s2[order[19]] * (1 - 1e-7)
    swapped = sel.copy()
    swapped[np.where(swapped == order[19])[0][0]] = order[20]
    ok, _, swaps = method.topk_is_valid(swapped, s2, 200, 20)
    assert ok and swaps == 1


def test_fp8_query_variant_is_identity_on_e4m3_rows_with_unit_scale():
    """Query rows already on the e4m3 grid with largest magnitude exactly 448
    quantise to themselves (scale 1): the fp8 x fp8 scores equal the plain ones."""
    rng = np.random.default_rng(41)
    vals = formats.E4M3_VALUES[np.isfinite(formats.E4M3_VALUES)]
    q = rng.choice(vals, size=(6, 3, 32))
    q[:, :, 0] = 448.0
    k = formats.round_to_bf16(rng.standard_normal((50, 32)))
    w = rng.standard_normal((6, 3))
    np.testing.assert_array_equal(method.quantize_query_e4m3(q), q)
    np.testing.assert_array_equal(method.index_scores_fp8q(q, w, k, 199, 4)[0], method.index_scores(q, w, k, 199, 4)[0])


def test_fp8_query_variant_matches_torch_e4m3_and_bounds_the_error():
    rng = np.random.default_rng(42)
    q = formats.round_to_bf16(rng.standard_normal((5, 4, 64)) * rng.uniform(0.01, 30, (5, 4, 1)))
    k = formats.round_to_bf16(rng.standard_normal((40, 64)))
    stored = method.quantize_query_e4m3(q)
    # per row: torch's own e4m3 conversion of q / scale, times the scale
    for t in range(5):
        for h in range(4):
            r = q[t, h].astype(np.float32)
            sc = np.float32(np.abs(r).max() / np.float32(448.0))
            y = torch.from_numpy(r / sc).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            np.testing.assert_array_equal(stored[t, h], y * np.float64(sc))
    # each quantised element is within half an e4m3 step (2^-4 relative, or the subnormal floor)
    sc = np.abs(q).max(axis=-1, keepdims=True).astype(np.float32) / np.float32(448.0)
    assert np.all(np.abs(stored - q) <= np.maximum(np.abs(q) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6))
    # so the scores move by at most sum_h |w_h| sum_i |dq_i| |k_i|
    w = np.abs(rng.standard_normal((5, 4)))
    s8 = method.index_scores_fp8q(q, w, k, 159, 4)[0]
    s = method.index_scores(q, w, k, 159, 4)[0]
    bound = np.einsum("th,thd,jd->tj", w, np.abs(stored - q), np.abs(k))
    assert np.all(np.abs(s8 - s) <= bound * (1 + 1e-9) + 1e-12)


# ----------------------------------------------------------------------------- non-finite inputs
#
# Contract: IEEE arithmetic throughout; the rectifier propagates NaN of either
# sign; a NaN score ranks above every number (+inf included), ties by lower
# index; visibility is positional only, never inferred from a score's value.


def test_topk_order_with_nan_and_infinities_equals_torch_stable_sort():
    """torch's CPU sort puts NaN above +inf (descending) and keeps equal keys in
    index order when stable: the selection's total order, from a library."""
    rng = np.random.default_rng(31)
    for trial in range(20):
        s = rng.standard_normal((1, 64))
        s[0, rng.choice(64, 5, replace=False)] = np.nan
        s[0, rng.choice(64, 3, replace=False)] = np.inf
        s[0, rng.choice(64, 3, replace=False)] = -np.inf
        s[0, 10:14] = s[0, 9]  # a run of equal finite values (ties by index)
        k = int(rng.integers(1, 64))
        got = method.select_topk(s, [64], k)[0]
        exp = torch.sort(torch.from_numpy(s[0]), descending=True, stable=True).indices[:k].numpy()
        np.testing.assert_array_equal(got, exp)


def test_scores_with_nan_and_infinities_follow_ieee():
    q = np.ones((1, 2, 4))
    k = np.ones((6, 4))
    k[1, 2] = np.nan          # NaN key element: NaN score whatever the weights
    k[2, 0] = -np.nan         # NaN of negative sign: still NaN (the rectifier keeps it)
    k[3, 1] = np.inf          # dot +inf in both heads
    k[4, :] = -1.0            # dots -4: rectified to 0
    w = np.array([[1.0, 0.0]])  # a zero weight times NaN or inf is still NaN
    s, vis = method.index_scores(q, w, k, t0=23, m=4)
    assert vis[0] == 6
    assert np.isnan(s[0, 1]) and np.isnan(s[0, 2])
    assert np.isnan(s[0, 3])  # 1 * inf + 0 * inf = inf + NaN
    assert s[0, 4] == 0.0 and s[0, 0] == 4.0 and s[0, 5] == 4.0
    w2 = np.array([[1.0, 1.0]])
    s2, _ = method.index_scores(q, w2, k, t0=23, m=4)
    assert s2[0, 3] == np.inf
    w3 = np.array([[1.0, -1.0]])
    s3, _ = method.index_scores(q, w3, k, t0=23, m=4)
    assert np.isnan(s3[0, 3])  # inf - inf
    w4 = np.array([[-1.0, -1.0]])
    s4, _ = method.index_scores(q, w4, k, t0=23, m=4)
    assert s4[0, 3] == -np.inf and s4[0, 0] == -8.0
    # a NaN in one head of the query, or in a weight, makes every score of that query NaN
    qn = q.copy()
    qn[0, 1, 3] = np.nan
    assert np.isnan(method.index_scores(qn, w2, k, 23, 4)[0]).all()
    assert np.isnan(method.index_scores(q, np.array([[np.nan, 1.0]]), k, 23, 4)[0]).all()


def test_nan_scores_are_selected_first_and_reported_valid():
    s = np.array([[0.5, np.nan, 2.0, -np.inf, np.nan, np.inf, 1.0, np.nan]])
    assert list(method.select_topk(s, [8], 5)[0]) == [1, 4, 7, 5, 2]
    assert list(method.select_topk(s, [8], 2)[0]) == [1, 4]  # NaN ties: lower index first
    assert list(method.select_topk(s, [5], 8)[0]) == [1, 4, 2, 0, 3, -1, -1, -1]
    row = s[0]
    assert method.topk_is_valid([1, 4, 7, 5, 2], row, 8, 5)[0]
    assert method.topk_is_valid([2, 5, 7, 4, 1], row, 8, 5)[0]  # any order
    assert not method.topk_is_valid([1, 4, 5, 2, 6], row, 8, 5)[0]  # a NaN entry left out
    assert not method.topk_is_valid([1, 7], row, 8, 2)[0]  # NaN ties go to the lower index
    assert method.topk_is_valid([1, 4], row, 8, 2)[0]
    # equal infinities tie: either one may be chosen
    s5 = np.array([np.inf, 1.0, np.inf, 0.0])
    assert method.topk_is_valid([0], s5, 4, 1)[0] and method.topk_is_valid([2], s5, 4, 1)[0]
    assert not method.topk_is_valid([1], s5, 4, 1)[0]
    # -inf scores are visible entries like any other
    s6 = np.array([-np.inf, -np.inf, 3.0])
    assert list(method.select_topk(s6[None], [3], 3)[0]) == [2, 0, 1]
    assert method.topk_is_valid([2, 1, 0], s6, 3, 3)[0]


def test_attention_propagates_nan_to_exactly_the_rows_it_touches():
    rng = np.random.default_rng(32)
    H, d, N, W, m = 4, 8, 10, 3, 4
    q = rng.standard_normal((2, H, d))
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kr, vr = rng.standard_normal((60, d)), rng.standard_normal((60, d))
    idx = np.array([[0, 2, 5], [1, 3, 7]])
    t0 = 40
    base, _ = method.csa_attend(q, kc, vc, idx, kr, vr, 0, t0, W, m, 0.3)
    assert np.isfinite(base).all()
    qn = q.copy()
    qn[0, 2, 5] = np.nan  # query 0, head 2
    o, lse = method.csa_attend(qn, kc, vc, idx, kr, vr, 0, t0, W, m, 0.3)
    assert np.isnan(o[0, 2]).all() and np.isnan(lse[0, 2])
    mask = np.ones_like(o, dtype=bool)
    mask[0, 2] = False
    np.testing.assert_array_equal(o[mask], base[mask])
    kn = kc.copy()
    kn[5, 1] = np.nan  # entry 5: selected by query 0 only
    o, lse = method.csa_attend(q, kn, vc, idx, kr, vr, 0, t0, W, m, 0.3)
    assert np.isnan(o[0]).all() and np.isnan(lse[0]).all()
    np.testing.assert_array_equal(o[1], base[1])
    vn = vc.copy()
    vn[7, 6] = -np.nan  # entry 7, column 6: selected by query 1 only
    o, _ = method.csa_attend(q, kc, vn, idx, kr, vr, 0, t0, W, m, 0.3)
    assert np.isnan(o[1, :, 6]).all()
    cols = np.arange(d) != 6
    np.testing.assert_array_equal(o[1][:, cols], base[1][:, cols])
    np.testing.assert_array_equal(o[0], base[0])
    vi = vc.copy()
    vi[2, 0] = np.inf  # entry 2 (query 0), column 0: a positive weight times inf
    o, _ = method.csa_attend(q, kc, vi, idx, kr, vr, 0, t0, W, m, 0.3)
    assert np.isposinf(o[0, :, 0]).all()
    np.testing.assert_array_equal(o[1], base[1])
    # an unselected or invisible entry's NaN reaches nothing
    kn2 = kc.copy()
    kn2[9] = np.nan
    o, _ = method.csa_attend(q, kn2, vc, idx, kr, vr, 0, t0, W, m, 0.3)
    np.testing.assert_array_equal(o, base)


# ----------------------------------------------------------------------------- attention


def _sdpa(q, K, V, scale, mask):
    """torch CPU scaled_dot_product_attention in float64 with one shared KV head."""
    T, H, d = q.shape
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1, H, T, d]
    Kt = torch.from_numpy(K)[None, None].expand(1, H, *K.shape)
    Vt = torch.from_numpy(V)[None, None].expand(1, H, *V.shape)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _layer(seed, n, T, t0, H, d, m, k, W, hi=2, di=8):
    """Random layer inputs, binary32-representable (entries are stored as binary32)."""
    rng = np.random.default_rng(seed)

    def r(*shape):
        return rng.standard_normal(shape).astype(np.float32).astype(np.float64)

    return r(T, H, d), r(n, d), r(n, d), r(T, hi, di), r(n, di), r(T, hi), r(m) * 0.5


def test_m1_all_selected_no_window_is_full_causal_attention():
    n, H, d = 48, 3, 16
    q, K, V, qi, ki, w, _ = _layer(30, n, n, 0, H, d, 1, n, 0)
    res = method.csa_layer(q, K, V, qi, ki, w, [0.0], m=1, top_k=n, W=0, scale=0.25, t0=0)
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    np.testing.assert_allclose(res["o"], _sdpa(q, K, V, 0.25, mask), rtol=1e-12, atol=1e-13)
    logits = torch.from_numpy(0.25 * np.einsum("thd,sd->ths", q, K)).masked_fill(~mask[:, None, :], -np.inf)
    np.testing.assert_allclose(res["lse"], torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-13)


def test_m1_all_selected_with_window_is_causal_attention_with_ln2_bias():
    n, H, d, W = 40, 2, 8, 6
    q, K, V, qi, ki, w, _ = _layer(31, n, n, 0, H, d, 1, n, W)
    res = method.csa_layer(q, K, V, qi, ki, w, [0.0], m=1, top_k=n, W=W, scale=0.3, t0=0)
    t = torch.arange(n)[:, None]
    s = torch.arange(n)[None, :]
    bias = torch.zeros(n, n, dtype=torch.float64)
    bias[(s <= t) & (s > t - W)] = math.log(2.0)  # a window token counts twice
    bias[s > t] = -math.inf
    np.testing.assert_allclose(res["o"], _sdpa(q, K, V, 0.3, bias), rtol=1e-12, atol=1e-13)


def test_csa_with_k_covering_all_entries_equals_hca_with_same_block():
    n, T, t0, H, d, m, W = 64, 20, 44, 4, 8, 4, 5
    q, K, V, qi, ki, w, z = _layer(32, n, T, t0, H, d, m, 1000, W)
    c = method.csa_layer(q, K, V, qi, ki, w, z, m=m, top_k=1000, W=W, scale=0.35, t0=t0)
    h = method.hca_layer(q, K, V, z, m_heavy=m, W=W, scale=0.35, t0=t0)
    np.testing.assert_allclose(c["o"], h["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(c["lse"], h["lse"], rtol=1e-13)


def test_no_visible_entry_is_sliding_window_attention():
    n, T, H, d, W = 30, 30, 2, 8, 7
    q, K, V, qi, ki, w, z = _layer(33, n, T, 0, H, d, 4, 5, W)
    res = method.csa_layer(q, K, V, qi, ki, w, z, m=4, top_k=0, W=W, scale=0.4, t0=0)
    t = torch.arange(n)[:, None]
    s = torch.arange(n)[None, :]
    band = (s <= t) & (s > t - W)
    np.testing.assert_allclose(res["o"], _sdpa(q, K, V, 0.4, band), rtol=1e-12, atol=1e-13)
    # HCA with blocks longer than the sequence sees only the window too
    h = method.hca_layer(q, K, V, rnd(34, 64), m_heavy=64, W=W, scale=0.4, t0=0)
    np.testing.assert_allclose(h["o"], res["o"], rtol=1e-12, atol=1e-13)


def test_constant_values_give_constant_output_and_empty_set_gives_zero():
    n, T, H, d = 24, 24, 2, 4
    q, K, _, qi, ki, w, z = _layer(35, n, T, 0, H, d, 4, 3, 0)
    V = np.full((n, d), 1.75)
    res = method.csa_layer(q, K, V, qi, ki, w, z, m=4, top_k=3, W=0, scale=0.5, t0=0)
    # positions 0..2 see nothing (no window, no complete block)
    np.testing.assert_array_equal(res["o"][:3], 0.0)
    assert np.all(np.isneginf(res["lse"][:3]))
    np.testing.assert_allclose(res["o"][3:], 1.75, rtol=1e-14)


def test_attention_skips_invalid_and_invisible_indices():
    n, H, d, W, m = 40, 2, 8, 3, 4
    q, K, V, *_ = _layer(36, n, 1, 0, H, d, m, 0, W)
    kc, vc = K[:10], V[:10]
    t0 = 19  # 5 visible entries
    a = method.csa_attend(q, kc, vc, np.array([[2, -1, 7, 4, 9]]), K, V, 0, t0, W, m, 0.3)
    b = method.csa_attend(q, kc, vc, np.array([[2, 4]]), K, V, 0, t0, W, m, 0.3)
    np.testing.assert_array_equal(a[0], b[0])


def test_attention_matches_brute_force():
    n, T, t0, H, d, m, W, k = 44, 6, 38, 3, 5, 4, 4, 3
    q, K, V, qi, ki, w, z = _layer(37, n, T, t0, H, d, m, k, W)
    res = method.csa_layer(q, K, V, qi, ki, w, z, m=m, top_k=k, W=W, scale=0.45, t0=t0)
    kc = res["k_cmp"]["values"].tolist()
    vc = res["v_cmp"]["values"].tolist()
    for i in range(T):
        bo, bl = brute.csa_query(t0 + i, q[i].tolist(), kc, vc, res["idx"][i].tolist(),
                                 K.tolist(), V.tolist(), W, m, 0.45)
        np.testing.assert_allclose(res["o"][i], bo, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(res["lse"][i], bl, rtol=1e-13)
        # the selected set is the brute-force top-k over visible entries
        c = (t0 + i + 1) // m
        sc = [(j, brute.score(qi[i].tolist(), w[i].tolist(), res["k_idx"]["values"][j].tolist()))
              for j in range(c)]
        assert set(brute.topk(sc, k)) == set(j for j in res["idx"][i] if j >= 0)
    z8 = rnd(39, 8) * 0.5
    h = method.hca_layer(q, K, V, z8, m_heavy=8, W=W, scale=0.45, t0=t0)
    hk = method.store(method.compress_exact(K, z8, 8), "f32")["values"].tolist()
    hv = method.store(method.compress_exact(V, z8, 8), "f32")["values"].tolist()
    for i in range(T):
        bo, bl = brute.hca_query(t0 + i, q[i].tolist(), hk, hv, 8, K.tolist(), V.tolist(), W, 0.45)
        np.testing.assert_allclose(h["o"][i], bo, rtol=1e-12, atol=1e-13)


def test_merge_of_parts_equals_whole():
    rng = np.random.default_rng(38)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((50, 8))
    V = rng.standard_normal((50, 8))
    o, lse = method.attend_entries(q, K, V, 0.3)
    cuts = [0, 7, 7, 30, 50]  # includes an empty part
    parts = [method.attend_entries(q, K[a:b], V[a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
    mo, ml = method.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(mo, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=1e-14)
    eo, el = method.merge_partials(np.zeros((2, 4, 8)), np.full((2, 4), -np.inf))
    assert np.all(eo == 0) and np.all(np.isneginf(el))
