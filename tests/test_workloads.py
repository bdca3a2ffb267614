"""The workload registry against the constants the pages print (tests/golden/page_constants.json)."""
import json
import os

import inputgen
from oracle import method

with open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")) as _f:
    G = json.load(_f)


def v(key):
    return G[key]["value"]


def test_registry_uses_page_constants():
    W = inputgen.WORKLOADS
    for name in ("csa_decode_flash_128k", "csa_decode_pro_1m", "csa_prefill_chunk_1m"):
        assert W[name].m == v("csa_block_m") and W[name].W == v("window_n_win")
    assert W["csa_decode_flash_128k"].k == v("csa_topk_flash")
    assert W["csa_decode_pro_1m"].k == W["csa_prefill_chunk_1m"].k == v("csa_topk_pro")
    assert W["hca_decode_1m"].m_heavy == v("hca_block_m_heavy")
    assert W["csa_decode_pro_1m"].n == W["hca_decode_1m"].n == v("context_1m_tokens")


def test_closed_form_counts():
    wl = inputgen.WORKLOADS["csa_decode_pro_1m"]
    assert wl.k * wl.m == v("fine_tokens_seen_by_pro_csa")
    h = inputgen.WORKLOADS["hca_decode_1m"]
    assert method.visible_entries(h.t0, h.m_heavy) == h.N_h == v("hca_entries_at_1m")
    p = inputgen.WORKLOADS["csa_prefill_chunk_1m"]
    assert p.t0 + p.T == p.n and p.cmp_begin * p.m == p.t0
    # the last chunk query sees every entry; the first sees those completed before it
    assert method.visible_entries(p.t0 + p.T - 1, p.m) == p.N_c
    assert method.visible_entries(p.t0, p.m) == 260096


def test_generator_is_seeded_and_chunk_local():
    a = inputgen.normal("x", (2, 70000, 3), seed=5)
    b = inputgen.normal("x", (2, 70000, 3), seed=5)
    c = inputgen.normal("x", (2, 70000, 3), seed=6)
    assert (a == b).all() and not (a == c).all()
    # rows of the second chunk do not depend on the tensor length
    d = inputgen.normal("x", (2, 140000, 3), seed=5)
    assert (d[:, :70000] == a).all()
    z = inputgen.normal("z_csa", (4,), seed=0, std=0.5)
    assert z.shape == (4,) and float(z.abs().max()) < 5
