"""Pins of the oracle's routing, layout, task list and sort/gather.

Routing is checked against a brute-force stable sort, closed forms (all-equal logits,
softcap-inverted logits), scipy's softmax when k = E, and invariants.  Layout is checked
against numpy's histogram and cumulative sum.
"""
import numpy as np
import pytest
import scipy.special

from mixture_experts_layer_softcap_amd import synth


def _bruteforce_topk(logits, k):
    # descending by value, ties by ascending index: a stable sort of the negated logits
    # (+0.0 added so that -0.0 and +0.0 compare equal and keep index order)
    return np.argsort(-(logits + np.float32(0.0)), axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("M,E,k", [(8, 16, 2), (64, 256, 8), (5, 7, 7), (3, 64, 1), (4, 1024, 8)])
def test_route_ids_match_bruteforce_sort(orc, M, E, k):
    g = np.random.default_rng(M * 1000 + E + k)
    logits = g.standard_normal((M, E)).astype(np.float32)
    logits[:, ::5] = np.round(logits[:, ::5], 1)  # plenty of exact ties
    ids, _ = orc.route(logits, k, 30.0)
    np.testing.assert_array_equal(ids, _bruteforce_topk(logits, k))


def test_route_ties_at_the_k_boundary_take_the_lower_index(orc):
    logits = np.zeros((2, 10), np.float32)
    logits[0, [7, 3, 5]] = 1.0      # three-way tie for 2 slots -> experts 3 and 5
    logits[1, [9, 2]] = 2.0
    logits[1, [8, 4, 6]] = 1.0      # tie at the boundary: 4 wins over 6 and 8
    ids, w = orc.route(logits, 2, 30.0)
    assert ids[0].tolist() == [3, 5]
    ids3, _ = orc.route(logits, 3, 30.0)
    assert ids3[1].tolist() == [2, 9, 4]


def test_route_negative_zero_equals_positive_zero(orc):
    logits = np.array([[-1.0, -0.0, 0.0, -2.0]], np.float32)
    ids, w = orc.route(logits, 2, 30.0)
    assert ids[0].tolist() == [1, 2]
    assert w[0].tolist() == [0.5, 0.5]


def test_route_nan_ranks_below_every_number(orc):
    # reading of the pages (silent on non-finite logits): a NaN ranks below -inf and NaNs tie,
    # so they are chosen last, lowest index first.  Brute force: a stable sort on the key
    # (is NaN, -value), with NaN values replaced by 0 so that only the flag orders them.
    g = np.random.default_rng(11)
    logits = g.standard_normal((6, 16)).astype(np.float32)
    logits[0, [2, 9]] = np.nan
    logits[1, :] = np.nan
    logits[2, 3] = -np.inf
    logits[2, [0, 5, 6]] = np.nan
    logits[3, ::2] = np.nan
    logits[4, 1:] = np.nan
    logits[5, 7] = np.inf
    logits[5, 8] = np.nan
    for k in (1, 4, 9, 16):
        ids, _ = orc.route(logits, k, 30.0)
        nan = np.isnan(logits)
        key = np.where(nan, 0.0, -(logits.astype(np.float64) + 0.0))
        ref = np.lexsort((key, nan), axis=1)[:, :k]   # primary: NaN flag, then -value
        np.testing.assert_array_equal(ids, ref)
    ids, _ = orc.route(logits, 2, 30.0)
    assert ids[1].tolist() == [0, 1] and ids[2, 0] != 3 and ids[4].tolist() == [0, 1]


@pytest.mark.parametrize("k", [1, 2, 8])
def test_route_all_equal_logits_give_exact_uniform_weights(orc, k):
    logits = np.full((3, 16), 0.75, np.float32)
    ids, w = orc.route(logits, k, 30.0)
    assert (ids == np.arange(k)[None, :]).all()
    assert (w == np.float32(1.0 / k)).all()


def test_route_ids_do_not_depend_on_the_cap(orc):
    g = np.random.default_rng(7)
    logits = (g.standard_normal((32, 256)) * 40).astype(np.float32)
    a, _ = orc.route(logits, 8, 30.0)
    b, _ = orc.route(logits, 8, 0.0)
    c, _ = orc.route(logits, 8, 5.0)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_route_weights_sum_to_one_and_do_not_increase(orc):
    d = synth.workload_inputs("fused_fp8_M128_E256_k8_K2048_N512", weights=False)
    _, w = orc.route(d["logits"], 8, 30.0)
    assert np.abs(w.astype(np.float64).sum(1) - 1.0).max() < 1e-6
    assert (np.diff(w, axis=1) <= 0).all()


def test_route_full_softmax_when_k_equals_e_and_no_cap(orc):
    g = np.random.default_rng(11)
    logits = (g.standard_normal((6, 12)) * 3).astype(np.float32)
    ids, w = orc.route(logits, 12, 0.0)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, 1), rtol=1e-6)


def test_route_softcap_closed_form(orc):
    # choose logits whose capped values are 2, 1, 0 (l = 30*atanh(c/30)), so the weights are
    # the closed-form softmax of (2, 1, 0); a missing or misplaced cap moves them by >1e-3
    c = np.array([2.0, 1.0, 0.0])
    logits = (30.0 * np.arctanh(c / 30.0)).astype(np.float32)[None, :]
    _, w = orc.route(logits, 3, 30.0)
    z = np.e ** 2 + np.e + 1.0
    np.testing.assert_allclose(w[0], [np.e ** 2 / z, np.e / z, 1.0 / z], rtol=2e-6)
    _, w_nocap = orc.route(logits, 3, 0.0)
    assert abs(float(w_nocap[0, 0]) - np.e ** 2 / z) > 1e-4


def test_route_cap_compresses_large_logits(orc):
    # with cap 30, logits 60 and 0 become 30*tanh(2) = 28.92... and 0
    logits = np.array([[60.0, 0.0]], np.float32)
    _, w = orc.route(logits, 2, 30.0)
    expect = 1.0 / (1.0 + np.exp(-30.0 * np.tanh(2.0)))
    np.testing.assert_allclose(w[0, 0], expect, rtol=1e-7)


@pytest.mark.parametrize("M,E,k", [(8, 16, 2), (128, 256, 8), (1, 4, 4)])
def test_layout_matches_histogram_and_cumsum(orc, M, E, k):
    g = np.random.default_rng(M + E)
    logits = g.standard_normal((M, E)).astype(np.float32)
    ids, _ = orc.route(logits, k, 30.0)
    counts, offsets = orc.layout(ids, E)
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert offsets[0] == 0 and offsets[E] == M * k and counts.sum() == M * k
    assert (np.diff(offsets) >= 0).all()


@pytest.mark.parametrize("chunk", [1, 3, 64])
def test_tasks_cover_every_row_once_per_n_block(orc, chunk):
    counts = np.array([0, 5, 1, 0, 130, 64, 0], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    nb = 3
    t = orc.tasks(counts, offsets, nb, chunk)
    assert len(t) == sum(-(-int(c) // chunk) for c in counts) * nb
    for b in range(nb):
        cover = np.zeros(int(offsets[-1]), np.int32)
        for e, r0, n, blk in t:
            if blk != b:
                continue
            assert 1 <= n <= chunk
            assert offsets[e] <= r0 and r0 + n <= offsets[e + 1]
            cover[r0:r0 + n] += 1
        assert (cover == 1).all()


def test_sort_gather_segments_and_rows(orc):
    M, E, k, K = 16, 8, 3, 256
    g = np.random.default_rng(5)
    ids, _ = orc.route(g.standard_normal((M, E)).astype(np.float32), k, 30.0)
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    q, s = orc.quant_act(x)
    counts, offsets = orc.layout(ids, E)
    sorted_ids, a_q, a_s = orc.sort_gather(ids, offsets, q, s)
    flat = ids.ravel()
    for e in range(E):
        seg = sorted_ids[offsets[e]:offsets[e + 1]]
        np.testing.assert_array_equal(seg, np.nonzero(flat == e)[0])
    for slot, r in enumerate(sorted_ids):
        np.testing.assert_array_equal(a_q[slot], q[r // k])
        np.testing.assert_array_equal(a_s[:, slot], s[r // k])
