"""Pins for the oracle's top-k softmax routing, by brute force in plain Python."""
import math
import random

import numpy as np

import oracle


def _brute(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]
    ex = [math.exp(float(row[e])) for e in order]
    s = math.fsum(ex)
    return order, [x / s for x in ex]


def test_topk_and_weights_brute_force():
    rng = np.random.default_rng(7)
    for T, E, k in [(5, 8, 2), (9, 4, 2), (33, 128, 8), (7, 256, 8), (3, 3, 3), (4, 1, 1)]:
        logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
        ids, w = oracle.route(logits, k)
        assert ids.dtype == np.int32 and w.dtype == np.float32
        for t in range(T):
            order, ww = _brute(logits[t], k)
            assert ids[t].tolist() == order
            np.testing.assert_allclose(w[t], ww, rtol=2e-7, atol=0)
            assert abs(math.fsum(map(float, w[t])) - 1.0) < 1e-6


def test_ties_break_to_lower_expert():
    logits = np.array([[0.5, 2.0, 0.5, 2.0, 0.5, -1.0]], dtype=np.float32)
    ids, w = oracle.route(logits, 3)
    assert ids.tolist() == [[1, 3, 0]]
    np.testing.assert_allclose(w[0, 0], w[0, 1], rtol=0)
    ids, _ = oracle.route(np.zeros((2, 5), dtype=np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2
    # -0.0 and 0.0 are equal logits: the lower id wins
    ids, _ = oracle.route(np.array([[-0.0, 0.0, -1.0]], dtype=np.float32), 1)
    assert ids.tolist() == [[0]]


def test_renormalisation_drops_other_experts():
    # softmax over all E then renormalising over the selected slots equals a
    # softmax over the selected logits alone: raising an unselected logit
    # (while it stays unselected) leaves the weights unchanged
    rng = random.Random(3)
    base = np.array([[3.0, 1.0, -2.0, -3.0]], dtype=np.float32)
    _, w0 = oracle.route(base, 2)
    for _ in range(5):
        b = base.copy()
        b[0, 2] = rng.uniform(-10, 0.9)
        b[0, 3] = rng.uniform(-10, 0.9)
        ids, w = oracle.route(b, 2)
        assert ids.tolist() == [[0, 1]]
        np.testing.assert_allclose(w, w0, rtol=1e-7)
    np.testing.assert_allclose(w0[0, 0], 1 / (1 + math.exp(-2.0)), rtol=1e-7)


def test_unnormalised_softmax_is_the_full_softmax():
    # scipy's softmax over all E experts, read at the selected slots
    from scipy.special import softmax
    rng = np.random.default_rng(21)
    logits = (rng.standard_normal((11, 40)) * 3).astype(np.float32)
    ids, w = oracle.route(logits, 5, renormalize=False)
    full = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), axis=1), rtol=2e-7)
    assert (w.sum(axis=1) < 1).all()


def test_sigmoid_scores_brute_force():
    rng = np.random.default_rng(22)
    logits = (rng.standard_normal((9, 24)) * 2).astype(np.float32)
    for renorm in (False, True):
        ids, w = oracle.route(logits, 4, scoring="sigmoid", renormalize=renorm)
        for t in range(logits.shape[0]):
            order, _ = _brute(logits[t], 4)
            assert ids[t].tolist() == order
            s = [1.0 / (1.0 + math.exp(-float(logits[t, e]))) for e in order]
            ref = [x / math.fsum(s) for x in s] if renorm else s
            np.testing.assert_allclose(w[t], ref, rtol=2e-7)


def test_bias_shifts_selection_and_scores():
    # the bias is one float32 addition to the logits; a large bias forces its
    # expert into slot 0 and a very negative one keeps it out
    rng = np.random.default_rng(23)
    logits = rng.standard_normal((6, 10)).astype(np.float32)
    bias = np.zeros(10, np.float32)
    bias[7], bias[2] = 50.0, -50.0
    ids, w = oracle.route(logits, 3, bias)
    assert (ids[:, 0] == 7).all() and not (ids == 2).any()
    for t in range(6):
        v = [float(np.float32(logits[t, e]) + np.float32(bias[e])) for e in range(10)]
        order, ww = _brute(np.array(v, np.float32), 3)
        assert ids[t].tolist() == order
        np.testing.assert_allclose(w[t], ww, rtol=2e-7)
    # float32 rounding of the sum decides ties: 1 + 2^-24 rounds to 1, so experts 0 and 1 tie
    ids, _ = oracle.route(np.array([[1.0, 1.0]], np.float32), 1, np.array([0.0, 2.0 ** -24], np.float32))
    assert ids.tolist() == [[0]]
