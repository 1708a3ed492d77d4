"""Pins of the oracle's routing and token sort: brute force, closed forms,
invariants and a hand-worked sort example."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- routing
def _brute_route(logits, k, score):
    T, E = logits.shape
    ids = np.empty((T, k), np.int64)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        sel = order[:k]
        l64 = logits[t].astype(np.float64)
        if score == "softmax":
            p = np.exp(l64 - l64.max())
            p /= p.sum()
        else:
            p = 1.0 / (1.0 + np.exp(-l64))
        ids[t] = sel
        w[t] = p[sel] / p[sel].sum()
    return ids, w


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 4, 2), (33, 8, 2), (16, 64, 8), (5, 256, 8),
                                   (3, 300, 6), (4, 5, 5)])
def test_route_brute_force(score, T, E, k):
    rng = np.random.default_rng(T * 1000 + E * 10 + k)
    logits = rng.standard_normal((T, E)).astype(np.float32) * 2
    ids, w = oracle.route(logits, k, score)
    bids, bw = _brute_route(logits, k, score)
    assert np.array_equal(ids, bids)
    assert np.allclose(w, bw, rtol=2e-6, atol=0)
    # invariants
    for t in range(T):
        assert len(set(ids[t])) == k and ids[t].min() >= 0 and ids[t].max() < E
    assert np.all(w > 0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 4 * k * 2.0 ** -24)


def test_route_ties_pick_lower_expert_and_raw_logit_order():
    # equal logits: the smaller expert index wins; sigmoid saturates to 1.0f for
    # both 30 and 40, but selection is on the raw logit.
    logits = np.array([[1.0, 3.0, 3.0, 0.5], [30.0, 40.0, -1.0, 40.0]], np.float32)
    ids, w = oracle.route(logits, 2, "sigmoid")
    assert ids.tolist() == [[1, 2], [1, 3]]
    assert w[1, 0] == w[1, 1] == np.float32(0.5)


def test_route_closed_forms():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((9, 8)).astype(np.float32)
    ids, w = oracle.route(logits, 2, "softmax")
    for t in range(9):
        a, b = ids[t]
        assert math.isclose(w[t, 0] / w[t, 1], math.exp(logits[t, a] - logits[t, b]), rel_tol=1e-5)
    # k = E: plain softmax, listed in descending order
    ids, w = oracle.route(logits, 8, "softmax")
    for t in range(9):
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[ids[t]], rtol=1e-5)
        assert np.all(np.diff(logits[t][ids[t]]) <= 0)
    # E = 1: weight 1 for everything
    ids, w = oracle.route(rng.standard_normal((4, 1)).astype(np.float32), 1, "sigmoid")
    assert np.all(ids == 0) and np.all(w == 1.0)
    # no renormalisation: the raw scores
    ids, w = oracle.route(logits, 2, "sigmoid", renorm=False)
    assert np.allclose(w, 1 / (1 + np.exp(-np.take_along_axis(logits, ids, 1).astype(np.float64))),
                       rtol=1e-6)


# -------------------------------------------------------------------- sort
def check_sort_invariants(ids, w, E, B, s):
    """Every property the sort's definition fixes; raises AssertionError."""
    T, k = ids.shape
    N = T * k
    flat, wflat = ids.ravel(), w.ravel()
    P, NB = N + E * B - k, -(-(N + E * B - k) // B)
    assert s["sorted_ids"].shape == (P,) and s["sorted_w"].shape == (P,)
    assert s["sorted_expert_ids"].shape == (NB,)
    cnt, off, nv = s["expert_counts"], s["expert_offsets"], int(s["num_valid"][0])
    assert np.array_equal(cnt, np.bincount(flat, minlength=E)) and cnt.sum() == N
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[E] == nv and nv <= P
    pad = np.diff(off)
    assert np.all(pad % B == 0) and np.array_equal(pad, -(-cnt // B) * B)
    real = s["sorted_ids"][s["sorted_ids"] != N]
    assert np.array_equal(np.sort(real), np.arange(N))  # a permutation of 0..N-1
    for e in range(E):
        seg = s["sorted_ids"][off[e]:off[e + 1]]
        r = seg[:cnt[e]]
        assert np.all(flat[r] == e) and np.all(np.diff(r) > 0)  # stable
        assert np.all(seg[cnt[e]:] == N)
        assert np.all(s["sorted_expert_ids"][off[e] // B:off[e + 1] // B] == e)
    assert np.all(s["sorted_ids"][nv:] == N) and np.all(s["sorted_w"][nv:] == 0)
    assert np.all(s["sorted_expert_ids"][nv // B:] == -1)
    m = s["sorted_ids"] != N
    assert np.array_equal(s["sorted_w"][m], wflat[s["sorted_ids"][m]])
    assert np.all(s["sorted_w"][~m] == 0)


def _brute_sort(ids, w, E, B):
    T, k = ids.shape
    N = T * k
    flat = ids.ravel()
    order = sorted(range(N), key=lambda a: (flat[a], a))
    P = N + E * B - k
    NB = -(-P // B)
    sid, sw, seid = [], [], []
    for e in range(E):
        mine = [a for a in order if flat[a] == e]
        nblk = -(-len(mine) // B)
        mine += [N] * (nblk * B - len(mine))
        sid += mine
        seid += [e] * nblk
    sw = [float(w.ravel()[a]) if a != N else 0.0 for a in sid]
    sid += [N] * (P - len(sid))
    sw += [0.0] * (P - len(sw))
    seid += [-1] * (NB - len(seid))
    return np.array(sid, np.int32), np.array(sw, np.float32), np.array(seid, np.int32)


def test_sort_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "sort_worked_example.json")))
    ids = np.array(g["topk_ids"], np.int32)
    w = (np.arange(ids.size, dtype=np.float32) + 1) / 8
    w = w.reshape(ids.shape)
    s = oracle.sort(ids, w, g["E"], g["B"])
    assert oracle.max_padded(g["T"], g["k"], g["E"], g["B"]) == g["P"]
    assert oracle.max_blocks(g["T"], g["k"], g["E"], g["B"]) == g["NB"]
    assert s["sorted_ids"].tolist() == g["sorted_ids"]
    assert s["sorted_expert_ids"].tolist() == g["sorted_expert_ids"]
    assert s["expert_counts"].tolist() == g["expert_counts"]
    assert s["expert_offsets"].tolist() == g["expert_offsets"]
    assert int(s["num_valid"][0]) == g["num_valid"]
    exp_w = [0.0 if i < 0 else float(w.ravel()[i]) for i in g["sorted_w_index"]]
    assert s["sorted_w"].tolist() == exp_w
    check_sort_invariants(ids, w, g["E"], g["B"], s)


@pytest.mark.parametrize("seed", range(40))
def test_sort_brute_force_fuzz(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(0, 60))
    B = int(rng.choice([1, 2, 3, 16, 32, 64, 128]))
    skew = rng.random() < 0.5
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        p = (1.0 / np.arange(1, E + 1) ** 1.5) if skew else np.ones(E)
        ids[t] = rng.choice(E, size=k, replace=False, p=p / p.sum())
    w = rng.random((T, k)).astype(np.float32)
    s = oracle.sort(ids, w, E, B)
    sid, sw, seid = _brute_sort(ids, w, E, B)
    assert np.array_equal(s["sorted_ids"], sid)
    assert np.array_equal(s["sorted_w"], sw)
    assert np.array_equal(s["sorted_expert_ids"], seid)
    check_sort_invariants(ids, w, E, B, s)


def test_sort_invariant_checker_catches_corruption():
    rng = np.random.default_rng(9)
    ids = np.stack([rng.choice(6, 2, replace=False) for _ in range(20)]).astype(np.int32)
    w = rng.random((20, 2)).astype(np.float32)
    good = oracle.sort(ids, w, 6, 4)
    check_sort_invariants(ids, w, 6, 4, good)

    def mutated(key, fn):
        s = {k: v.copy() for k, v in good.items()}
        fn(s[key])
        return s

    nv = int(good["num_valid"][0])
    first_e = int(np.argmax(good["expert_counts"] > 1))
    o = good["expert_offsets"][first_e]
    mutations = [
        ("sorted_ids", lambda a: a.__setitem__(slice(o, o + 2), a[o:o + 2][::-1].copy())),  # unstable
        ("sorted_ids", lambda a: a.__setitem__(nv, 0)),                                      # tail
        ("sorted_w", lambda a: a.__setitem__(0, a[0] + 1)),
        ("sorted_expert_ids", lambda a: a.__setitem__(0, a[0] + 1)),
        ("expert_counts", lambda a: a.__setitem__(0, a[0] + 1)),
        ("expert_offsets", lambda a: a.__setitem__(1, a[1] + 1)),
        ("num_valid", lambda a: a.__setitem__(0, a[0] + 4)),
    ]
    for key, fn in mutations:
        with pytest.raises(AssertionError):
            check_sort_invariants(ids, w, 6, 4, mutated(key, fn))


def test_sizing_formula_values():
    """max_num_tokens_padded = T*k + E*B - k and max_num_m_blocks = ceil(P / B)
    (AITER article, section 3.1), at the five workloads' shapes."""
    cases = [((16, 2, 4, 32), 158, 5), ((32, 2, 8, 32), 318, 10), ((4096, 2, 8, 128), 9214, 72),
             ((512, 2, 8, 128), 2046, 16), ((128, 8, 256, 128), 33784, 264),
             ((128, 8, 256, 32), 9208, 288)]
    for (T, k, E, B), P, NB in cases:
        assert oracle.max_padded(T, k, E, B) == P
        assert oracle.max_blocks(T, k, E, B) == NB
    # the bound holds for any routing: num_valid <= P whenever k <= E
    rng = np.random.default_rng(11)
    for _ in range(200):
        E = int(rng.integers(1, 20))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 10))
        B = int(rng.integers(1, 9))
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        s = oracle.sort(ids, np.ones((T, k), np.float32), E, B)
        assert int(s["num_valid"][0]) <= oracle.max_padded(T, k, E, B)


def test_sort_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.sort(np.array([[0, 4]], np.int32), np.ones((1, 2), np.float32), 4, 2)
