"""Pins of the oracle's CSA2 hierarchical indexer (CPU only): block scores by hand and by
brute force, the candidate pool's content and order, and the two selections the pages'
design rests on: a pool covering every block reproduces the full top-k, and a Reindex with
the Full layer's own query reproduces the Full layer's top-k whenever the pool holds at
least k blocks (every top-k position's block outscores all but fewer than k blocks)."""

import itertools

import numpy as np

from oracle import csa_oracle as O


def test_block_scores_hand_case():
    s = np.array([1.0, 5.0, 2.0, -np.inf, 3.0, 3.0, 0.0, 0.0, -np.inf, -np.inf])
    assert np.array_equal(O.block_scores(s, 4), [5.0, 3.0, -np.inf])
    blocks, pool = O.candidate_pool(s, 4, 1)
    assert np.array_equal(blocks, [0])
    assert np.array_equal(pool, [0, 1, 2, -1])                 # position 3 is not a candidate
    blocks, pool = O.candidate_pool(s, 4, 3)                   # the empty block is never chosen
    assert np.array_equal(blocks, [0, 1, -1])
    assert np.array_equal(pool, [0, 1, 2, 4, 5, 6, 7] + [-1] * 5)


def test_block_choice_brute_force_with_ties():
    # every small row of few distinct values: the chosen blocks are the n best by (max, index)
    rng = np.random.default_rng(40)
    for _ in range(200):
        n = int(rng.integers(1, 30))
        s = rng.integers(0, 4, n).astype(float)
        s[rng.random(n) < 0.2] = -np.inf
        nbk = int(rng.integers(1, 5))
        blocks, _ = O.candidate_pool(s, 3, nbk)
        bmax = [max(s[3 * j:3 * j + 3]) for j in range(-(-n // 3))]
        order = sorted((j for j in range(len(bmax)) if bmax[j] > -np.inf), key=lambda j: (-bmax[j], j))
        want = sorted(order[:nbk]) + [-1] * (nbk - len(order[:nbk]))
        assert list(blocks) == want


def test_pool_covering_every_block_reproduces_the_full_topk():
    rng = np.random.default_rng(41)
    B, S, N, H, d, k, m = 2, 2, 200, 4, 16, 12, 4
    qI, w = rng.normal(size=(B, S, H, d)), rng.normal(size=(B, S, H))
    KI = rng.normal(size=(B, N, d))
    q_pos = np.array([[4 * N - 2, 4 * N - 1], [4 * 150, 4 * 150 + 3]])
    full = O.index_scores(qI, w, KI, q_pos, m)
    _, pool = O.candidate_pool(full, 8, -(-N // 8))
    assert np.array_equal(O.reindex_topk(qI, w, KI, pool, q_pos, m, k), O.topk_indices(full, k))


def test_reindex_with_the_full_query_keeps_the_full_topk():
    rng = np.random.default_rng(42)
    B, S, N, H, d, m = 3, 1, 4096, 4, 16, 4
    for k in (8, 32, 64):
        qI, w = rng.normal(size=(B, S, H, d)), np.abs(rng.normal(size=(B, S, H)))
        KI = rng.normal(size=(B, N, d))
        q_pos = np.full((B, S), 4 * N - 1)
        full = O.index_scores(qI, w, KI, q_pos, m)
        _, pool = O.candidate_pool(full, 8, k)                 # exactly k blocks: the tight case
        assert np.array_equal(O.reindex_topk(qI, w, KI, pool, q_pos, m, k), O.topk_indices(full, k))


def test_reindex_is_the_topk_over_the_pool_positions():
    # another query over the same pool: brute force over the pool's positions
    rng = np.random.default_rng(43)
    B, S, N, H, d, m, k = 1, 1, 300, 3, 8, 4, 10
    KI = rng.normal(size=(B, N, d))
    q1, w1 = rng.normal(size=(B, S, H, d)), rng.normal(size=(B, S, H))
    q2, w2 = rng.normal(size=(B, S, H, d)), rng.normal(size=(B, S, H))
    q_pos = np.array([[4 * 280 + 1]])                          # the last 20 entries are not visible yet
    _, pool = O.candidate_pool(O.index_scores(q1, w1, KI, q_pos, m), 8, 6)
    got = O.reindex_topk(q2, w2, KI, pool, q_pos, m, k)[0, 0]
    cands = [int(p) for p in pool[0, 0] if p >= 0]
    assert max(cands) < 280
    sc = {p: float(np.dot(w2[0, 0], np.maximum(q2[0, 0] @ KI[0, p], 0.0))) for p in cands}
    best = sorted(sorted(cands, key=lambda p: (-sc[p], p))[:k])
    assert list(got[:len(best)]) == best and np.all(got[len(best):] == -1)
