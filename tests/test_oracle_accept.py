"""Pins for the oracle's greedy tree acceptance and accepted-path KV commit.

Acceptance is pinned by hand-worked examples, by a brute force that walks
parent pointers over every root path (the oracle reads ancestor masks), over
all 5,040 eight-row tree shapes, and by the chain special case.  The commit
is pinned element by element through an independent reader of the layouts,
and by row independence: after the commit, the chain of committed rows over
the compacted cache attends exactly like the committed tree rows did over
the uncompacted one.
"""
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _examples():
    with open(os.path.join(GOLDEN, "accept_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = [p.split() for p in line.split("|")]
            parents = np.array([int(x) for x in parts[0]])
            draft = np.array([int(x) for x in parts[1]], dtype=np.int32)
            target = np.array([int(x) for x in parts[2]], dtype=np.int32)
            path = [int(x) for x in parts[3]]
            yield parents, draft, target, path, int(parts[4][0])


def test_worked_examples(orc):
    n_cases = 0
    for parents, draft, target, path, bonus in _examples():
        n, got, b = orc.tree_accept(synth.ancestor_masks(parents), draft, target)
        assert n == len(path)
        assert list(got[:n]) == path
        assert np.all(got[n:] == -1)
        assert b == bonus
        n_cases += 1
    assert n_cases == 5


def _brute(parents, draft, target):
    """Every root path from node 0, by parent pointers; deepest matching
    path, lowest end node among equals."""
    T = len(parents)
    best = (1, 0)                       # (depth, end node)
    for end in range(T):
        path = []
        v = end
        while v >= 0:
            path.append(v)
            v = parents[v]
        path.reverse()
        if path[0] != 0:
            continue
        if all(draft[path[k]] == target[path[k - 1]] for k in range(1, len(path))):
            if len(path) > best[0]:
                best = (len(path), end)
    end = best[1]
    path = []
    v = end
    while v >= 0:
        path.append(v)
        v = parents[v]
    return path[::-1], int(target[end])


def test_matches_brute_force_on_every_8_row_shape(orc):
    rng = np.random.default_rng(11)
    lengths = np.zeros(9, dtype=int)
    for parents in synth.all_tree_shapes(8):
        draft, target = synth.make_tree_tokens(rng, parents, vocab=3)
        n, got, b = orc.tree_accept(synth.ancestor_masks(parents), draft, target)
        want, wb = _brute(parents, draft, target)
        assert list(got[:n]) == want and b == wb, (parents, draft, target)
        lengths[n] += 1
    # the inputs exercise short and long commits alike
    assert lengths[1] > 0 and lengths[4:].sum() > 100


def test_matches_brute_force_on_64_node_trees_and_forests(orc):
    rng = np.random.default_rng(12)
    for trial in range(300):
        T = int(rng.integers(1, 65))
        parents = synth.make_tree_parents(rng, T, int(rng.integers(2, 10)))
        if trial % 3 == 0 and T > 2:                  # detach a subtree: a forest
            parents = parents.copy()
            parents[int(rng.integers(1, T))] = -1
        draft, target = synth.make_tree_tokens(rng, parents, vocab=int(rng.integers(2, 6)))
        n, got, b = orc.tree_accept(synth.ancestor_masks(parents), draft, target)
        want, wb = _brute(parents, draft, target)
        assert list(got[:n]) == want and b == wb


def test_chain_commits_the_longest_matching_prefix(orc):
    rng = np.random.default_rng(13)
    for trial in range(200):
        T = int(rng.integers(1, 65))
        draft = rng.integers(0, 4, size=T).astype(np.int32)
        target = rng.integers(0, 4, size=T).astype(np.int32)
        k = 1
        while k < T and draft[k] == target[k - 1]:
            k += 1
        n, got, b = orc.tree_accept(synth.ancestor_masks(synth.chain_parents(T)), draft, target)
        assert n == k and list(got[:n]) == list(range(k)) and b == target[k - 1]


# ------------------------------------------------------------- commit

def _k_block(kv, g, pos, b):
    return kv.k_codes[g, pos, b].copy(), int(kv.k_scales[g, pos, b])


def _v_codes(orc, kv, g, pos):
    grp, e = divmod(pos, 32)
    return [orc.code_get(kv.v_codes[g, grp, d], e) for d in range(kv.head_dim)]


def _v_scales(kv, g, pos):
    grp, e = divmod(pos, 32)
    return [int(kv.v_scales[g, grp, b, e]) for b in range(kv.head_dim // 32)]


@pytest.mark.parametrize("L,T,seed", [(0, 8, 1), (29, 8, 2), (61, 17, 3), (100, 64, 4)])
def test_commit_moves_exactly_the_committed_tokens(orc, L, T, seed):
    rng = np.random.default_rng(seed)
    hkv, d = 2, 64
    cap = L + T + 5
    kv = synth.make_kv(rng, hkv, d, L + T, cap)
    before = synth.KVCache(kv.k_codes.copy(), kv.k_scales.copy(), kv.v_codes.copy(),
                           kv.v_scales.copy(), hkv, d, cap, kv.n_filled)
    parents = synth.make_tree_parents(rng, T, 8)
    draft, target = synth.make_tree_tokens(rng, parents, vocab=2, p_follow=0.9)
    n, path, _ = orc.tree_accept(synth.ancestor_masks(parents), draft, target)
    orc.kv_commit(kv, L, T, path, n)
    for g in range(hkv):
        for pos in range(cap):
            src = L + int(path[pos - L]) if L <= pos < L + n else pos
            for b in range(d // 32):
                w0, s0 = _k_block(before, g, src, b)
                w1, s1 = _k_block(kv, g, pos, b)
                assert np.array_equal(w0, w1) and s0 == s1
            assert _v_codes(orc, kv, g, pos) == _v_codes(orc, before, g, src)
            assert _v_scales(kv, g, pos) == _v_scales(before, g, src)


def test_commit_then_chain_equals_tree_rows(orc):
    """Row independence: the committed tree rows attend over the uncompacted
    cache exactly as the chain of those rows attends over the compacted one."""
    rng = np.random.default_rng(21)
    hq, hkv, d, L, T = 4, 2, 64, 70, 12
    kv = synth.make_kv(rng, hkv, d, L + T, L + T + 3)
    q = synth.make_q(rng, T, hq, d)
    parents = synth.make_tree_parents(rng, T, 6)
    mask = synth.ancestor_masks(parents)
    draft, target = synth.make_tree_tokens(rng, parents, vocab=2, p_follow=0.95)
    n, path, _ = orc.tree_accept(mask, draft, target)
    assert n >= 3
    tree = orc.attention(q, kv, L, mask, 0.125)
    orc.kv_commit(kv, L, T, path, n)
    # the chain: row j is committed node path[j]; rows past n are unused
    qc = np.zeros_like(q)
    qc[:n] = q[path[:n]]
    chain = orc.attention(qc[:n], kv, L, synth.ancestor_masks(synth.chain_parents(n)), 0.125)
    for j in range(n):
        for h in range(hq):
            a = tree["out"][path[j] * hq + h]
            c = chain["out"][j * hq + h]
            assert np.array_equal(a, c)
            assert tree["lse"][path[j] * hq + h] == chain["lse"][j * hq + h]


def test_commit_rejects_bad_paths(orc):
    rng = np.random.default_rng(5)
    kv = synth.make_kv(rng, 1, 64, 40, 40)
    with pytest.raises(ValueError):
        orc.kv_commit(kv, 30, 10, np.array([0, 10] + [-1] * 8, dtype=np.int32), 2)
    with pytest.raises(ValueError):
        orc.kv_commit(kv, 31, 10, np.arange(10, dtype=np.int32), 3)     # L + T > cap
