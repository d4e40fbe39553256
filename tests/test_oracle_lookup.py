"""Pins for the oracle's lookup drafting: hand-worked examples, and an
independent formulation (for n from n_max down to n_min, the latest start p
with h[p:p+n] == the last n tokens and a token after it) on random short
histories with a small vocabulary, where matches of every length occur."""
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_examples(orc):
    n = 0
    with open(os.path.join(GOLDEN, "lookup_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            p = [x.split() for x in line.split("|")]
            n_min, n_max, k = (int(x) for x in p[0])
            h = np.array([int(x) for x in p[1]], dtype=np.int32)
            want = [int(x) for x in p[2]]
            count, match, pos = (int(x) for x in p[3])
            r = orc.lookup_draft(h[None], [len(h)], n_min, n_max, k)
            assert list(r["tokens"][0]) == want, line
            assert (r["count"][0], r["match"][0], r["pos"][0]) == (count, match, pos), line
            n += 1
    assert n == 5


def _by_length(h, n_min, n_max, k):
    N = len(h)
    for n in range(n_max, n_min - 1, -1):
        if n > N - 1:
            continue
        tail = list(h[N - n:])
        for p in range(N - 1 - n, -1, -1):          # p + n <= N - 1
            if list(h[p:p + n]) == tail:
                e = p + n - 1
                c = min(k, N - 1 - e)
                return list(h[e + 1:e + 1 + c]) + [-1] * (k - c), c, n, e
    return [-1] * k, 0, 0, -1


def test_matches_the_by_length_formulation():
    import oracle as orc
    rng = np.random.default_rng(51)
    for trial in range(3000):
        N = int(rng.integers(0, 40))
        vocab = int(rng.integers(1, 4))
        n_min = int(rng.integers(1, 5))
        n_max = int(rng.integers(n_min, 9))
        k = int(rng.integers(0, 6))
        h = rng.integers(0, vocab, size=N).astype(np.int32)
        stride = N + int(rng.integers(0, 3))
        row = np.full((1, stride), 77, dtype=np.int32)
        row[0, :N] = h
        r = orc.lookup_draft(row, [N], n_min, n_max, k)
        tok, c, m, e = _by_length(h, n_min, n_max, k)
        assert list(r["tokens"][0]) == tok
        assert (r["count"][0], r["match"][0], r["pos"][0]) == (c, m, e), (h, n_min, n_max, k)


def test_batch_rows_are_independent_and_lengths_clamp(orc):
    rng = np.random.default_rng(52)
    B, stride = 6, 200
    hist = np.stack([synth.make_lookup_history(rng, stride, 5, 10) for _ in range(B)])
    lengths = np.array([200, 150, 0, 1, 250, -3], dtype=np.int32)
    r = orc.lookup_draft(hist, lengths, 6, 12, 8)
    for b in range(B):
        N = min(max(int(lengths[b]), 0), stride)
        one = orc.lookup_draft(hist[b:b + 1, :N] if N else np.zeros((1, 1), np.int32), [N], 6, 12, 8)
        for key in ("tokens", "count", "match", "pos"):
            assert np.array_equal(r[key][b], one[key][0])


def test_planted_copy_is_found():
    import oracle as orc
    rng = np.random.default_rng(53)
    for trial in range(20):
        N = 5000
        h = synth.make_lookup_history(rng, N, 151936, 12)
        r = orc.lookup_draft(h[None], [N], 6, 12, 8)
        assert r["match"][0] == 12
        e = int(r["pos"][0])
        assert np.array_equal(h[e - 11:e + 1], h[N - 12:])
        assert list(r["tokens"][0][:r["count"][0]]) == list(h[e + 1:e + 1 + r["count"][0]])
