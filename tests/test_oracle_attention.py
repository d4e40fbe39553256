"""Pins for the oracle's attention and merge.

What pins what:
  * integer logits  -- numpy int64 contraction of the unpacked codes;
  * whole attention -- brute-force fp64 attention over the dequantized
    matrices (Q^ = sq*q8, K^ = sk*(c-4), V^ = sv*(c-4)), a different
    formulation (dense matrix products instead of per-block integer sums);
  * int8 Q rounding -- the same brute force on the raw fp32 Q agrees within
    the bound the rounding allows;
  * row independence (elpis-lossless, "Lossless" and "Trust base"): every
    row of every one of the 5,040 8-row tree shapes ("Proofs and tests")
    equals, bit for bit, the chain computation of its root-to-node path;
  * a single chain equals the causal chunk rule, bit for bit;
  * closed forms: an all-zero Q row averages the visible V^ rows; a planted
    dominant key returns its V^ row;
  * split-K with a log-sum-exp merge (elpis "Why fast": split-K and the
    merge) equals the unsplit call over any partition.
"""
import numpy as np
import pytest

import synth


def _cache(seed, hkv, d, n, cap=None):
    return synth.make_kv(np.random.default_rng(seed), hkv, d, n, cap)


def _dequant(orc, codes, scales, n):
    """K (token-major) values [Hkv][n][D] in fp64."""
    c = orc.unpack_codes(codes[:, :n]).astype(np.float64)             # [Hkv][n][D]
    s = np.vectorize(orc.f16_bits_to_f64)(scales[:, :n].astype(np.int64))  # [Hkv][n][NB]
    return np.repeat(s, 32, axis=-1) * (c - 4.0)


def _dequant_v(orc, kv, n):
    """V (key-transposed groups of 32 keys) values [Hkv][n][D] in fp64."""
    hkv, ng, d, _ = kv.v_codes.shape
    c = orc.unpack_codes(kv.v_codes.reshape(hkv, ng, d, 1, 3)).astype(np.float64)  # [Hkv][ng][D][32]
    c = c.transpose(0, 1, 3, 2).reshape(hkv, ng * 32, d)[:, :n]
    s = np.vectorize(orc.f16_bits_to_f64)(kv.v_scales.astype(np.int64))           # [Hkv][ng][NB][32]
    s = s.transpose(0, 1, 3, 2).reshape(hkv, ng * 32, d // 32)[:, :n]
    return np.repeat(s, 32, axis=-1) * (c - 4.0)


def _visible(T, L, mask):
    n = L + T
    vis = np.zeros((T, n), dtype=bool)
    vis[:, :L] = True
    for t in range(T):
        for a in range(T):
            if mask is None:
                vis[t, L + a] = a <= t
            else:
                vis[t, L + a] = bool((int(mask[t]) >> a) & 1)
    return vis


def _brute(orc, q, kv, L, mask, scale, quantize=True):
    T, hq, d = q.shape
    G = hq // kv.n_kv_heads
    n = L + T
    K = _dequant(orc, kv.k_codes, kv.k_scales, n)
    V = _dequant_v(orc, kv, n)
    vis = _visible(T, L, mask)
    out = np.zeros((T, hq, d))
    lse = np.zeros((T, hq))
    for t in range(T):
        for h in range(hq):
            if quantize:
                qi, sq = orc.quantize_q_row(q[t, h])
                qh = float(sq) * qi.astype(np.float64)
            else:
                qh = q[t, h].astype(np.float64)
            x = scale * (K[h // G] @ qh)
            x = np.where(vis[t], x, -np.inf)
            m = x.max()
            p = np.exp(x - m)
            out[t, h] = (p @ V[h // G]) / p.sum()
            lse[t, h] = m + np.log(p.sum())
    return out.reshape(T * hq, d), lse.reshape(-1)


CASES = [
    # (name, Hq, Hkv, D, L, T, kind, seed)
    ("tiny", 4, 1, 64, 512, 8, "chain", 0),
    ("gqa_tree", 4, 2, 64, 45, 7, "tree", 21),
    ("gqa_prefill", 6, 2, 96, 33, 9, "prefill", 22),
]


@pytest.mark.parametrize("name,hq,hkv,d,L,T,kind,seed", CASES)
def test_oracle_matches_brute_force(orc, name, hq, hkv, d, L, T, kind, seed):
    rng = np.random.default_rng(seed)
    kv = synth.make_kv(rng, hkv, d, L + T, L + T + 5)
    q = synth.make_q(rng, T, hq, d)
    if kind == "tree":
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 4))
    elif kind == "chain":
        mask = synth.ancestor_masks(synth.chain_parents(T))
    else:
        mask = None
    scale = 1.0 / np.sqrt(d)
    res = orc.attention(q, kv, L, mask, scale, want_logits=True)
    out_b, lse_b = _brute(orc, q, kv, L, mask, scale)
    assert np.max(np.abs(res["out"] - out_b)) <= 1e-12 * np.max(np.abs(out_b))
    assert np.max(np.abs(res["lse"] - lse_b)) <= 1e-12 * np.max(np.abs(lse_b))

    # integer logits: exact int64 contraction of q8 with (code - 4) per block
    kcode = orc.unpack_codes(kv.k_codes[:, :L + T]).astype(np.int64) - 4
    G = hq // hkv
    for r in range(T * hq):
        t, h = divmod(r, hq)
        qi = res["qi8"][r].astype(np.int64)
        blocks = (kcode[h // G] * qi[None, :]).reshape(L + T, d // 32, 32).sum(-1)
        assert np.array_equal(res["logits"][r], blocks)

    # raw fp32 Q: the int8 rounding moves each logit by at most
    # scale * (sq/2) * ||k^||_1, so the output moves by at most
    # (exp(2 * max dx) - 1) * max|v^|.
    out_raw, _ = _brute(orc, q, kv, L, mask, scale, quantize=False)
    K = _dequant(orc, kv.k_codes, kv.k_scales, L + T)
    V = _dequant_v(orc, kv, L + T)
    for r in range(T * hq):
        t, h = divmod(r, hq)
        dx = scale * float(res["sq"][r]) / 2 * np.abs(K[h // G]).sum(-1).max()
        bound = (np.exp(2 * dx) - 1) * np.abs(V[h // G]).max()
        assert np.max(np.abs(res["out"][r] - out_raw[r])) <= bound * (1 + 1e-9)


def test_every_8_row_tree_equals_its_chains(orc):
    """All 7! = 5,040 parent arrays of the 8-row tree: each row must equal
    the causal computation of its root-to-node path, bit for bit.  The tree
    rows' K/V enter both caches through the oracle's own quantizer, at L + a
    in the tree cache and at L + m (m = position on the path) in a chain's."""
    hq, hkv, d, L, T = 2, 1, 32, 24, 8
    rng = np.random.default_rng(11)
    base = synth.make_kv(rng, hkv, d, L, L + T)
    q = synth.make_q(rng, T, hq, d)
    knew = synth.make_new_rows(rng, T, hkv, d)
    vnew = synth.make_new_rows(rng, T, hkv, d)
    scale = 1.0 / np.sqrt(d)

    def cache_with(rows):
        c = synth.KVCache(base.k_codes.copy(), base.k_scales.copy(), base.v_codes.copy(),
                          base.v_scales.copy(), hkv, d, L + T, L + len(rows))
        orc.kv_quant_pack(knew[rows], L, c.k_codes, c.k_scales, "k")
        orc.kv_quant_pack(vnew[rows], L, c.v_codes, c.v_scales, "v")
        return c

    kv = cache_with(list(range(T)))
    chain_cache = {}

    def chain(path):
        key = tuple(path)
        if key not in chain_cache:
            k = len(path)
            ckv = cache_with(list(path))
            cq = q[list(path)]
            rows = [(k - 1) * hq + h for h in range(hq)]
            res = orc.attention(cq, ckv, L, None, scale, rows=rows)
            chain_cache[key] = (res["out"], res["lse"])
        return chain_cache[key]

    n_shapes = 0
    for parent in synth.all_tree_shapes(T):
        mask = synth.ancestor_masks(parent)
        res = orc.attention(q, kv, L, mask, scale)
        for i in range(T):
            path = [a for a in range(T) if (int(mask[i]) >> a) & 1]
            o, l = chain(path)
            assert np.array_equal(res["out"][i * hq:(i + 1) * hq], o)
            assert np.array_equal(res["lse"][i * hq:(i + 1) * hq], l)
        n_shapes += 1
    assert n_shapes == 5040
    assert len(chain_cache) == 128      # every root-to-node path of 8 nodes


def test_chain_tree_equals_causal_and_single_row(orc):
    rng = np.random.default_rng(12)
    hq, hkv, d, L, T = 4, 2, 64, 70, 13
    kv = synth.make_kv(rng, hkv, d, L + T)
    q = synth.make_q(rng, T, hq, d)
    a = orc.attention(q, kv, L, synth.ancestor_masks(synth.chain_parents(T)))
    b = orc.attention(q, kv, L, None)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])
    kv1 = synth.make_kv(rng, hkv, d, L + 1)
    q1 = synth.make_q(rng, 1, hq, d)
    a = orc.attention(q1, kv1, L, np.array([1], dtype=np.uint64))
    b = orc.attention(q1, kv1, L, None)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


def test_zero_q_row_is_mean_of_visible_values(orc):
    rng = np.random.default_rng(13)
    hq, hkv, d, L, T = 4, 1, 64, 40, 6
    kv = synth.make_kv(rng, hkv, d, L + T)
    q = synth.make_q(rng, T, hq, d)
    q[3, 2] = 0.0
    parent = synth.make_tree_parents(rng, T, 6)
    mask = synth.ancestor_masks(parent)
    res = orc.attention(q, kv, L, mask)
    V = _dequant_v(orc, kv, L + T)[0]
    vis = _visible(T, L, mask)[3]
    want = V[vis].mean(axis=0)
    got = res["out"][3 * hq + 2]
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want)) + 1e-18
    assert res["lse"][3 * hq + 2] == pytest.approx(np.log(vis.sum()), rel=1e-14)


def test_planted_dominant_key(orc):
    rng = np.random.default_rng(14)
    hq, hkv, d, L, T = 2, 1, 64, 300, 1
    kv = synth.make_kv(rng, hkv, d, L + T)
    jstar = 123
    allseven = orc.pack_block([7] * 32)
    kv.k_codes[0, jstar, :] = allseven
    kv.k_scales[0, jstar, :] = np.float16(0.1).view(np.uint16)
    q = np.ones((T, hq, d), dtype=np.float32)
    # q = 1 everywhere gives q8 = 127 and sq = 1/127, so a key's logit is
    # scale * sk * sum_d (c_d - 4).  The planted key: 16 * 0.1 * 64 * 3 = 307.
    # A random key: scale <= 0.1 and sum_d (c_d - 4) = -32 +- 18, so its logit
    # sits about 250 below and its weight is far under 1e-100.
    res = orc.attention(q, kv, L, np.array([1], dtype=np.uint64), scale=16.0)
    V = _dequant_v(orc, kv, L + T)[0]
    for h in range(hq):
        assert np.max(np.abs(res["out"][h] - V[jstar])) < 1e-20


@pytest.mark.parametrize("seed", [15, 16, 17])
def test_split_partials_merge_to_unsplit(orc, seed):
    rng = np.random.default_rng(seed)
    hq, hkv, d, L, T = 4, 2, 64, 150, 9
    kv = synth.make_kv(rng, hkv, d, L + T)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 5))
    whole = orc.attention(q, kv, L, mask)
    n = L + T
    for S in (1, 2, 5, 11):
        cuts = np.sort(rng.integers(0, n + 1, size=S - 1))
        edges = [0] + list(cuts) + [n]
        po, pl = [], []
        for s in range(S):
            r = orc.attention(q, kv, L, mask, k_begin=edges[s], k_end=edges[s + 1])
            po.append(r["out"])
            pl.append(r["lse"])
        out, lse = orc.merge(np.stack(po), np.stack(pl))
        assert np.max(np.abs(out - whole["out"])) <= 1e-12 * np.max(np.abs(whole["out"]))
        assert np.max(np.abs(lse - whole["lse"])) <= 1e-12 * np.max(np.abs(whole["lse"]))
    # a split that sees no key reports lse = -inf and zeros
    r = orc.attention(q, kv, L, mask, k_begin=L + T, k_end=L + T)
    assert np.all(r["lse"] == -np.inf) and not np.any(r["out"])


def test_merge_closed_forms(orc):
    # two splits with equal lse average their outputs; an empty split is ignored
    po = np.array([[[1.0, 3.0]], [[3.0, 5.0]], [[100.0, 100.0]]])
    pl = np.array([[0.5], [0.5], [-np.inf]])
    out, lse = orc.merge(po, pl)
    assert np.array_equal(out, [[2.0, 4.0]])
    assert lse[0] == pytest.approx(0.5 + np.log(2.0), rel=1e-15)
    out, lse = orc.merge(po[2:], pl[2:])
    assert lse[0] == -np.inf and not np.any(out)


def test_row_subset_matches_full_call(orc):
    rng = np.random.default_rng(18)
    hq, hkv, d, L, T = 6, 2, 64, 90, 5
    kv = synth.make_kv(rng, hkv, d, L + T)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 3))
    full = orc.attention(q, kv, L, mask)
    rows = [17, 0, 29, 5]
    sub = orc.attention(q, kv, L, mask, rows=rows)
    assert np.array_equal(sub["out"], full["out"][rows])
    assert np.array_equal(sub["lse"], full["lse"][rows])
