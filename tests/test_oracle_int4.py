"""Pins for the oracle's second KV format: 4-bit codes with one fp16 scale
per (token, KV head).  The layout and quantizer are readings; these tests pin
the oracle to hand-worked rows, to the quantizer's error bound, to this
file's own reader of the layouts, and its attention to a dense fp64 brute
force and to the row-independence and chain == causal invariants."""
import numpy as np
import pytest

import synth


def _k_val(kv, g, j, d):
    c = (int(kv.k_codes[g, j, d // 8]) >> (4 * (d % 8))) & 15
    return c - 8


def _v_val(kv, g, j, d):
    c = (int(kv.v_codes[g, j // 32, d, (j % 32) // 8]) >> (4 * (j % 8))) & 15
    return c - 8


def _f16(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def _dense(kv, g, n):
    d = kv.head_dim
    K = np.array([[_k_val(kv, g, j, e) for e in range(d)] for j in range(n)], dtype=np.float64)
    V = np.array([[_v_val(kv, g, j, e) for e in range(d)] for j in range(n)], dtype=np.float64)
    sk = np.array([_f16(kv.k_scales[g, j]) for j in range(n)])
    sv = np.array([_f16(kv.v_scales[g, j]) for j in range(n)])
    return K, V, sk, sv


def test_quantizer_worked_rows(orc):
    x = np.zeros(32, dtype=np.float32)
    x[:4] = [7.0, -7.0, 3.5, 2.5]
    w, s = orc.quantize_kv4_row(x)
    assert s == 0x3C00                       # fp16(7 / 7) = 1.0
    codes = [(int(w[e // 8]) >> (4 * (e % 8))) & 15 for e in range(32)]
    # 7 -> 15, -7 -> 1, 3.5 -> rint 4 (ties to even) -> 12, 2.5 -> 2 -> 10, zeros -> 8
    assert codes == [15, 1, 12, 10] + [8] * 28
    w, s = orc.quantize_kv4_row(np.zeros(64, dtype=np.float32))
    assert s == 0 and np.all(w == 0x88888888)
    w, s = orc.quantize_kv4_row(np.full(32, 1e6, dtype=np.float32))
    assert s == 0x7BFF and np.all(w == 0xFFFFFFFF)   # saturated scale, every code 15


def test_quantizer_error_bound(orc):
    rng = np.random.default_rng(71)
    for trial in range(300):
        d = int(rng.choice([32, 64, 256]))
        x = (rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        w, s16 = orc.quantize_kv4_row(x)
        s = _f16(s16)
        codes = np.array([(int(w[e // 8]) >> (4 * (e % 8))) & 15 for e in range(d)])
        assert codes.min() >= 1
        xhat = s * (codes - 8)
        inr = np.abs(x) <= 7 * s
        assert np.all(np.abs(x[inr] - xhat[inr]) <= s * (0.5 + 1e-6))
        assert np.all(np.abs(xhat[~inr]) == 7 * s)


def test_pack_writes_only_its_positions(orc):
    rng = np.random.default_rng(72)
    hkv, d, cap = 2, 64, 70
    x = rng.standard_normal((5, hkv, d)).astype(np.float32)
    pos0 = 29
    kv = synth.make_kv4(rng, hkv, d, cap, cap)
    k0, ks0, v0, vs0 = (a.copy() for a in (kv.k_codes, kv.k_scales, kv.v_codes, kv.v_scales))
    orc.kv4_quant_pack(x, pos0, kv.k_codes, kv.k_scales, "k")
    orc.kv4_quant_pack(x, pos0, kv.v_codes, kv.v_scales, "v")
    old = synth.KVCache(k0, ks0, v0, vs0, hkv, d, cap, cap, "i4")
    for g in range(hkv):
        for j in range(cap):
            new = pos0 <= j < pos0 + 5
            if new:
                w, s = orc.quantize_kv4_row(x[j - pos0, g])
                want = [((int(w[e // 8]) >> (4 * (e % 8))) & 15) - 8 for e in range(d)]
                assert kv.k_scales[g, j] == s and kv.v_scales[g, j] == s
            else:
                want = [_k_val(old, g, j, e) for e in range(d)]
                assert kv.k_scales[g, j] == ks0[g, j] and kv.v_scales[g, j] == vs0[g, j]
            assert [_k_val(kv, g, j, e) for e in range(d)] == want
            wantv = want if new else [_v_val(old, g, j, e) for e in range(d)]
            assert [_v_val(kv, g, j, e) for e in range(d)] == wantv


@pytest.mark.parametrize("hq,hkv,d,L,T,kind,seed", [
    (4, 1, 64, 40, 8, "chain", 1), (6, 2, 64, 33, 5, "tree", 2), (4, 2, 128, 20, 7, "prefill", 3),
])
def test_attention_matches_dense_brute_force(orc, hq, hkv, d, L, T, kind, seed):
    rng = np.random.default_rng(seed)
    kv = synth.make_kv4(rng, hkv, d, L + T, L + T + 3)
    q = synth.make_q(rng, T, hq, d)
    mask = None
    if kind == "chain":
        mask = synth.ancestor_masks(synth.chain_parents(T))
    elif kind == "tree":
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 4))
    scale = 0.1
    r = orc.attention(q, kv, L, mask, scale, want_logits=True)
    G = hq // hkv
    N = L + T
    for t in range(T):
        for h in range(hq):
            g = h // G
            K, V, sk, sv = _dense(kv, g, N)
            qi = r["qi8"][t * hq + h].astype(np.float64)
            S = K @ qi
            assert np.array_equal(r["logits"][t * hq + h], S.astype(np.int64))
            x = scale * float(r["sq"][t * hq + h]) * sk * S
            vis = np.ones(N, bool)
            for a in range(T):
                vis[L + a] = (a <= t) if mask is None else bool((int(mask[t]) >> a) & 1)
            m = x[vis].max()
            p = np.where(vis, np.exp(x - m), 0.0)
            o = (p[:, None] * (sv[:, None] * V)).sum(0) / p.sum()
            assert np.max(np.abs(o - r["out"][t * hq + h])) <= 1e-12
            assert abs(r["lse"][t * hq + h] - (m + np.log(p.sum()))) <= 1e-12


def test_tree_rows_equal_their_chains_and_chain_is_causal(orc):
    rng = np.random.default_rng(74)
    hq, hkv, d, L, T = 4, 2, 64, 50, 8
    q = synth.make_q(rng, T, hq, d)
    for trial in range(20):
        parents = synth.make_tree_parents(rng, T, 5)
        x = rng.standard_normal((T, hkv, d)).astype(np.float32)
        base = synth.make_kv4(rng, hkv, d, L, L + T)
        kv = synth.KVCache(base.k_codes.copy(), base.k_scales.copy(), base.v_codes.copy(),
                           base.v_scales.copy(), hkv, d, L + T, L + T, "i4")
        orc.kv4_quant_pack(x, L, kv.k_codes, kv.k_scales, "k")
        orc.kv4_quant_pack(x, L, kv.v_codes, kv.v_scales, "v")
        tree = orc.attention(q, kv, L, synth.ancestor_masks(parents), 0.125)
        for i in range(T):
            path = []
            v = i
            while v >= 0:
                path.append(v)
                v = parents[v]
            path = path[::-1]
            n = len(path)
            ch = synth.KVCache(base.k_codes.copy(), base.k_scales.copy(), base.v_codes.copy(),
                               base.v_scales.copy(), hkv, d, L + T, L + T, "i4")
            orc.kv4_quant_pack(x[path], L, ch.k_codes, ch.k_scales, "k")
            orc.kv4_quant_pack(x[path], L, ch.v_codes, ch.v_scales, "v")
            qc = q[path]
            causal = orc.attention(qc, ch, L, None, 0.125)
            for h in range(hq):
                assert np.array_equal(tree["out"][i * hq + h], causal["out"][(n - 1) * hq + h])


@pytest.mark.parametrize("L,T,seed", [(0, 8, 1), (29, 8, 2), (61, 17, 3), (100, 64, 4)])
def test_commit4_moves_exactly_the_committed_tokens(orc, L, T, seed):
    rng = np.random.default_rng(seed + 80)
    hkv, d = 2, 64
    cap = L + T + 5
    kv = synth.make_kv4(rng, hkv, d, L + T, cap)
    old = synth.KVCache(kv.k_codes.copy(), kv.k_scales.copy(), kv.v_codes.copy(),
                        kv.v_scales.copy(), hkv, d, cap, kv.n_filled, "i4")
    parents = synth.make_tree_parents(rng, T, 8)
    draft, target = synth.make_tree_tokens(rng, parents, vocab=2, p_follow=0.9)
    n, path, _ = orc.tree_accept(synth.ancestor_masks(parents), draft, target)
    orc.kv_commit(kv, L, T, path, n)
    for g in range(hkv):
        for pos in range(cap):
            src = L + int(path[pos - L]) if L <= pos < L + n else pos
            assert [_k_val(kv, g, pos, e) for e in range(d)] == [_k_val(old, g, src, e) for e in range(d)]
            assert [_v_val(kv, g, pos, e) for e in range(d)] == [_v_val(old, g, src, e) for e in range(d)]
            assert kv.k_scales[g, pos] == old.k_scales[g, src]
            assert kv.v_scales[g, pos] == old.v_scales[g, src]
