"""GPU: the context split across devices, emulated on one GPU (split-K over
the context, elpis-lossless "Trust base").  One slice of the cache holds
context keys only and goes through stv_context_partials; the other holds the
rest of the context and the tree keys and goes through
stv_attention_partials; stv_split_merge joins them.  With the slice boundary
on a split boundary, the result equals one verify call over the whole cache
with the same two splits, bit for bit, and matches the oracle.
"""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_tree_verify_amd as stv
    stv.load_library()
    return stv, torch


def _slice(host, k0, k1):
    """Keys [k0, k1) of a cache as a cache of their own (k0 a multiple of 32)."""
    assert k0 % 32 == 0
    g0, g1 = k0 // 32, (k1 + 31) // 32
    if host.fmt == "i4":
        return synth.KVCache(host.k_codes[:, k0:k1].copy(), host.k_scales[:, k0:k1].copy(),
                             host.v_codes[:, g0:g1].copy(), host.v_scales[:, k0:k1].copy(),
                             host.n_kv_heads, host.head_dim, k1 - k0, k1 - k0, "i4")
    return synth.KVCache(host.k_codes[:, k0:k1].copy(), host.k_scales[:, k0:k1].copy(),
                         host.v_codes[:, g0:g1].copy(), host.v_scales[:, g0:g1].copy(),
                         host.n_kv_heads, host.head_dim, k1 - k0, k1 - k0, host.fmt)


CASES = [
    # name, hq, hkv, d, L, T, fmt (few-row, 16-row and wave-specialized kernels; 4-bit few-row)
    ("one_token", 24, 4, 256, 5000, 1, "b3"),
    ("tree8", 24, 4, 256, 5000, 8, "b3"),
    ("tree64", 24, 4, 256, 3000, 64, "b3"),
    ("tree8_4bit", 24, 4, 256, 4000, 8, "i4"),
    ("tree8_d64", 8, 2, 64, 777, 8, "b3"),
]


@pytest.mark.parametrize("name,hq,hkv,d,L,T,fmt", CASES, ids=[c[0] for c in CASES])
def test_context_shards_equal_one_call(gpu, orc, name, hq, hkv, d, L, T, fmt):
    stv, torch = gpu
    rng = np.random.default_rng(500 + T)
    make = synth.make_kv if fmt == "b3" else synth.make_kv4
    host = make(rng, hkv, d, L + T)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8) if T > 1
                                else synth.chain_parents(1))
    scale = 1.0 / math.sqrt(d)
    qd = torch.from_numpy(q).cuda()
    N = L + T
    S, _ = stv.attention_plan(T, hq, hkv, d, L, False, 2, fmt)
    assert S == 2
    P = 32 * -(-(-(-N // 32)) // 2)                 # 32 * ceil(ceil(N / 32) / 2)
    assert P <= L

    # one call over the whole cache, two splits
    lse1 = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    one = stv.verify_attention(qd, stv.KVCache.from_host(host), L, mask, scale, out_lse=lse1,
                               n_splits=2)

    # slice A: context keys [0, P); slice B: keys [P, N) with the tree keys
    kva = stv.KVCache.from_host(_slice(host, 0, P))
    kvb = stv.KVCache.from_host(_slice(host, P, N))
    assert stv.context_plan(T, hq, hkv, d, P, 1, fmt)[0] == 1
    pa, la = stv.context_partials(qd, kva, P, scale, n_splits=1)
    pb, lb = stv.attention_partials(qd, kvb, L - P, mask, scale, n_splits=1)
    po = torch.cat([pa, pb]).reshape(2, T * hq, d).contiguous()
    pl = torch.cat([la, lb]).reshape(2, T * hq).contiguous()
    lse2 = torch.empty(T * hq, dtype=torch.float32, device="cuda")
    merged = stv.split_merge(po, pl, out_lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(merged, one.reshape(T * hq, d)), "sharded result differs from one call"
    assert torch.equal(lse2, lse1.reshape(-1))

    # and both match the oracle (slice A against the oracle's key range too)
    rows = np.linspace(0, T * hq - 1, min(T * hq, 12)).round().astype(np.int32)
    ref = orc.attention(q, host, L, mask, scale, rows=rows)
    got = merged.cpu().numpy()[rows]
    err = np.max(np.abs(got - ref["out"]), axis=-1) / np.max(np.abs(ref["out"]), axis=-1)
    assert err.max() <= TOL
    ref_a = orc.attention(q, host, L, mask, scale, k_begin=0, k_end=P, rows=rows)
    got_a = pa.reshape(T * hq, d).cpu().numpy()[rows]
    err_a = np.max(np.abs(got_a - ref_a["out"]), axis=-1) / np.max(np.abs(ref_a["out"]), axis=-1)
    assert err_a.max() <= TOL
