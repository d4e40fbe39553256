"""GPU parity of tree acceptance and the accepted-path KV commit against the
oracle: integer outputs and every cache word and scale bit-exact."""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_tree_verify_amd as stv
    stv.load_library()
    return stv, torch


def _accept(gpu, mask, draft, target):
    stv, torch = gpu
    d = torch.from_numpy(draft).cuda()
    t = torch.from_numpy(target).cuda()
    path, n, bonus = stv.tree_accept(mask, d, t)
    return int(n.item()), path.cpu().numpy(), int(bonus.item())


def test_accept_every_8_row_shape(gpu, orc):
    rng = np.random.default_rng(31)
    for parents in synth.all_tree_shapes(8):
        draft, target = synth.make_tree_tokens(rng, parents, vocab=3)
        mask = synth.ancestor_masks(parents)
        n, path, bonus = _accept(gpu, mask, draft, target)
        wn, wpath, wb = orc.tree_accept(mask, draft, target)
        assert n == wn and np.array_equal(path, wpath) and bonus == wb, parents


def test_accept_random_trees_and_forests(gpu, orc):
    rng = np.random.default_rng(32)
    for trial in range(400):
        T = int(rng.integers(1, 65))
        parents = synth.make_tree_parents(rng, T, int(rng.integers(2, 12)))
        if trial % 4 == 0 and T > 2:
            parents = parents.copy()
            parents[int(rng.integers(1, T))] = -1
        draft, target = synth.make_tree_tokens(rng, parents, vocab=int(rng.integers(2, 5)),
                                               p_follow=float(rng.uniform(0.3, 1.0)))
        mask = synth.ancestor_masks(parents)
        n, path, bonus = _accept(gpu, mask, draft, target)
        wn, wpath, wb = orc.tree_accept(mask, draft, target)
        assert n == wn and np.array_equal(path, wpath) and bonus == wb


def _host(kv):
    return (kv.k_codes.cpu().numpy().view(np.uint32), kv.k_scales.cpu().numpy().view(np.uint16),
            kv.v_codes.cpu().numpy().view(np.uint32), kv.v_scales.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("hkv,d,L,T,seed", [
    (1, 64, 0, 1, 1), (2, 64, 29, 8, 2), (4, 256, 61, 17, 3), (4, 256, 1000, 64, 4),
    (2, 128, 95, 64, 5), (3, 128, 31, 33, 6),
])
def test_commit_matches_oracle(gpu, orc, hkv, d, L, T, seed):
    stv, torch = gpu
    rng = np.random.default_rng(seed)
    cap = L + T + 7
    host = synth.make_kv(rng, hkv, d, L + T, cap)
    parents = synth.make_tree_parents(rng, T, 8)
    draft, target = synth.make_tree_tokens(rng, parents, vocab=2, p_follow=0.9)
    mask = synth.ancestor_masks(parents)
    kv = stv.KVCache.from_host(host)
    path, n, _ = stv.tree_accept(mask, torch.from_numpy(draft).cuda(),
                                 torch.from_numpy(target).cuda())
    stv.kv_commit(kv, L, path, n)
    torch.cuda.synchronize()
    wn, wpath, _ = orc.tree_accept(mask, draft, target)
    orc.kv_commit(host, L, T, wpath, wn)
    got = _host(kv)
    for g, w, name in zip(got, (host.k_codes, host.k_scales, host.v_codes, host.v_scales),
                          ("k_codes", "k_scales", "v_codes", "v_scales")):
        assert np.array_equal(g, w), name


def test_commit_ignores_malformed_device_inputs(gpu):
    """A count or path entry out of range (set from the host) leaves the cache as it was."""
    stv, torch = gpu
    rng = np.random.default_rng(7)
    host = synth.make_kv(rng, 2, 64, 50, 50)
    kv = stv.KVCache.from_host(host)
    before = _host(kv)
    T, L = 10, 40
    for n_val, path_val in ((0, list(range(10))), (11, list(range(10))),
                            (3, [0, 2, 10] + [-1] * 7), (2, [0, -5] + [-1] * 8)):
        path = torch.tensor(path_val, dtype=torch.int32, device="cuda")
        n = torch.tensor([n_val], dtype=torch.int32, device="cuda")
        stv.kv_commit(kv, L, path, n)
    torch.cuda.synchronize()
    for a, b in zip(_host(kv), before):
        assert np.array_equal(a, b)


def test_verify_accept_commit_round(gpu, orc):
    """One whole round on the GPU: verify the tree, accept, commit, then the
    chain of committed rows over the compacted cache matches the oracle and
    the committed tree rows."""
    stv, torch = gpu
    rng = np.random.default_rng(41)
    hq, hkv, d, L, T = 24, 4, 256, 3000, 64
    host = synth.make_kv(rng, hkv, d, L + T, L + T + 5)
    q = synth.make_q(rng, T, hq, d)
    parents = synth.make_tree_parents(rng, T, 8)
    mask = synth.ancestor_masks(parents)
    draft, target = synth.make_tree_tokens(rng, parents, vocab=2, p_follow=0.95)
    scale = 1.0 / math.sqrt(d)
    kv = stv.KVCache.from_host(host)
    qd = torch.from_numpy(q).cuda()
    tree_out = stv.verify_attention(qd, kv, L, mask, scale)
    path, n, _ = stv.tree_accept(mask, torch.from_numpy(draft).cuda(),
                                 torch.from_numpy(target).cuda())
    stv.kv_commit(kv, L, path, n)
    nn = int(n.item())
    p = path.cpu().numpy()[:nn]
    assert nn >= 2
    chain_mask = synth.ancestor_masks(synth.chain_parents(nn))
    chain_out = stv.verify_attention(qd[torch.from_numpy(p.astype(np.int64)).cuda()].contiguous(),
                                     kv, L, chain_mask, scale)
    torch.cuda.synchronize()
    ref = orc.attention(q, host, L, mask, scale)["out"].reshape(T, hq, d)
    a = tree_out.cpu().numpy()[p]
    b = chain_out.cpu().numpy()
    for x in (a, b):
        err = np.max(np.abs(x - ref[p]), axis=-1) / np.max(np.abs(ref[p]), axis=-1)
        assert err.max() <= 2e-3
