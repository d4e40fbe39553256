"""GPU parity for the second KV format (4-bit codes, one scale per token-head)
against the oracle: int8 Q and the whole-row int32 Q.K^T sums bit-exact,
outputs within 2e-3 per row (max_d |o - o_ref| / max_d |o_ref|), lse within
2e-3; the 4-bit pack bit-exact."""
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


def _row_err(got, ref):
    den = np.max(np.abs(ref), axis=-1)
    return np.max(np.abs(got - ref), axis=-1) / np.where(den > 0, den, 1.0)


def _visible(T, L, mask, n):
    vis = np.zeros((T, n), dtype=bool)
    vis[:, :L] = True
    for t in range(T):
        for a in range(T):
            vis[t, L + a] = (a <= t) if mask is None else bool((int(mask[t]) >> a) & 1)
    return vis


def run4(gpu, orc, hq, hkv, d, L, T, kind, seed, n_splits=0, rows=None, check_logits=True,
         scale_mul=1.0):
    stv, torch = gpu
    rng = np.random.default_rng(seed)
    host = synth.make_kv4(rng, hkv, d, L + T, L + T + 3)
    q = synth.make_q(rng, T, hq, d)
    mask = None
    if kind == "chain":
        mask = synth.ancestor_masks(synth.chain_parents(T))
    elif kind == "tree":
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8))
    scale = scale_mul / math.sqrt(d)
    ref = orc.attention(q, host, L, mask, scale, rows=rows, want_logits=check_logits)
    kv = stv.KVCache.from_host(host)
    qd = torch.from_numpy(q).cuda()
    lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")

    def call(debug):
        if kind == "prefill":
            return stv.prefill_attention(qd, kv, L, scale, out_lse=lse, n_splits=n_splits,
                                         debug=debug)
        return stv.verify_attention(qd, kv, L, mask, scale, out_lse=lse, n_splits=n_splits,
                                    debug=debug)

    flat = np.arange(T * hq) if rows is None else np.asarray(rows)
    out = call(False)
    torch.cuda.synchronize()
    o = out.reshape(T * hq, d).cpu().numpy()[flat]
    assert np.all(np.isfinite(o))
    err = _row_err(o, ref["out"])
    assert err.max() <= TOL, f"max row error {err.max():.3g}"
    assert np.max(np.abs(lse.reshape(-1).cpu().numpy()[flat] - ref["lse"])) <= TOL
    names = ("logits", "q8", "qscale") if check_logits else ("q8", "qscale")
    _, dbg = call(names)
    torch.cuda.synchronize()
    assert np.array_equal(dbg["q8"].reshape(T * hq, d).cpu().numpy()[flat], ref["qi8"])
    assert np.array_equal(dbg["qscale"].reshape(-1).cpu().numpy()[flat].view(np.uint32),
                          ref["sq"].view(np.uint32))
    if check_logits:
        lg = dbg["logits"].reshape(T * hq, L + T).cpu().numpy()[flat]
        vis = _visible(T, L, mask, L + T)
        for i, r in enumerate(flat):
            v = vis[r // hq]
            assert np.array_equal(lg[i][v], ref["logits"][i][v]), f"logits differ, row {r}"
    return err.max()


CASES = [
    ("tiny_chain", 4, 1, 64, 512, 8, "chain", 0, 0),
    ("tiny_3split", 4, 1, 64, 512, 8, "chain", 0, 3),
    ("tree64_ragged", 24, 4, 256, 1000, 64, "tree", 201, 0),
    ("tree8_d128", 8, 2, 128, 777, 8, "tree", 202, 0),
    ("tree17_d128", 8, 2, 128, 333, 17, "tree", 203, 5),
    ("decode_t1", 24, 4, 256, 2049, 1, "tree", 204, 0),
    ("tree_L0", 4, 2, 64, 0, 5, "tree", 205, 0),
    ("prefill_small", 12, 2, 128, 100, 70, "prefill", 206, 0),
    ("prefill_splits", 8, 1, 64, 300, 40, "prefill", 207, 4),
    ("tree8_d256_r48", 24, 4, 256, 1500, 8, "tree", 208, 0),
    ("prefill_r60", 24, 4, 256, 200, 10, "prefill", 209, 3),
]


@pytest.mark.parametrize("name,hq,hkv,d,L,T,kind,seed,ns", CASES, ids=[c[0] for c in CASES])
def test_parity_int4(gpu, orc, name, hq, hkv, d, L, T, kind, seed, ns):
    run4(gpu, orc, hq, hkv, d, L, T, kind, seed, n_splits=ns)


def test_full_size_tree_sampled_rows(gpu, orc):
    rows = np.linspace(0, 64 * 24 - 1, 24).round().astype(np.int32)
    run4(gpu, orc, 24, 4, 256, 65536, 64, "tree", 208, rows=rows, check_logits=False)


@pytest.mark.parametrize("T,n_rows", [(1, 24), (8, 12)], ids=["one_token", "tree8"])
def test_full_size_262k_sampled_rows(gpu, orc, T, n_rows):
    """One token and the 8-row tree over 262,144 keys (the few-row kernel,
    in the split plan the benchmark times)."""
    rows = np.linspace(0, T * 24 - 1, n_rows).round().astype(np.int32)
    run4(gpu, orc, 24, 4, 256, 262144 - T, T, "tree", 210 + T, rows=rows, check_logits=False)


@pytest.mark.parametrize("scale_mul", [8.0, 32.0])
def test_parity_int4_peaked(gpu, orc, scale_mul):
    """Nearly one-hot softmax: the running max moves often, which rescales
    the few-row kernel's per-row V-scale sums with the accumulators, and the
    32-row kernel's accumulators at the 64-node tree."""
    run4(gpu, orc, 24, 4, 256, 1500, 1, "tree", 212, scale_mul=scale_mul)
    run4(gpu, orc, 24, 4, 256, 900, 8, "tree", 213, scale_mul=scale_mul)
    run4(gpu, orc, 24, 4, 256, 700, 16, "tree", 214, scale_mul=scale_mul)
    # the 64-node tree: the 32-row kernel rescales its accumulators
    run4(gpu, orc, 24, 4, 256, 1200, 64, "tree", 215, scale_mul=scale_mul)


@pytest.mark.parametrize("d,pos0,n_tok", [(64, 0, 1), (128, 29, 8), (256, 61, 64), (256, 0, 100)])
def test_pack4_matches_oracle(gpu, orc, d, pos0, n_tok):
    stv, torch = gpu
    rng = np.random.default_rng(pos0 + d)
    hkv, cap = 3, pos0 + n_tok + 40
    x = (rng.standard_normal((n_tok, hkv, d)) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
    x[0, 0, :] = 0.0                                   # a zero row: scale 0, codes 8
    host = synth.make_kv4(rng, hkv, d, cap, cap)
    kv = stv.KVCache.from_host(host)
    xd = torch.from_numpy(x).cuda()
    stv.kv_quant_pack(xd, pos0, kv, "k")
    stv.kv_quant_pack(xd, pos0, kv, "v")
    torch.cuda.synchronize()
    orc.kv4_quant_pack(x, pos0, host.k_codes, host.k_scales, "k")
    orc.kv4_quant_pack(x, pos0, host.v_codes, host.v_scales, "v")
    assert np.array_equal(kv.k_codes.cpu().numpy().view(np.uint32), host.k_codes)
    assert np.array_equal(kv.k_scales.cpu().numpy().view(np.uint16), host.k_scales)
    assert np.array_equal(kv.v_codes.cpu().numpy().view(np.uint32), host.v_codes)
    assert np.array_equal(kv.v_scales.cpu().numpy().view(np.uint16), host.v_scales)


@pytest.mark.parametrize("hkv,d,L,T,seed", [(2, 64, 29, 8, 1), (4, 256, 1000, 64, 2),
                                            (3, 128, 31, 33, 3)])
def test_commit4_matches_oracle(gpu, orc, hkv, d, L, T, seed):
    stv, torch = gpu
    rng = np.random.default_rng(seed + 90)
    cap = L + T + 7
    host = synth.make_kv4(rng, hkv, d, L + T, cap)
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
    assert np.array_equal(kv.k_codes.cpu().numpy().view(np.uint32), host.k_codes)
    assert np.array_equal(kv.k_scales.cpu().numpy().view(np.uint16), host.k_scales)
    assert np.array_equal(kv.v_codes.cpu().numpy().view(np.uint32), host.v_codes)
    assert np.array_equal(kv.v_scales.cpu().numpy().view(np.uint16), host.v_scales)


def test_shape_sweep_kernel_boundaries_int4(gpu, orc):
    """The 4-bit format on both sides of its plan's boundaries (64 | 65 rows
    per KV head: few-row / 32-row kernel; 96 | 97: two / four row tiles),
    over head dims, context lengths and split counts, against the oracle on
    sampled rows, int8 Q and int32 logits bit for bit."""
    rng = np.random.default_rng(1500)
    for i, (g, T) in enumerate([(1, 64), (2, 32), (2, 33), (6, 10), (6, 11), (6, 16), (6, 17),
                                (8, 8), (8, 9), (3, 22), (6, 64), (8, 64)]):
        hkv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128, 256]))
        L = int(rng.choice([0, 1, 31, 700, 2049]))
        ns = int(rng.choice([0, 0, 1, 2, 3, 5]))
        hq = g * hkv
        rows = np.unique(np.linspace(0, T * hq - 1, 12).round().astype(np.int64))
        run4(gpu, orc, hq, hkv, d, L, T, "tree", 1600 + i, n_splits=ns, rows=rows)
