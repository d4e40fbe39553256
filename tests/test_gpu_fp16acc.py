"""GPU: the fp16-accumulated P.V variant of verify attention against the
fp64 oracle (elpis, "What fast means": the fp16-accumulated P.V decode
kernel, which the pages list as unresolved).

The variant rounds each 32-key tile's P.V product to fp16 and adds it into
fp16 accumulators; the running max follows every increase, so P <= 1.  Two
kinds of assertion hold it:

1. Measured figures.  Every case's maximum row error
   max_d |o - o_ref| / max_d |o_ref| is held to a cap a few times the error
   measured on MI355X, listed per case below.  At the pages' shape (the
   8-row tree over 262,144 keys) and at one token over 262,144 keys the cap
   is 2e-3, the fp32 path's bar.  One case exceeds that bar and keeps its
   own documented cap: a single split over 1,500 keys at head_dim 128,
   where each accumulator takes 47 fp16 additions.

2. A bound derived from the arithmetic, at every size, in terms of the
   accumulator's own magnitude.  A stream of tiles k = 1..n (one split; in
   the few-row kernel, one wave's tiles of a split) keeps O_k = alpha_k
   O_{k-1} + t_k in fp16, with three roundings per tile (the tile product,
   the rescale, the add), each at most u = 2^-11 times its result.  Divided
   by the final row sum l_n (which is at least alpha-scaled l_k), the error
   of tile k is at most u (2 |o_k| + 2 |o_{k-1}|), where o_k is the
   normalized output of the stream's prefix of k tiles.  Hence per row

       |o - o_ref| <= TOL max|o_ref| + 4 u sum_k max_d |o_k| + 3 n 2^-25,

   the last term for fp16 subnormal spacing (l_k >= 1: the prefix maximum
   has P = 1); the split merge and the few-row kernel's wave merge are
   convex combinations in fp32 and add nothing.  TOL = 2e-3 covers, as for
   the fp32 path, the fp16 rounding of P and V and the fp32 sums.  The
   prefix outputs o_k come from the oracle over each tile's key range,
   combined by log-sum-exp in fp64.

The lse takes no fp16 accumulation and stays within 2e-3.  The test also
checks that the variant is a different computation from the fp32 path.
"""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3
U16 = 2.0 ** -11
KEY_TILE = 32
DEC_MAX_ROWS = 16        # rows per KV head up to which the few-row kernel runs (3-bit)
DEC_WAVES = 4            # its waves, each streaming every fourth tile of a split


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_tree_verify_amd as stv
    stv.load_library()
    return stv, torch


def _row_err_abs(got, ref):
    return np.max(np.abs(got - ref), axis=-1)


def _streams(n_keys, S, few_row):
    """Tile indices of each fp16 accumulation stream, in the order the
    kernel adds them."""
    n_tiles = -(-n_keys // KEY_TILE)
    per = -(-n_tiles // S)
    out = []
    for s in range(S):
        tiles = list(range(s * per, min(n_tiles, (s + 1) * per)))
        if not tiles:
            continue
        if few_row:
            out.extend(t for t in (tiles[w::DEC_WAVES] for w in range(DEC_WAVES)) if t)
        else:
            out.append(tiles)
    return out


def _prefix_bound(orc, q, host, L, mask, scale, rows, n_keys, streams):
    """4 u sum_k max_d |o_k| + 3 n 2^-25 per row, maximised over streams."""
    tiles = sorted({t for st in streams for t in st})
    part = {}
    for t in tiles:
        r = orc.attention(q, host, L, mask, scale, k_begin=KEY_TILE * t,
                          k_end=min(n_keys, KEY_TILE * (t + 1)), rows=rows)
        part[t] = (r["out"], r["lse"])
    worst = np.zeros(len(rows))
    for st in streams:
        o_run = np.zeros_like(part[st[0]][0])
        lse_run = np.full(len(rows), -np.inf)
        acc = np.zeros(len(rows))
        for t in st:
            o_t, lse_t = part[t]
            new = np.logaddexp(lse_run, lse_t)
            fin = np.isfinite(new)
            w_run = np.where(fin & np.isfinite(lse_run), np.exp(lse_run - np.where(fin, new, 0)), 0.0)
            w_t = np.where(fin & np.isfinite(lse_t), np.exp(lse_t - np.where(fin, new, 0)), 0.0)
            o_run = w_run[:, None] * o_run + w_t[:, None] * o_t
            lse_run = new
            acc += np.max(np.abs(o_run), axis=-1)
        worst = np.maximum(worst, 4 * U16 * acc + 3 * len(st) * 2.0 ** -25)
    return worst


def run_fp16acc(gpu, orc, hq, hkv, d, L, T, seed, cap, rows=None, n_splits=0, scale_mul=1.0,
                host=None, q=None, mask=None, derived=True):
    stv, torch = gpu
    rng = np.random.default_rng(seed)
    if host is None:
        host = synth.make_kv(rng, hkv, d, L + T, L + T + 5)
    if q is None:
        q = synth.make_q(rng, T, hq, d)
    if mask is None:
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, min(8, T)) if T > 1
                                    else synth.chain_parents(1))
    scale = scale_mul / math.sqrt(d)
    flat = np.arange(T * hq) if rows is None else np.asarray(rows)
    ref = orc.attention(q, host, L, mask, scale, rows=flat)
    kv = stv.KVCache.from_host(host)
    qd = torch.from_numpy(q).cuda()
    lse16 = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    lse32 = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    o16 = stv.verify_attention_fp16acc(qd, kv, L, mask, scale, out_lse=lse16, n_splits=n_splits)
    o32 = stv.verify_attention(qd, kv, L, mask, scale, out_lse=lse32, n_splits=n_splits)
    torch.cuda.synchronize()
    fd = torch.from_numpy(flat).cuda()
    g16 = o16.reshape(T * hq, d)[fd].cpu().numpy()
    g32 = o32.reshape(T * hq, d)[fd].cpu().numpy()
    assert np.all(np.isfinite(g16))
    S, _ = stv.attention_plan(T, hq, hkv, d, L, False, n_splits)
    ref_o = ref["out"]
    den = np.maximum(np.max(np.abs(ref_o), axis=-1), 1e-30)
    err16 = _row_err_abs(g16, ref_o)
    rel16 = float(np.max(err16 / den))
    streams = _streams(L + T, S, T * (hq // hkv) <= DEC_MAX_ROWS)
    print(f"fp16-acc max row error {rel16:.3g} (cap {cap:g}), fp32 path "
          f"{np.max(_row_err_abs(g32, ref_o) / den):.3g}; {S} splits, "
          f"{max(len(s) for s in streams)} tiles per stream")
    assert rel16 <= cap, f"max row error {rel16:.3g} above the case's cap {cap:g}"
    if derived:
        bound = TOL * np.max(np.abs(ref_o), axis=-1) + _prefix_bound(
            orc, q, host, L, mask, scale, flat, L + T, streams)
        assert np.all(err16 <= bound), f"row error {err16.max():.3g} above derived bound"
    l16 = lse16.reshape(-1)[fd].cpu().numpy()
    assert np.max(np.abs(l16 - ref["lse"])) <= TOL
    return {"rel16": rel16, "identical": bool(np.array_equal(g16, g32)), "splits": S}


CASES = [
    # name, hq, hkv, d, L, T, seed, n_splits, cap on the max row error
    ("dec_one_token", 24, 4, 256, 4000, 1, 300, 0, 1e-3),          # few-row kernel
    ("dec_one_token_d64", 4, 1, 64, 777, 1, 301, 3, 2e-3),
    ("tree8", 24, 4, 256, 5000, 8, 302, 0, 2e-3),                   # 16-row kernel
    ("tree8_d128_one_split", 8, 2, 128, 1500, 8, 303, 1, 6e-3),     # 47 tiles, measured 2.8e-3
    ("tree64", 24, 4, 256, 3000, 64, 304, 0, 2e-3),                 # 32-row split kernel
    ("tree3_ragged", 6, 2, 64, 45, 3, 305, 2, 2e-3),
]


@pytest.mark.parametrize("name,hq,hkv,d,L,T,seed,ns,cap", CASES, ids=[c[0] for c in CASES])
def test_fp16acc_within_bound(gpu, orc, name, hq, hkv, d, L, T, seed, ns, cap):
    run_fp16acc(gpu, orc, hq, hkv, d, L, T, seed, cap, n_splits=ns)


def test_fp16acc_peaked(gpu, orc):
    """Peaked logits move the running max often (many fp16 rescales)."""
    run_fp16acc(gpu, orc, 24, 4, 256, 6000, 8, 310, 2e-3, scale_mul=16.0)


def test_fp16acc_differs_from_fp32_path(gpu, orc):
    """One split over a long context: the fp16 sums must show up."""
    r = run_fp16acc(gpu, orc, 24, 4, 256, 20000, 8, 311, 2e-2, rows=[0, 5, 100, 191],
                    n_splits=1)
    assert not r["identical"]


def test_fp16acc_rejects_4bit_cache(gpu):
    stv, torch = gpu
    rng = np.random.default_rng(312)
    host = synth.make_kv4(rng, 1, 64, 100)
    kv = stv.KVCache.from_host(host)
    q = torch.from_numpy(synth.make_q(rng, 1, 4, 64)).cuda()
    with pytest.raises(stv.StvError):
        stv.verify_attention_fp16acc(q, kv, 99, [1])


@pytest.mark.parametrize("name", ["tree8_262k", "decode_262k"])
def test_fp16acc_262k_sampled(gpu, orc, name):
    """The pages' shape (the 8-row tree over 262,144 keys) and one token over
    262,144 keys, in the automatic split plan: sampled rows of every KV head
    against the oracle, held to 2e-3 (measured on MI355X: 2.7e-4 at the
    8-row tree).  The derived bound is left out here: it needs the oracle
    over each of the 8,194 tiles."""
    geom = [g for g in synth.EXTRA_CONFIGS if g.name == name][0]
    rng = np.random.default_rng(geom.seed)
    host = synth.make_kv(rng, geom.n_kv_heads, geom.head_dim, geom.n_keys)
    q = synth.make_q(rng, geom.n_rows, geom.n_q_heads, geom.head_dim)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, geom.n_rows, geom.max_depth)
                                if geom.n_rows > 1 else synth.chain_parents(1))
    hq = geom.n_q_heads
    heads = (0, 5, 11, 23)
    rows = sorted({t * hq + h for t in ((0, 3, geom.n_rows - 1) if geom.n_rows > 1 else (0,))
                   for h in heads})
    run_fp16acc(gpu, orc, hq, geom.n_kv_heads, geom.head_dim, geom.ctx_len, geom.n_rows,
                geom.seed, 2e-3, rows=rows, host=host, q=q, mask=mask, derived=False)
