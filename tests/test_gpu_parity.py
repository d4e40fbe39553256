"""GPU parity: the HIP path through the C ABI against the CPU oracle.

The bar: quantized Q (int8 codes and fp32 scales) and the int32 per-block
Q.K^T sums bit-exact; attention outputs within 2e-3 relative error per row,
measured as max_d |o - o_ref| / max_d |o_ref| (the oracle is fp64); lse
within 2e-3 absolute.  Inputs are seeded and synthetic (synth module).
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


def _visible(T, L, mask, n):
    vis = np.zeros((T, n), dtype=bool)
    vis[:, :L] = True
    for t in range(T):
        for a in range(T):
            vis[t, L + a] = (a <= t) if mask is None else bool((int(mask[t]) >> a) & 1)
    return vis


def _row_err(got, ref):
    den = np.max(np.abs(ref), axis=-1)
    num = np.max(np.abs(got - ref), axis=-1)
    return num / np.where(den > 0, den, 1.0)


def _mask_for(rng, kind, T, depth=8):
    if kind == "prefill":
        return None
    if kind == "chain":
        return synth.ancestor_masks(synth.chain_parents(T))
    return synth.ancestor_masks(synth.make_tree_parents(rng, T, depth))


def run_case(gpu, orc, hq, hkv, d, L, T, kind, seed, n_splits=0, scale_mul=1.0,
             cap_extra=3, rows=None, check_logits=True, host=None, q=None, mask=None):
    """Oracle vs GPU on one input.  The outputs come from the production
    kernel (no debug outputs requested); a second call with debug outputs
    checks the int8 Q and the int32 logits bit for bit."""
    stv, torch = gpu
    rng = np.random.default_rng(seed)
    if host is None:
        host = synth.make_kv(rng, hkv, d, L + T, L + T + cap_extra)
    if q is None:
        q = synth.make_q(rng, T, hq, d)
    if mask is None and kind != "prefill":
        mask = _mask_for(rng, kind, T)
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
    flat_d = torch.from_numpy(flat).cuda()
    out = call(False)
    torch.cuda.synchronize()
    out_g = out.reshape(T * hq, d)[flat_d].cpu().numpy()
    lse_g = lse.reshape(-1)[flat_d].cpu().numpy()
    err = _row_err(out_g, ref["out"])
    assert np.all(np.isfinite(out_g))
    assert err.max() <= TOL, f"max row error {err.max():.3g}"
    assert np.max(np.abs(lse_g - ref["lse"])) <= TOL

    names = ("logits", "q8", "qscale") if check_logits else ("q8", "qscale")
    out2, dbg = call(names)
    torch.cuda.synchronize()
    q8 = dbg["q8"].reshape(T * hq, d)[flat_d].cpu().numpy()
    qs = dbg["qscale"].reshape(-1)[flat_d].cpu().numpy()
    assert np.array_equal(q8, ref["qi8"]), "int8 Q differs"
    assert np.array_equal(qs.view(np.uint32), ref["sq"].view(np.uint32)), "Q scale differs"
    if check_logits:
        lg = dbg["logits"].reshape(T * hq, L + T, d // 32)[flat_d].cpu().numpy()
        vis = _visible(T, L, mask, L + T)
        for i, r in enumerate(flat):
            v = vis[r // hq]
            assert np.array_equal(lg[i][v], ref["logits"][i][v]), f"int32 logits differ, row {r}"
    err2 = _row_err(out2.reshape(T * hq, d)[flat_d].cpu().numpy(), ref["out"])
    assert err2.max() <= TOL
    return out, err.max()


CASES = [
    # name,            Hq, Hkv,  D,    L,   T, kind,     seed, n_splits
    ("tiny_auto",        4, 1,   64,  512,   8, "chain",   0, 0),
    ("tiny_1split",      4, 1,   64,  512,   8, "chain",   0, 1),
    ("tiny_3split",      4, 1,   64,  512,   8, "chain",   0, 3),
    ("tree64_ragged",   24, 4,  256, 1000,  64, "tree",  101, 0),
    ("tree64_1split",   24, 4,  256,  333,  64, "tree",  102, 1),
    ("tree8_d128",       8, 2,  128,  777,   8, "tree",  103, 0),
    ("tree17_d128",      8, 2,  128,  333,  17, "tree",  104, 5),
    ("decode_t1",       24, 4,  256, 2049,   1, "tree",  105, 0),
    ("decode_t1_L0",    24, 4,  256,    0,   1, "tree",  106, 0),
    ("tree_L0",          4, 2,   64,    0,   5, "tree",  107, 0),
    ("tree_1key_ctx",    4, 2,   64,    1,  33, "tree",  108, 0),
    ("prefill_small",   12, 2,  128,  100,  70, "prefill", 109, 0),
    ("prefill_splits",  24, 4,  256,   64,  40, "prefill", 110, 4),
    ("prefill_L0",       6, 3,   64,    0,  97, "prefill", 111, 0),
    # 17..64 rows per KV head: the 16-row shared-tile kernel
    ("tree8_d256_r48",  24, 4,  256, 1234,   8, "tree",  112, 0),
    ("tree3_r18",       24, 4,  256,  500,   3, "tree",  113, 2),
    ("tree16_r64",       8, 2,  128,  300,  16, "tree",  114, 0),
    ("prefill_r60",     24, 4,  256,  200,  10, "prefill", 115, 3),
    ("prefill_r36_d64",  8, 2,   64,   50,   9, "prefill", 116, 0),
]


@pytest.mark.parametrize("name,hq,hkv,d,L,T,kind,seed,ns", CASES, ids=[c[0] for c in CASES])
def test_parity(gpu, orc, name, hq, hkv, d, L, T, kind, seed, ns):
    run_case(gpu, orc, hq, hkv, d, L, T, kind, seed, n_splits=ns)


@pytest.mark.parametrize("scale_mul", [8.0, 32.0])
def test_parity_peaked(gpu, orc, scale_mul):
    """Large logit scales make the softmax nearly one-hot (the workload's own
    distributions give diffuse attention, which averages errors away)."""
    run_case(gpu, orc, 24, 4, 256, 700, 16, "tree", 120, scale_mul=scale_mul)
    run_case(gpu, orc, 12, 2, 128, 90, 50, "prefill", 121, scale_mul=scale_mul)
    run_case(gpu, orc, 24, 4, 256, 900, 8, "tree", 124, scale_mul=scale_mul)     # 48 rows per KV head
    run_case(gpu, orc, 24, 4, 256, 1500, 1, "tree", 125, scale_mul=scale_mul)    # one token


def test_parity_planted_keys(gpu, orc):
    """Context keys whose codes follow sign(q) of one row dominate that row."""
    rng = np.random.default_rng(122)
    hq, hkv, d, L, T = 8, 2, 128, 400, 8
    host = synth.make_kv(rng, hkv, d, L + T, L + T)
    q = synth.make_q(rng, T, hq, d)
    for t in range(T):
        h = (3 * t) % hq
        j = int(rng.integers(0, L))
        codes = np.where(q[t, h] > 0, 7, 1).astype(int)
        for b in range(d // 32):
            host.k_codes[h // (hq // hkv), j, b] = orc.pack_block(codes[32 * b:32 * b + 32])
    run_case(gpu, orc, hq, hkv, d, L, T, "tree", 123, host=host, q=q)


def _f16_bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("kind,T", [("tree", 64), ("prefill", 40), ("prefill", 200),
                                    ("tree", 8), ("tree", 10), ("prefill", 8)])
def test_k_scale_exponent_spread(gpu, orc, kind, T):
    """Keys whose fp16 block scales span more than three binades, or hold
    zeros and subnormals, next to ordinary keys in one call.  For more than
    64 rows per KV head the kernel sums a key's blocks in int32 with integer
    scales when the spread allows it and takes the per-block fp32 epilogue
    for tiles where it does not; the 16-row kernel (48 and 60 rows: with and
    without its V-unpacking wave) takes the fp32 epilogue on every tile.  All
    match the oracle."""
    rng = np.random.default_rng(150 if kind == "tree" else 151)
    hq, hkv, d, L = 24, 4, 256, 2000
    host = synth.make_kv(rng, hkv, d, L + T, L + T + 3)
    ks = host.k_scales                       # [Hkv][cap][D/32], fp16 bits

    def key(tile, i):
        return 32 * tile + i

    # four binades (0.01 .. 0.2): the tile takes the fp32 epilogue
    ks[0, key(3, 5)] = _f16_bits([0.01, 0.2, 0.05, 0.05, 0.05, 0.05, 0.05, 0.05])
    # one block 64 times the others: fp32 epilogue
    ks[1, key(7, 0), 0] = _f16_bits(ks[1, key(7, 0), 0].view(np.float16).astype(np.float32) * 64)
    # exactly three binades (2^-7 and just under 2^-3): integer path
    ks[2, key(12, 9)] = _f16_bits([2**-7, 0.1249, 2**-7, 0.1249, 0.05, 0.02, 0.0625, 0.09])
    # every block subnormal
    ks[3, key(10, 31)] = _f16_bits(rng.uniform(1e-7, 5e-6, 8))
    # the smallest normal next to subnormals (one exponent for all)
    ks[2, key(14, 8)] = _f16_bits([2**-14, 2**-15, 2**-16, 2**-17] * 2)
    # zero blocks, and a key of zeros only
    ks[:, key(11, 2), ::3] = 0
    ks[1, key(13, 4)] = 0
    # a tree or chunk key (position >= L) with a wide spread
    ks[0, L + 2] = _f16_bits([0.001, 0.5, 0.05, 0.05, 0.05, 0.05, 0.05, 0.05])
    run_case(gpu, orc, hq, hkv, d, L, T, kind, 152, host=host)
    run_case(gpu, orc, hq, hkv, d, L, T, kind, 153, host=host, scale_mul=16.0)


@pytest.mark.parametrize("kind,T", [("tree", 64), ("prefill", 40), ("prefill", 200),
                                    ("tree", 8), ("prefill", 10)])
def test_k_scale_integer_sum_bound(gpu, orc, kind, T):
    """The largest sums the integer-scale path can meet.  Rows whose Q
    elements are all equal quantize to int8 +-127; keys with every code 0
    (k = -4) then give block sums of -+16,256, and their scales put seven
    blocks three binades above the eighth with the largest significand
    (65504 and 8188), so sum_b M_b * S_b = 16,256 * (7 * 16,376 + 2,047) in
    magnitude, 88% of the int32 range.  The int32 block sums stay bit-exact
    and the outputs match the oracle."""
    rng = np.random.default_rng(154 if kind == "tree" else 155)
    hq, hkv, d, L = 24, 4, 256, 700
    host = synth.make_kv(rng, hkv, d, L + T, L + T + 3)
    q = synth.make_q(rng, T, hq, d)
    q[:, 0::3] = 1.0
    q[:, 1::3] = -1.0
    heavy = rng.choice(L, 40, replace=False)
    zero_codes = orc.pack_block(np.zeros(32, dtype=int))
    scales = np.array([0x6FFF] + [0x7BFF] * 7, dtype=np.uint16)
    assert np.float16(scales.view(np.float16)[0]) == 8188 and scales.view(np.float16)[1] == 65504
    for j in heavy:
        host.k_codes[:, j] = zero_codes
        host.k_scales[:, j] = scales
    # logits of the heavy keys near +-6 for the equal-element rows
    run_case(gpu, orc, hq, hkv, d, L, T, kind, 156, host=host, q=q, scale_mul=1.6e-6)


IMAGE_CASES = [
    # Hq, Hkv, D, L, T, fmt, n_splits: eight or more groups of 128 rows per
    # KV head, where the causal chunk unpacks each tile once into images
    (24, 4, 256, 1500, 200, "b3", 0),
    (24, 4, 256, 333, 180, "b3", 3),
    (8, 1, 128, 700, 130, "b3", 0),
    (8, 2, 64, 901, 260, "b3", 2),
    (24, 4, 256, 0, 200, "b3", 0),          # no context keys: early row groups see few tiles
]


@pytest.mark.parametrize("hq,hkv,d,L,T,fmt,ns", IMAGE_CASES,
                         ids=[f"d{c[2]}_L{c[3]}_T{c[4]}_S{c[6]}" for c in IMAGE_CASES])
def test_prefill_tile_images(gpu, orc, hq, hkv, d, L, T, fmt, ns):
    """The causal chunk with many row groups: a pre-pass unpacks each tile
    once into the workspace and the kernel copies the images into LDS.  The
    result equals, bit for bit, the same call whose workspace holds only the
    partials (each row group unpacking the tiles itself), and matches the
    oracle on sampled rows, at every head_dim.  (The 4-bit format unpacks
    in the kernel: its plan asks for no image space.)"""
    stv, torch = gpu
    rng = np.random.default_rng(170 + d + T)
    host = synth.make_kv(rng, hkv, d, L + T, L + T + 5)
    S4, ws4 = stv.attention_plan(T, hq, hkv, d, L, True, ns, "i4")
    assert ws4 == stv.workspace_bytes(T, hq, d, S4)
    q = synth.make_q(rng, T, hq, d)
    S, ws_full = stv.attention_plan(T, hq, hkv, d, L, True, ns, fmt)
    part = stv.workspace_bytes(T, hq, d, S)
    assert ws_full > part, "the plan asks for image space"
    kv = stv.KVCache.from_host(host)
    qd = torch.from_numpy(q).cuda()
    lse_a = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    out_a = stv.prefill_attention(qd, kv, L, out_lse=lse_a, n_splits=ns)
    small = torch.empty(max(part, 16), dtype=torch.uint8, device="cuda")
    out_b = stv.prefill_attention(qd, kv, L, out_lse=lse_b, n_splits=ns, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    rows = np.unique(np.concatenate([[0, T * hq - 1], rng.integers(0, T * hq, 40)]))
    ref = orc.attention(q, host, L, None, 1.0 / math.sqrt(d), rows=rows)
    got = out_a.reshape(T * hq, d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert _row_err(got, ref["out"]).max() <= TOL
    lg = lse_a.reshape(-1)[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.max(np.abs(lg - ref["lse"])) <= TOL


def test_residue_sweep(gpu, orc):
    """Context lengths over every residue of the 32-key tile, and split
    boundaries moved with them (a length-dependent corruption shows up as
    a parity failure at one residue)."""
    rng = np.random.default_rng(130)
    for r in range(32):
        L = 2048 + r
        run_case(gpu, orc, 4, 1, 64, L, 8, "tree", 1000 + r, n_splits=int(rng.integers(0, 9)))


def test_all_8_row_tree_shapes(gpu, orc):
    """Every one of the 5,040 8-row tree shapes against the oracle."""
    stv, torch = gpu
    hq, hkv, d, L, T = 4, 1, 64, 40, 8
    rng = np.random.default_rng(131)
    host = synth.make_kv(rng, hkv, d, L + T, L + T)
    q = synth.make_q(rng, T, hq, d)
    kv = stv.KVCache.from_host(host)
    qd = torch.from_numpy(q).cuda()
    scale = 4.0 / math.sqrt(d)
    masks, outs = [], []
    for parent in synth.all_tree_shapes(T):
        m = synth.ancestor_masks(parent)
        masks.append(m)
        outs.append(stv.verify_attention(qd, kv, L, m, scale))
    torch.cuda.synchronize()
    worst = 0.0
    for m, o in zip(masks, outs):
        ref = orc.attention(q, host, L, m, scale)
        err = _row_err(o.reshape(T * hq, d).cpu().numpy(), ref["out"]).max()
        worst = max(worst, err)
    assert len(masks) == 5040
    assert worst <= TOL, worst


def test_determinism(gpu, orc):
    stv, torch = gpu
    rng = np.random.default_rng(140)
    host = synth.make_kv(rng, 4, 256, 5000 + 64, 5000 + 64)
    q = torch.from_numpy(synth.make_q(rng, 64, 24, 256)).cuda()
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, 64, 8))
    kv = stv.KVCache.from_host(host)
    a = stv.verify_attention(q, kv, 5000, mask)
    b = stv.verify_attention(q, kv, 5000, mask)
    c = stv.prefill_attention(q, kv, 5000)
    d2 = stv.prefill_attention(q, kv, 5000)
    # the 16-row and the few-row kernels: 8 rows and one row of the tree
    m8 = synth.ancestor_masks(synth.make_tree_parents(rng, 8, 8))
    e = stv.verify_attention(q[:8].contiguous(), kv, 5000, m8)
    f = stv.verify_attention(q[:8].contiguous(), kv, 5000, m8)
    g1 = stv.verify_attention(q[:1].contiguous(), kv, 5000, mask[:1])
    h1 = stv.verify_attention(q[:1].contiguous(), kv, 5000, mask[:1])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d2)
    assert torch.equal(e, f) and torch.equal(g1, h1)


def test_determinism_rows_1_to_8(gpu, orc):
    """Tree row counts 1..8 (the few-row and 16-row kernels), each call
    repeated: bitwise-identical outputs and lse."""
    stv, torch = gpu
    rng = np.random.default_rng(141)
    host = synth.make_kv(rng, 4, 256, 7000 + 8, 7000 + 8)
    kv = stv.KVCache.from_host(host)
    for T in range(1, 9):
        q = torch.from_numpy(synth.make_q(rng, T, 24, 256)).cuda()
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8) if T > 1
                                    else synth.chain_parents(1))
        outs = []
        for _ in range(3):
            lse = torch.empty((T, 24), dtype=torch.float32, device="cuda")
            o = stv.verify_attention(q, kv, 7000, mask, out_lse=lse)
            outs.append((o, lse))
        torch.cuda.synchronize()
        for o, lse in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1]), T


def test_split_merge_parity(gpu, orc):
    stv, torch = gpu
    rng = np.random.default_rng(150)
    for S, rows, d in ((1, 5, 64), (7, 33, 256), (64, 3, 128), (3, 10, 200), (2, 1001, 256),
                       (8, 77, 128), (9, 40, 64)):
        po = rng.standard_normal((S, rows, d)).astype(np.float32)
        pl = (rng.standard_normal((S, rows)) * 5).astype(np.float32)
        pl[rng.random((S, rows)) < 0.2] = -np.inf
        pl[:, 0] = -np.inf                              # a row no split saw
        out_ref, lse_ref = orc.merge(po.astype(np.float64), pl.astype(np.float64))
        out_lse = torch.empty(rows, dtype=torch.float32, device="cuda")
        out = stv.split_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                              out_lse=out_lse)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        ls = out_lse.cpu().numpy()
        empty = ~np.isfinite(lse_ref)                   # rows no split saw
        assert empty[0]
        assert np.all(o[empty] == 0) and np.all(ls[empty] == -np.inf)
        seen = ~empty
        err = np.max(np.abs(o[seen] - out_ref[seen]), axis=-1) / np.max(np.abs(out_ref[seen]), axis=-1)
        assert err.max() <= 1e-5
        assert np.max(np.abs(ls[seen] - lse_ref[seen])) <= 1e-5 * np.max(np.abs(lse_ref[seen]) + 1)


def test_kv_quant_pack_parity(gpu, orc):
    """GPU pack of K and V against the oracle's pack, bit for bit, including
    appends that start and end inside a 32-key group of V."""
    stv, torch = gpu
    rng = np.random.default_rng(160)
    for hkv, d, cap, n, pos0 in ((4, 256, 300, 64, 17), (1, 64, 50, 7, 43), (2, 128, 4200, 4096, 100),
                                 (2, 64, 96, 1, 95), (3, 128, 70, 33, 0)):
        x = (rng.standard_normal((n, hkv, d)) * 10.0 ** rng.uniform(-3, 3, (n, hkv, 1))).astype(np.float32)
        x[0, 0, :32] = 0.0                         # zero block
        x[min(1, n - 1), 0, 32:64] = 1e-9          # scale rounds to zero
        x[n - 1, hkv - 1, :32] = 1e6               # scale saturates
        host = synth.make_kv(rng, hkv, d, cap, cap)     # random old contents everywhere
        kv = stv.KVCache.from_host(host)
        xd = torch.from_numpy(x).cuda()
        stv.kv_quant_pack(xd, pos0, kv, "k")
        stv.kv_quant_pack(xd, pos0, kv, "v")
        torch.cuda.synchronize()
        orc.kv_quant_pack(x, pos0, host.k_codes, host.k_scales, "k")
        orc.kv_quant_pack(x, pos0, host.v_codes, host.v_scales, "v")
        assert np.array_equal(kv.k_codes.cpu().numpy().view(np.uint32), host.k_codes)
        assert np.array_equal(kv.k_scales.cpu().numpy().view(np.uint16), host.k_scales)
        assert np.array_equal(kv.v_codes.cpu().numpy().view(np.uint32), host.v_codes)
        assert np.array_equal(kv.v_scales.cpu().numpy().view(np.uint16), host.v_scales)


def test_pack_then_verify_end_to_end(gpu, orc):
    """The new rows' K/V go through kv_quant_pack, then attention reads only
    the cache: both sides run the same sequence."""
    stv, torch = gpu
    rng = np.random.default_rng(170)
    hq, hkv, d, L, T = 24, 4, 256, 3000, 16
    host = synth.make_kv(rng, hkv, d, L, L + T)
    knew = rng.standard_normal((T, hkv, d)).astype(np.float32)
    vnew = rng.standard_normal((T, hkv, d)).astype(np.float32)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8))
    kv = stv.KVCache.from_host(host)
    stv.kv_quant_pack(torch.from_numpy(knew).cuda(), L, kv, "k")
    stv.kv_quant_pack(torch.from_numpy(vnew).cuda(), L, kv, "v")
    out = stv.verify_attention(torch.from_numpy(q).cuda(), kv, L, mask)
    torch.cuda.synchronize()
    orc.kv_quant_pack(knew, L, host.k_codes, host.k_scales, "k")
    orc.kv_quant_pack(vnew, L, host.v_codes, host.v_scales, "v")
    ref = orc.attention(q, host, L, mask)
    err = _row_err(out.reshape(T * hq, d).cpu().numpy(), ref["out"])
    assert err.max() <= TOL


# Full-size workloads, in the launch configuration the benchmark times (the
# automatic split plan), checked on rows the oracle computes one by one.
# The int32 logits are checked on the sampled rows wherever the debug buffer
# ([T*Hq][L+T][D/32] int32) stays within a few GB of device memory: 12.9 GB at
# the 64-node tree over 262K; the prefill chunk's 116 GB is left out.
FULL = [(g, r) for g, r in [(synth.CONFIGS[1], 24), (synth.CONFIGS[2], 16), (synth.CONFIGS[3], 64),
                            (synth.CONFIGS[4], 32), (synth.EXTRA_CONFIGS[0], 24),
                            (synth.EXTRA_CONFIGS[1], 24)]]


@pytest.mark.parametrize("geom,n_rows", FULL, ids=[g.name for g, _ in FULL])
def test_full_size_sampled(gpu, orc, geom, n_rows):
    rng = np.random.default_rng(geom.seed)
    host = synth.make_kv(rng, geom.n_kv_heads, geom.head_dim, geom.n_keys)
    q = synth.make_q(rng, geom.n_rows, geom.n_q_heads, geom.head_dim)
    kind = "prefill" if geom.kind == "prefill" else "tree"
    mask = None
    if kind == "tree":
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, geom.n_rows, geom.max_depth))
    total = geom.n_rows * geom.n_q_heads
    pick = np.random.default_rng(geom.seed + 100)
    rows = np.unique(np.concatenate([[0, total - 1], pick.integers(0, total, n_rows - 2)]))
    run_case(gpu, orc, geom.n_q_heads, geom.n_kv_heads, geom.head_dim, geom.ctx_len,
             geom.n_rows, kind, geom.seed, host=host, q=q, mask=mask, rows=rows,
             check_logits=kind == "tree")


PLANTED = [g for g in synth.CONFIGS + synth.EXTRA_CONFIGS if g.name in ("tree64_262k", "tree8_262k")]


@pytest.mark.parametrize("geom", PLANTED, ids=[g.name for g in PLANTED])
def test_full_size_planted(gpu, orc, geom):
    """Dominant keys at 262,144 context, in the automatic split plan: for one
    row of each KV head, six keys whose codes follow the signs of that row's
    query and whose K scales (0.30 .. 0.50) put them 11 to 19 nats above the
    rest -- inside three different splits, on both sides of one split
    boundary, and at the root's tree key in the last tile, which every row
    sees.  The softmax then weighs a few keys in different splits against
    each other and against 262K diffuse ones, which tests the merge far more
    than the workload's own near-uniform attention does."""
    stv, _ = gpu
    rng = np.random.default_rng(geom.seed + 50)
    hq, hkv, d, L, T = (geom.n_q_heads, geom.n_kv_heads, geom.head_dim, geom.ctx_len,
                        geom.n_rows)
    host = synth.make_kv(rng, hkv, d, geom.n_keys)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, geom.max_depth))
    S, _ = stv.attention_plan(T, hq, hkv, d, L, False, 0)
    assert S >= 8
    P = 32 * -(-(-(-geom.n_keys // 32)) // S)
    G = hq // hkv
    positions = [s * P + P // 2 for s in (1, S // 2, S - 2)] + [P * (S // 3) - 1, P * (S // 3), L]
    strengths = [0.30, 0.34, 0.38, 0.42, 0.46, 0.50]
    planted = []
    for g in range(hkv):
        t, h = int(rng.integers(0, T)), g * G + int(rng.integers(0, G))
        codes = np.where(q[t, h] > 0, 7, 1).astype(int)
        blocks = np.stack([orc.pack_block(codes[32 * b:32 * b + 32]) for b in range(d // 32)])
        for j, sk in zip(positions, strengths):
            host.k_codes[g, j] = blocks
            host.k_scales[g, j] = np.float16(sk).view(np.uint16)
        planted.append(t * hq + h)
    pick = np.random.default_rng(geom.seed + 51)
    rows = np.unique(np.concatenate([planted, pick.integers(0, T * hq, 60)]))
    ref = run_case(gpu, orc, hq, hkv, d, L, T, "tree", 0, host=host, q=q, mask=mask, rows=rows,
                   check_logits=False)
    # the planted rows really are dominated by their planted keys
    got = orc.attention(q, host, L, mask, 1.0 / math.sqrt(d), rows=planted)
    lse_ctx = orc.attention(q, host, L, mask, 1.0 / math.sqrt(d), rows=planted,
                            k_begin=0, k_end=P)["lse"]
    assert np.all(got["lse"] - lse_ctx > 5.0), got["lse"] - lse_ctx
    assert ref is not None


@pytest.mark.parametrize("T", [1, 8])
def test_context_length_sweep(gpu, orc, T):
    """Error against the fp64 oracle at ten context lengths from 1 to
    262,143 keys (one token and the 8-row tree, automatic split plan)."""
    worst = []
    for i, L in enumerate([1, 100, 1000, 4095, 8192, 16385, 32768, 65537, 131072, 262143]):
        rng = np.random.default_rng(600 + 10 * T + i)
        host = synth.make_kv(rng, 4, 256, L + T)
        q = synth.make_q(rng, T, 24, 256)
        mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8) if T > 1
                                    else synth.chain_parents(1))
        rows = np.unique(np.linspace(0, T * 24 - 1, 8).round().astype(np.int32))
        _, err = run_case(gpu, orc, 24, 4, 256, L, T, "tree", 0, rows=rows, host=host, q=q,
                          mask=mask, check_logits=L <= 16385)
        worst.append(err)
    print(f"T={T}: max row error per context length {['%.2g' % e for e in worst]}")


def test_partials_then_merge_equals_verify(gpu, orc):
    """The split phase plus the merge entry point reproduce the verify call
    bit for bit (the verify call runs exactly these two kernels)."""
    stv, torch = gpu
    rng = np.random.default_rng(180)
    hq, hkv, d, L, T = 24, 4, 256, 9000, 12
    host = synth.make_kv(rng, hkv, d, L + T)
    q = torch.from_numpy(synth.make_q(rng, T, hq, d)).cuda()
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8))
    kv = stv.KVCache.from_host(host)
    lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    out = stv.verify_attention(q, kv, L, mask, out_lse=lse)
    po, pl = stv.attention_partials(q, kv, L, mask)
    S = po.shape[0]
    assert S > 1
    lse2 = torch.empty(T * hq, dtype=torch.float32, device="cuda")
    out2 = stv.split_merge(po.reshape(S, T * hq, d), pl.reshape(S, T * hq), out_lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(T * hq, d), out2)
    assert torch.equal(lse.reshape(-1), lse2)
    # the partials themselves match the oracle's partials over the same key ranges
    n_keys = L + T
    split_len = 32 * -(-(-(-n_keys // 32)) // S)        # 32 * ceil(ceil(N / 32) / S)
    qh = q.cpu().numpy()
    for s in (0, S // 2, S - 1):
        k0, k1 = s * split_len, min(n_keys, (s + 1) * split_len)
        ref = orc.attention(qh, host, L, mask, k_begin=k0, k_end=k1, rows=[0, 7, T * hq - 1])
        got = po[s].reshape(T * hq, d)[[0, 7, T * hq - 1]].cpu().numpy()
        assert _row_err(got, ref["out"]).max() <= TOL
        gl = pl[s].reshape(-1)[[0, 7, T * hq - 1]].cpu().numpy()
        assert np.max(np.abs(gl - ref["lse"])) <= TOL


@pytest.mark.parametrize("hq,hkv,n_splits", [(24, 4, 5), (24, 4, 22), (6, 1, 1), (6, 1, 3),
                                             (32, 4, 7), (8, 1, 43)])
def test_wave_specialized_item_runs(gpu, orc, hq, hkv, n_splits):
    """The wave-specialized kernel (3-bit, head_dim 256, 64 tree rows) sends
    work item w = (head * S + split) * row groups + row group to the XCD run
    w / ceil(items / 8).  Item counts that are not multiples of eight, runs
    shorter than eight and more than one round: the partials go into
    NaN-filled buffers, so an item that no work-group computes shows, and the
    partials of sampled splits match the oracle's over the same key ranges on
    rows of every row group, so one computed for the wrong split or written to
    the wrong place shows too.  The merge matches the one-split call."""
    stv, torch = gpu
    T, d, L = 64, 256, 6000          # 190 tiles: 22 splits stay 22 (264 items, two rounds)
    rng = np.random.default_rng(1200 + 100 * hq + n_splits)
    host = synth.make_kv(rng, hkv, d, L + T)
    kv = stv.KVCache.from_host(host)
    q = torch.from_numpy(synth.make_q(rng, T, hq, d)).cuda()
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8))
    S, _ = stv.attention_plan(T, hq, hkv, d, L, False, n_splits)
    po = torch.full((S, T, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((S, T, hq), float("nan"), dtype=torch.float32, device="cuda")
    stv.attention_partials(q, kv, L, mask, n_splits=n_splits, part_o=po, part_lse=pl)
    torch.cuda.synchronize()
    assert not torch.isnan(po).any() and not torch.isnan(pl).any()
    n_keys = L + T
    split_len = 32 * -(-(-(-n_keys // 32)) // S)        # 32 * ceil(ceil(N / 32) / S)
    rows = np.unique(np.linspace(0, T * hq - 1, 16).round().astype(np.int64))
    qh = q.cpu().numpy()
    for s in sorted({0, 1 % S, S // 2, S - 1}):
        k0, k1 = s * split_len, min(n_keys, (s + 1) * split_len)
        ref = orc.attention(qh, host, L, mask, k_begin=k0, k_end=k1, rows=rows)
        got = po[s].reshape(T * hq, d)[torch.from_numpy(rows).cuda()].cpu().numpy()
        assert _row_err(got, ref["out"]).max() <= TOL, f"split {s}"
        gl = pl[s].reshape(-1)[torch.from_numpy(rows).cuda()].cpu().numpy()
        # a row that sees no key of the split (the last one holds only tree
        # keys here) has lse -inf on both sides
        same = gl == ref["lse"]
        assert np.all(same | (np.abs(gl - ref["lse"]) <= TOL)), f"split {s}"
    out = stv.split_merge(po.reshape(S, T * hq, d), pl.reshape(S, T * hq))
    one = stv.verify_attention(q, kv, L, mask, n_splits=1)
    torch.cuda.synchronize()
    assert _row_err(out.cpu().numpy(), one.reshape(T * hq, d).cpu().numpy()).max() <= TOL


# (query heads per KV head, tree rows): rows per KV head on both sides of
# each kernel boundary (16 | 17: few-row / 16-row; 32 | 33; 64 | 65: 16-row /
# 32-row; 96 | 97: two / four row tiles per work-group), and the largest.
_BOUNDARY_SHAPES = [(1, 16), (1, 17), (2, 8), (2, 9), (2, 16), (2, 17), (2, 32), (2, 33),
                    (2, 48), (2, 49), (6, 2), (6, 3), (6, 5), (6, 6), (6, 10), (6, 11),
                    (6, 16), (6, 17), (8, 4), (8, 8), (8, 12), (8, 13), (3, 22), (3, 32),
                    (6, 64), (8, 64), (1, 64), (4, 25)]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("T,ns", [(8, 0), (8, 3), (10, 0), (10, 2)])
def test_16row_kernel_roles(gpu, orc, d, T, ns):
    """The 16-row kernel (17 to 64 rows per KV head) at each head dim: 48 rows
    (T = 8, GQA group 6), where the work-group's fourth wave has no rows and
    unpacks every V row while the other three unpack K, and 60 rows (T = 10),
    where all four waves compute and every thread unpacks one K item and one
    V row; a ragged context (1,000 keys: a partial last tile per split)."""
    rows = np.arange(T * 6)
    run_case(gpu, orc, 6, 1, d, 1000, T, "tree", 1700 + 10 * T + d // 64 + ns, n_splits=ns,
             rows=rows)


def test_shape_sweep_kernel_boundaries(gpu, orc):
    """Seeded shapes on both sides of every boundary of the plan's kernel
    choice, over the head dims, context lengths (including none) and split
    counts: outputs and lse against the oracle on sampled rows, int8 Q and
    int32 logits bit for bit."""
    rng = np.random.default_rng(1300)
    for i, (g, T) in enumerate(_BOUNDARY_SHAPES):
        hkv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128, 256]))
        L = int(rng.choice([0, 1, 31, 33, 700, 2049, 3000]))
        ns = int(rng.choice([0, 0, 1, 2, 3, 5, 7]))
        hq = g * hkv
        rows = np.unique(np.linspace(0, T * hq - 1, 12).round().astype(np.int64))
        run_case(gpu, orc, hq, hkv, d, L, T, "tree", 1400 + i, n_splits=ns, rows=rows)
