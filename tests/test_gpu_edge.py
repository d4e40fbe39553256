"""GPU parity on shapes and values the ABI accepts that the workloads do not
produce: all-zero query rows, forests of draft paths, a chain of 64 (mask
bit 63), and V block scales far above the workloads' U(0.01, 0.1).  Each
runs through the kernel that owns its row count (at most 16 rows per KV
head: the few-row kernel; 17..64: the 16-row kernel; more: the 32-row
kernel) and is compared with the oracle as in test_gpu_parity.
"""
import math

import numpy as np
import pytest

import synth
from test_gpu_parity import TOL, _row_err, run_case

pytestmark = pytest.mark.gpu

# (T, heads) that select each kernel with 24 query / 4 KV heads (6 rows per
# tree row and KV head): T = 1, 2 -> few-row; 3..10 -> 16-row; >= 11 -> 32-row
KERNEL_T = [(1, "few-row"), (8, "16-row"), (64, "32-row")]


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_tree_verify_amd as stv
    stv.load_library()
    return stv, torch


def _decode3(words):
    """Codes of 3-word blocks in the byte-plane layout, read by this file
    alone: element e = 4 qq + i sits in word qq // 2 at bits 8i + 3 (qq % 2)
    for qq < 6; for qq = 6, 7 its two low bits are word qq - 6 bits 8i + 6,
    its high bit word 2 bit 8i + 6 + (qq - 6).  [..., 3] -> [..., 32]."""
    w = words.astype(np.int64)
    out = np.empty(words.shape[:-1] + (32,), dtype=np.int64)
    for qq in range(8):
        for i in range(4):
            if qq < 6:
                c = (w[..., qq // 2] >> (8 * i + 3 * (qq % 2))) & 7
            else:
                lo = (w[..., qq - 6] >> (8 * i + 6)) & 3
                c = lo | (((w[..., 2] >> (8 * i + 6 + qq - 6)) & 1) << 2)
            out[..., 4 * qq + i] = c
    return out


def _v_hat(host, g):
    """Dequantized V of KV head g, [keys][D] in fp64."""
    codes = _decode3(host.v_codes[g])                       # [ng][D][32 keys]
    s = host.v_scales[g].view(np.float16).astype(np.float64)  # [ng][NB][32 keys]
    s = np.repeat(s, 32, axis=1)                            # [ng][D][32 keys]
    v = s * (codes - 4)
    return v.transpose(0, 2, 1).reshape(-1, host.head_dim)


@pytest.mark.parametrize("T,kernel", KERNEL_T, ids=[k for _, k in KERNEL_T])
def test_zero_q_rows(gpu, orc, T, kernel):
    """All-zero query rows (the prologue's sq = 0 branch) next to ordinary
    rows.  Such a row's logits are all 0, so its output is the plain mean of
    the V rows it sees (the closed form the oracle is pinned to)."""
    rng = np.random.default_rng(700 + T)
    hq, hkv, d, L = 24, 4, 256, 1500
    host = synth.make_kv(rng, hkv, d, L + T, L + T + 2)
    q = synth.make_q(rng, T, hq, d)
    q[0, :] = 0.0                      # every head of tree row 0
    q[T - 1, 7] = 0.0                  # one head of the last row
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8) if T > 1
                                else synth.chain_parents(1))
    out, _ = run_case(gpu, orc, hq, hkv, d, L, T, "tree", 0, host=host, q=q, mask=mask)
    got = out.reshape(T, hq, d).cpu().numpy()
    vh = [_v_hat(host, g) for g in range(hkv)]
    # the test's reader agrees with the oracle's on a few keys
    for j in (0, 31, L - 1, L + T - 1):
        assert np.array_equal(vh[1][j], orc.v_values(host, 1, j))
    for t, h in [(0, 0), (0, 13), (0, hq - 1), (T - 1, 7)]:
        keys = list(range(L)) + [L + a for a in range(T) if (int(mask[t]) >> a) & 1]
        mean = np.mean(vh[h // (hq // hkv)][keys], axis=0)
        err = np.max(np.abs(got[t, h] - mean)) / np.max(np.abs(mean))
        assert err <= TOL, (t, h, err)


FOREST = [(2, np.array([-1, -1])),                                   # two roots: few-row
          (8, np.array([-1, 0, -1, 2, 0, 3, -1, 6])),               # three trees: 16-row
          (40, None)]                                               # random forest: 32-row


@pytest.mark.parametrize("T,parent", FOREST, ids=["few-row", "16-row", "32-row"])
def test_forest_masks(gpu, orc, T, parent):
    """Masks of several trees (rows whose mask holds only their own bit start
    a new tree): every kernel honours each row's own path."""
    rng = np.random.default_rng(720 + T)
    if parent is None:
        parent = synth.make_tree_parents(rng, T, 8)
        parent[[5, 17, 30]] = -1                   # detach three subtrees
    mask = synth.ancestor_masks(parent)
    assert sum(int(m).bit_count() == 1 for m in mask) >= 2
    run_case(gpu, orc, 24, 4, 256, 900, T, "tree", 721 + T, mask=mask)
    run_case(gpu, orc, 24, 4, 256, 900, T, "tree", 722 + T, mask=mask, scale_mul=8.0)


def test_chain_of_64(gpu, orc):
    """A chain of 64 draft rows: row 63's mask holds bit 63 (every other
    mask bit too).  Compared with the oracle, and with the causal chunk of 64
    rows, which the oracle pins bit for bit to the chain."""
    stv, torch = gpu
    T, hq, hkv, d, L = 64, 24, 4, 256, 700
    rng = np.random.default_rng(730)
    host = synth.make_kv(rng, hkv, d, L + T, L + T)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.chain_parents(T))
    assert int(mask[63]) == (1 << 64) - 1
    out, _ = run_case(gpu, orc, hq, hkv, d, L, T, "chain", 731, host=host, q=q, mask=mask)
    kv = stv.KVCache.from_host(host)
    causal = stv.prefill_attention(torch.from_numpy(q).cuda(), kv, L)
    torch.cuda.synchronize()
    # same kernel family and split plan, the visibility test in another form
    err = _row_err(out.reshape(T * hq, d).cpu().numpy(), causal.reshape(T * hq, d).cpu().numpy())
    assert err.max() <= TOL


def _set_v_scales(rng, host, lo, hi, L):
    """Context V block scales drawn log-uniform in [lo, hi] (fp16 bits)."""
    nb = host.head_dim // 32
    s = np.exp(rng.uniform(np.log(lo), np.log(hi), size=host.v_scales.shape))
    bits = s.astype(np.float16).view(np.uint16)
    ng_ctx = -(-L // 32)
    host.v_scales[:, :ng_ctx] = bits[:, :ng_ctx]
    assert host.v_scales.shape[2] == nb


LARGE_V = [(1, 6.55e4, "few-row"), (2, 6.55e4, "few-row"), (8, 1.6e4, "16-row"),
           (64, 1.6e4, "32-row")]


@pytest.mark.parametrize("T,hi,kernel", LARGE_V, ids=[f"{k}_T{t}" for t, _, k in LARGE_V])
def test_large_v_scales_pack_then_verify(gpu, orc, T, hi, kernel):
    """V block scales from 1e2 up to the fp16 range, with the new rows' K/V
    packed on the GPU first (values up to ~2e5, scales up to 65504 for the
    few-row kernel).  The few-row kernel multiplies P by the V scale in
    fp16, so a tile with a scale of 256 or more bounds P by 1; the 16-row and
    32-row kernels dequantize V to s (c - 4) in fp16, which holds scales up
    to 16,376 (the range include/stv.h states)."""
    stv, torch = gpu
    rng = np.random.default_rng(740 + T)
    hq, hkv, d, L = 24, 4, 256, 2000
    host = synth.make_kv(rng, hkv, d, L, L + T)
    _set_v_scales(rng, host, 1e2, hi, L)
    knew = synth.make_new_rows(rng, T, hkv, d)
    # block scales amax / 3 of about hi / 4 at four standard deviations
    vnew = (synth.make_new_rows(rng, T, hkv, d) * (hi / 4.0)).astype(np.float32)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8) if T > 1
                                else synth.chain_parents(1))
    kv = stv.KVCache.from_host(host)
    stv.kv_quant_pack(torch.from_numpy(knew).cuda(), L, kv, "k")
    stv.kv_quant_pack(torch.from_numpy(vnew).cuda(), L, kv, "v")
    torch.cuda.synchronize()
    orc.kv_quant_pack(knew, L, host.k_codes, host.k_scales, "k")
    orc.kv_quant_pack(vnew, L, host.v_codes, host.v_scales, "v")
    assert np.array_equal(kv.v_scales.cpu().numpy().view(np.uint16), host.v_scales)
    assert np.array_equal(kv.v_codes.cpu().numpy().view(np.uint32), host.v_codes)
    vmax = np.max(host.v_scales.view(np.float16).astype(np.float64))
    assert vmax > (1e4 if hi > 2e4 else 4e3)
    for scale_mul in (1.0, 8.0):
        run_case(gpu, orc, hq, hkv, d, L, T, "tree", 0, host=host, q=q, mask=mask,
                 scale_mul=scale_mul)


def test_large_v_scales_4bit_few_row(gpu, orc):
    """The 4-bit cache in the few-row kernel (up to 64 rows per KV head)
    with V scales up to 8,000: P times the key's V scale stays in fp16."""
    stv, torch = gpu
    rng = np.random.default_rng(760)
    hq, hkv, d, L, T = 24, 4, 256, 1800, 8
    host = synth.make_kv4(rng, hkv, d, L + T)
    s = np.exp(rng.uniform(np.log(1e2), np.log(8e3), size=host.v_scales.shape))
    host.v_scales[:] = s.astype(np.float16).view(np.uint16)
    q = synth.make_q(rng, T, hq, d)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8))
    kv = stv.KVCache.from_host(host)
    out = stv.verify_attention(torch.from_numpy(q).cuda(), kv, L, mask, 8.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ref = orc.attention(q, host, L, mask, 8.0 / math.sqrt(d))
    got = out.reshape(T * hq, d).cpu().numpy()
    assert np.all(np.isfinite(got))
    assert _row_err(got, ref["out"]).max() <= TOL
