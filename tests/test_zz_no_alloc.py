"""GPU: the verify entry point that allocates nothing
(stv_verify_attention_noalloc), for callers that cannot allocate device
memory.  Its split partials live in the library's per-GPU scratch array; it
must give what stv_verify_attention gives at the same split count, bit for
bit, on consecutive calls that reuse the array (the second one smaller), and
match the oracle within the parity tolerance."""
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
    return np.max(np.abs(got - ref), axis=-1) / np.max(np.abs(ref), axis=-1)


def _case(stv, torch, orc, hq, hkv, d, L, T, seed, n_splits_ref=0, fmt="b3"):
    rng = np.random.default_rng(seed)
    host = (synth.make_kv4 if fmt == "i4" else synth.make_kv)(rng, hkv, d, L + T)
    q = torch.from_numpy(synth.make_q(rng, T, hq, d)).cuda()
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8))
    kv = stv.KVCache.from_host(host)
    lse_a = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    a = stv.verify_attention(q, kv, L, mask, out_lse=lse_a, n_splits=n_splits_ref)
    b = stv.verify_attention_noalloc(q, kv, L, mask, out_lse=lse_b)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(lse_a, lse_b)
    rows = np.unique(np.linspace(0, T * hq - 1, 12).round().astype(np.int32))
    ref = orc.attention(q.cpu().numpy(), host, L, mask, 1.0 / math.sqrt(d), rows=rows)
    got = b.reshape(T * hq, d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert _row_err(got, ref["out"]).max() <= TOL


def test_noalloc_two_calls_then_smaller(gpu, orc):
    stv, torch = gpu
    # 64-node tree over 20K keys: some 20 splits of 1.6 MB partials in the scratch
    S1, ws1 = stv.attention_plan(64, 24, 4, 256, 20000, False, 0)
    assert S1 > 1 and ws1 <= stv.noalloc_scratch_bytes()
    _case(stv, torch, orc, 24, 4, 256, 20000, 64, 950)
    # then a smaller call reusing the array: the 8-row tree over 3K keys
    _case(stv, torch, orc, 24, 4, 256, 3000, 8, 951)


def test_noalloc_caps_the_automatic_split_count(gpu, orc):
    """A shape whose automatic plan's partials would pass the 64 MiB array:
    the call takes as many splits as fit, and then equals the workspace entry
    point asked for that count.  The split count follows the device's
    occupancy, so the first of a few 64-node-tree shapes whose plan passes the
    array is used: the 4-bit format's 32-row kernel fills two work-groups per
    CU once (32 query / 4 KV heads: 32 splits of 2.1 MB), while the 3-bit
    wave-specialized kernel's one round of one work-group per CU stays below
    the array at 64 rows."""
    stv, torch = gpu
    T, d, L = 64, 256, 8000
    for hq, hkv, fmt in ((32, 4, "i4"), (64, 4, "i4"), (32, 4, "b3"), (128, 1, "b3")):
        S_auto, ws_auto = stv.attention_plan(T, hq, hkv, d, L, False, 0, fmt)
        if ws_auto > stv.noalloc_scratch_bytes():
            break
    else:
        pytest.skip("no candidate's automatic plan passes the scratch on this device")
    fit = stv.noalloc_scratch_bytes() // (T * hq * (d + 1) * 4)
    assert 1 < fit < S_auto
    _case(stv, torch, orc, hq, hkv, d, L, T, 952, n_splits_ref=int(fit), fmt=fmt)


def test_noalloc_rejects_too_many_splits(gpu):
    stv, torch = gpu
    rng = np.random.default_rng(953)
    T, hq, hkv, d, L = 64, 24, 4, 256, 9000
    host = synth.make_kv(rng, hkv, d, L + T)
    kv = stv.KVCache.from_host(host)
    q = torch.from_numpy(synth.make_q(rng, T, hq, d)).cuda()
    mask = synth.ancestor_masks(synth.chain_parents(T))
    fit = stv.noalloc_scratch_bytes() // (T * hq * (d + 1) * 4)
    # twice what fits: the plan rounds a requested count to whole tiles per
    # split, and this one stays above the fit after rounding
    ask = 2 * int(fit)
    S, _ = stv.attention_plan(T, hq, hkv, d, L, False, ask)
    assert S > fit
    with pytest.raises(stv.StvError) as e:
        stv.verify_attention_noalloc(q, kv, L, mask, n_splits=ask)
    assert e.value.code == stv.STV_EWORKSPACE
