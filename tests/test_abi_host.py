"""Host-side checks of the C-ABI library: it loads, exports every entry point
that include/stv.h declares, and rejects bad arguments before any HIP call.

No test here makes a call that passes validation with a device pointer, so
nothing is ever launched: valid masks are exercised by pairing them with a
workspace that is too small, which the library checks after the mask.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stv.h")
FAKE = 0x10000          # never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def lib():
    import speculative_tree_verify_amd as stv
    if not os.path.exists(stv.LIB_PATH):
        from speculative_tree_verify_amd import build_lib
        build_lib.build()
    return stv.load_library()


@pytest.fixture(scope="module")
def stvmod():
    import speculative_tree_verify_amd as stv
    return stv


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(stv_[a-z_0-9]+)\(", text, re.M)))


def test_header_declares_the_four_operations():
    names = _declared()
    for op in ("stv_kv_quant_pack", "stv_verify_attention", "stv_prefill_attention",
               "stv_split_merge", "stv_attention_plan", "stv_last_error", "stv_abi_version",
               "stv_tree_accept", "stv_kv_commit", "stv_lookup_plan", "stv_lookup_draft",
               "stv_verify_attention_fp16acc", "stv_context_plan", "stv_context_partials",
               "stv_workspace_bytes", "stv_verify_attention_noalloc",
               "stv_noalloc_scratch_bytes"):
        assert op in names


def test_library_exports_every_declared_symbol(lib, stvmod):
    out = subprocess.run(["nm", "-D", "--defined-only", stvmod.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(\S+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.stv_abi_version() == 5 == stvmod.ABI_VERSION
    # the header states the same version
    with open(os.path.join(ROOT, "include", "stv.h")) as f:
        assert re.search(r"Currently 5\b", f.read())


def _layer(stvmod, hkv=4, d=256, cap=1000):
    return stvmod._KVLayer(FAKE, FAKE, FAKE, FAKE, hkv, d, cap)


def _verify(lib, stvmod, T=8, hq=24, layer=None, L=100, mask=None, scale=0.0625, out=FAKE,
            ws=None, ws_bytes=0, n_splits=0, q=FAKE):
    layer = layer or _layer(stvmod)
    if mask is None:
        mask = synth.ancestor_masks(synth.chain_parents(T))
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint64))
    return lib.stv_verify_attention(q, T, hq, ctypes.byref(layer), L,
                                    m.ctypes.data if m.size else None, scale, out, None,
                                    ws, ws_bytes, n_splits, None, None, None, None)


def _err(lib):
    return lib.stv_last_error().decode()


def test_verify_argument_errors(lib, stvmod):
    E = stvmod
    assert _verify(lib, stvmod, T=0, mask=np.zeros(0)) == E.STV_EINVAL
    assert _verify(lib, stvmod, T=65, mask=np.zeros(65)) == E.STV_EINVAL
    assert "64" in _err(lib)
    assert _verify(lib, stvmod, hq=25) == E.STV_EINVAL                          # Hq % Hkv
    assert _verify(lib, stvmod, layer=_layer(stvmod, d=96)) == E.STV_EINVAL     # D % 32 == 0 but unsupported
    assert _verify(lib, stvmod, layer=_layer(stvmod, d=100)) == E.STV_EINVAL
    assert _verify(lib, stvmod, layer=_layer(stvmod, hkv=0)) == E.STV_EINVAL
    assert _verify(lib, stvmod, L=993) == E.STV_ECAPACITY                       # 993 + 8 > 1000
    assert "capacity" in _err(lib)
    assert _verify(lib, stvmod, L=-1) == E.STV_EINVAL
    assert _verify(lib, stvmod, q=None) == E.STV_EINVAL
    assert _verify(lib, stvmod, out=None) == E.STV_EINVAL
    assert _verify(lib, stvmod, scale=float("inf")) == E.STV_EINVAL
    assert _verify(lib, stvmod, scale=0.0) == E.STV_EINVAL
    assert _verify(lib, stvmod, scale=-0.5) == E.STV_EINVAL
    assert _verify(lib, stvmod, n_splits=-2) == E.STV_EINVAL
    layer = stvmod._KVLayer(FAKE, None, FAKE, FAKE, 4, 256, 1000)
    assert _verify(lib, stvmod, layer=layer) == E.STV_EINVAL


def test_format_errors(lib, stvmod):
    E = stvmod
    layer = stvmod._KVLayer(FAKE, FAKE, FAKE, FAKE, 4, 256, 1000, 7)
    assert _verify(lib, stvmod, layer=layer) == E.STV_EINVAL
    assert "kv_format" in _err(lib)
    unaligned = stvmod._KVLayer(FAKE + 4, FAKE, FAKE, FAKE, 4, 256, 1000, 1)
    assert _verify(lib, stvmod, layer=unaligned) == E.STV_EINVAL
    assert "aligned" in _err(lib)
    s, ws = ctypes.c_int32(), ctypes.c_size_t()
    assert lib.stv_attention_plan(8, 24, 4, 256, 100, 0, 2, 0, ctypes.byref(s),
                                  ctypes.byref(ws)) == E.STV_EINVAL
    f = lib.stv_kv_quant_pack
    assert f(FAKE, 10, 0, 4, FAKE, FAKE, 4, 256, 100, None) == E.STV_EINVAL
    assert f(FAKE + 4, 10, 0, 2, FAKE, FAKE, 4, 256, 100, None) == E.STV_EINVAL   # x alignment
    unknown = stvmod._KVLayer(FAKE, FAKE, FAKE, FAKE, 4, 256, 1000, 3)
    assert lib.stv_kv_commit(ctypes.byref(unknown), 0, 8, FAKE, FAKE, None) == E.STV_EINVAL
    assert "kv_format" in _err(lib)


def test_alignment_errors(lib, stvmod):
    """q, out, the workspace and the partials move in 16-byte vectors."""
    E = stvmod
    assert _verify(lib, stvmod, q=FAKE + 4) == E.STV_EINVAL
    assert "aligned" in _err(lib)
    assert _verify(lib, stvmod, out=FAKE + 8) == E.STV_EINVAL
    assert _verify(lib, stvmod, ws=FAKE + 12, ws_bytes=1 << 30) == E.STV_EINVAL
    m = np.ascontiguousarray(synth.ancestor_masks(synth.chain_parents(8)))
    layer = _layer(stvmod)
    assert lib.stv_attention_partials(FAKE, 8, 24, ctypes.byref(layer), 100, m.ctypes.data,
                                      0.0625, 2, FAKE + 4, FAKE, None) == E.STV_EINVAL
    f = lib.stv_split_merge
    assert f(FAKE + 4, FAKE, 2, 10, 64, FAKE, None, None) == E.STV_EINVAL
    assert f(FAKE, FAKE, 2, 10, 64, FAKE + 4, None, None) == E.STV_EINVAL
    assert "aligned" in _err(lib)


def test_context_errors(lib, stvmod):
    E = stvmod
    s, ws = ctypes.c_int32(), ctypes.c_size_t()
    assert lib.stv_context_plan(8, 24, 4, 256, 0, 0, 0, ctypes.byref(s), ctypes.byref(ws)) == E.STV_EINVAL
    assert lib.stv_context_plan(65, 24, 4, 256, 100, 0, 0, ctypes.byref(s), ctypes.byref(ws)) == E.STV_EINVAL
    assert lib.stv_context_plan(8, 24, 4, 256, 1000, 2, 0, ctypes.byref(s), ctypes.byref(ws)) == E.STV_EINVAL
    layer = _layer(stvmod)          # capacity 1000
    f = lib.stv_context_partials
    assert f(FAKE, 8, 24, ctypes.byref(layer), 1001, 0.0625, 0, FAKE, FAKE, None) == E.STV_ECAPACITY
    assert f(FAKE, 8, 24, ctypes.byref(layer), 0, 0.0625, 0, FAKE, FAKE, None) == E.STV_EINVAL
    assert f(FAKE, 8, 24, ctypes.byref(layer), 100, 0.0625, 0, None, FAKE, None) == E.STV_EINVAL
    assert f(FAKE, 8, 24, ctypes.byref(layer), 100, 0.0625, 0, FAKE, None, None) == E.STV_EINVAL
    assert f(FAKE, 65, 24, ctypes.byref(layer), 100, 0.0625, 0, FAKE, FAKE, None) == E.STV_EINVAL


def test_fp16acc_errors(lib, stvmod):
    """The fp16-accumulated variant checks what verify checks, and reads the
    3-bit format only."""
    E = stvmod
    m = np.ascontiguousarray(synth.ancestor_masks(synth.chain_parents(8)))
    f = lib.stv_verify_attention_fp16acc
    four = stvmod._KVLayer(FAKE, FAKE, FAKE, FAKE, 4, 256, 1000, 1)
    assert f(FAKE, 8, 24, ctypes.byref(four), 100, m.ctypes.data, 0.0625, FAKE, None, None, 0,
             0, None) == E.STV_EINVAL
    assert "3-bit" in _err(lib)
    three = _layer(stvmod)
    assert f(FAKE, 8, 24, ctypes.byref(three), 993, m.ctypes.data, 0.0625, FAKE, None, None, 0,
             0, None) == E.STV_ECAPACITY
    bad = m.copy()
    bad[3] &= ~np.uint64(1 << 3)
    assert f(FAKE, 8, 24, ctypes.byref(three), 100, bad.ctypes.data, 0.0625, FAKE, None, None,
             0, 0, None) == E.STV_EMASK


def test_verify_mask_errors(lib, stvmod):
    E = stvmod
    good = synth.ancestor_masks(np.array([-1, 0, 0, 1, 1, 2, 3, 6]))
    bad = good.copy()
    bad[3] &= ~np.uint64(1 << 3)                        # own bit missing
    assert _verify(lib, stvmod, mask=bad) == E.STV_EMASK
    bad = good.copy()
    bad[2] |= np.uint64(1 << 5)                         # bit above the row
    assert _verify(lib, stvmod, mask=bad) == E.STV_EMASK
    bad = good.copy()
    bad[6] = np.uint64((1 << 6) | (1 << 2))             # parent 2, but misses 2's ancestor 0
    assert _verify(lib, stvmod, mask=bad) == E.STV_EMASK
    bad = good.copy()
    bad[4] = np.uint64((1 << 4) | (1 << 3) | (1 << 2) | 1)   # two branches: not a path
    assert _verify(lib, stvmod, mask=bad) == E.STV_EMASK
    assert "anc_mask[4]" in _err(lib)


def _big_plan_args(stvmod, lib, T):
    # a context long enough that the automatic plan splits it (S > 1)
    L = 60000
    s = ctypes.c_int32()
    ws = ctypes.c_size_t()
    assert lib.stv_attention_plan(T, 24, 4, 256, L, 0, 0, 0, ctypes.byref(s), ctypes.byref(ws)) == 0
    assert s.value > 1 and ws.value > 0
    return L, ws.value


def test_valid_masks_pass_validation(lib, stvmod):
    """Every 8-row tree shape, a forest, and random 64-node trees pass the mask
    check: the call then stops at the (deliberately small) workspace."""
    layer = _layer(stvmod, cap=70000)
    L, need = _big_plan_args(stvmod, lib, 8)
    n = 0
    for parent in synth.all_tree_shapes(8):
        rc = _verify(lib, stvmod, T=8, layer=layer, L=L, mask=synth.ancestor_masks(parent),
                     ws=FAKE, ws_bytes=need - 1)
        assert rc == stvmod.STV_EWORKSPACE, _err(lib)
        n += 1
    assert n == 5040
    forest = synth.ancestor_masks(np.array([-1, -1, 0, 1, -1, 4]))
    rc = _verify(lib, stvmod, T=6, layer=layer, L=L, mask=forest, ws=FAKE, ws_bytes=0)
    assert rc == stvmod.STV_EWORKSPACE
    rng = np.random.default_rng(5)
    L64, need64 = _big_plan_args(stvmod, lib, 64)
    for _ in range(50):
        m = synth.ancestor_masks(synth.make_tree_parents(rng, 64, 8))
        rc = _verify(lib, stvmod, T=64, layer=layer, L=L64, mask=m, ws=FAKE, ws_bytes=need64 - 1)
        assert rc == stvmod.STV_EWORKSPACE, _err(lib)
        assert "workspace" in _err(lib)


def test_prefill_argument_errors(lib, stvmod):
    E = stvmod
    layer = _layer(stvmod, cap=5000)

    def call(T=100, L=100, ws=None, ws_bytes=0, n_splits=0):
        return lib.stv_prefill_attention(FAKE, T, 24, ctypes.byref(layer), L, 0.0625, FAKE, None,
                                         ws, ws_bytes, n_splits, None, None, None, None)
    assert call(T=0) == E.STV_EINVAL
    assert call(T=4901, L=100) == E.STV_ECAPACITY
    assert call(n_splits=4, ws=FAKE, ws_bytes=10) == E.STV_EWORKSPACE


def test_kv_pack_argument_errors(lib, stvmod):
    E = stvmod
    f = lib.stv_kv_quant_pack
    for which in (E.STV_K, E.STV_V):
        assert f(FAKE, -1, 0, which, FAKE, FAKE, 4, 256, 100, None) == E.STV_EINVAL
        assert f(FAKE, 10, 95, which, FAKE, FAKE, 4, 256, 100, None) == E.STV_ECAPACITY
        assert f(FAKE, 10, -1, which, FAKE, FAKE, 4, 256, 100, None) == E.STV_ECAPACITY
        assert f(FAKE, 10, 0, which, FAKE, FAKE, 4, 48, 100, None) == E.STV_EINVAL
        assert f(FAKE, 10, 0, which, FAKE, FAKE, 0, 256, 100, None) == E.STV_EINVAL
        assert f(None, 10, 0, which, FAKE, FAKE, 4, 256, 100, None) == E.STV_EINVAL
        assert f(FAKE, 0, 100, which, FAKE, FAKE, 4, 256, 100, None) == E.STV_OK   # nothing to do
        assert _err(lib) == ""
    assert f(FAKE, 10, 0, 4, FAKE, FAKE, 4, 256, 100, None) == E.STV_EINVAL
    assert "which" in _err(lib)


def test_merge_argument_errors(lib, stvmod):
    E = stvmod
    f = lib.stv_split_merge
    assert f(FAKE, FAKE, 0, 10, 256, FAKE, None, None) == E.STV_EINVAL
    assert f(FAKE, FAKE, 2, -1, 256, FAKE, None, None) == E.STV_EINVAL
    assert f(FAKE, FAKE, 2, 10, 0, FAKE, None, None) == E.STV_EINVAL
    assert f(FAKE, FAKE, 2, 10, 2000, FAKE, None, None) == E.STV_EINVAL
    assert f(None, FAKE, 2, 10, 256, FAKE, None, None) == E.STV_EINVAL
    assert f(FAKE, FAKE, 2, 0, 256, FAKE, None, None) == E.STV_OK          # no rows: no launch


def test_accept_and_commit_argument_errors(lib, stvmod):
    E = stvmod
    acc = lib.stv_tree_accept
    good = synth.ancestor_masks(np.array([-1, 0, 0, 1]))
    m = np.ascontiguousarray(good)
    assert acc(m.ctypes.data, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.STV_EINVAL
    assert acc(m.ctypes.data, 65, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.STV_EINVAL
    assert acc(None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.STV_EINVAL
    assert acc(m.ctypes.data, 4, FAKE, None, FAKE, FAKE, FAKE, None) == E.STV_EINVAL
    assert acc(m.ctypes.data, 4, FAKE, FAKE, FAKE, FAKE, None, None) == E.STV_EINVAL
    bad = good.copy()
    bad[3] = np.uint64(1 << 3)
    bad[2] |= np.uint64(1 << 3)
    mb = np.ascontiguousarray(bad)
    assert acc(mb.ctypes.data, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.STV_EMASK
    com = lib.stv_kv_commit
    layer = _layer(stvmod, cap=100)
    assert com(ctypes.byref(layer), 90, 11, FAKE, FAKE, None) == E.STV_ECAPACITY
    assert com(ctypes.byref(layer), -1, 8, FAKE, FAKE, None) == E.STV_EINVAL
    assert com(ctypes.byref(layer), 0, 0, FAKE, FAKE, None) == E.STV_EINVAL
    assert com(ctypes.byref(layer), 0, 65, FAKE, FAKE, None) == E.STV_EINVAL
    assert com(ctypes.byref(layer), 0, 8, None, FAKE, None) == E.STV_EINVAL
    assert com(ctypes.byref(_layer(stvmod, d=96, cap=100)), 0, 8, FAKE, FAKE, None) == E.STV_EINVAL
    assert com(None, 0, 8, FAKE, FAKE, None) == E.STV_EINVAL


def test_lookup_argument_errors(lib, stvmod):
    E = stvmod
    ws = ctypes.c_size_t()
    assert lib.stv_lookup_plan(3, 9000, ctypes.byref(ws)) == E.STV_OK
    assert ws.value == 3 * 3 * 8                     # ceil(8999 / 4096) = 3 chunks
    assert lib.stv_lookup_plan(-1, 10, ctypes.byref(ws)) == E.STV_EINVAL
    assert lib.stv_lookup_plan(1, 0, ctypes.byref(ws)) == E.STV_EINVAL
    f = lib.stv_lookup_draft

    def call(B=2, stride=100, n_min=6, n_max=12, k=8, ws_bytes=64, hist=FAKE, tokens=FAKE):
        return f(hist, FAKE, B, stride, n_min, n_max, k, tokens, FAKE, FAKE, FAKE, FAKE,
                 ws_bytes, None)
    assert call(n_min=0) == E.STV_EINVAL
    assert call(n_min=7, n_max=6) == E.STV_EINVAL
    assert call(n_max=65) == E.STV_EINVAL
    assert call(k=-1) == E.STV_EINVAL
    assert call(hist=None) == E.STV_EINVAL
    assert call(tokens=None) == E.STV_EINVAL
    assert call(ws_bytes=15) == E.STV_EWORKSPACE
    assert call(B=0) == E.STV_OK


@pytest.mark.parametrize("T,hq,hkv,d,L,causal", [
    (1, 24, 4, 256, 8192, 0), (64, 24, 4, 256, 32768, 0), (64, 24, 4, 256, 262144, 0),
    (8, 24, 4, 256, 262144, 0), (4096, 24, 4, 256, 32768, 1), (8, 4, 1, 64, 512, 0),
])
@pytest.mark.parametrize("fmt", ["b3", "i4"])
def test_plan_is_consistent(stvmod, T, hq, hkv, d, L, causal, fmt):
    for req in (0, 1, 3, 17, 100000):
        S, ws = stvmod.attention_plan(T, hq, hkv, d, L, bool(causal), req, fmt)
        n_tiles = -(-(L + T) // 32)
        assert 1 <= S <= n_tiles
        if req:
            assert S <= req
        part = S * T * hq * (d + 1) * 4 if S > 1 else 0
        assert part == stvmod.workspace_bytes(T, hq, d, S)
        if causal and fmt == "b3" and -(-T * (hq // hkv) // 32) > 28:
            # eight or more groups of 128 rows per KV head: the workspace also
            # holds one unpacked image per tile and KV head, after the partials
            img = ws - -(-part // 256) * 256
            assert img > 0 and img % (hkv * n_tiles) == 0
            assert (img // (hkv * n_tiles)) % 1024 == 0
        else:
            assert ws == part
        # the documented split layout covers every key, each split non-empty
        P = 32 * -(-n_tiles // S)
        assert (S - 1) * P < L + T <= S * P
    S0, _ = stvmod.attention_plan(T, hq, hkv, d, L, bool(causal), 0)
    S1, _ = stvmod.attention_plan(T, hq, hkv, d, L, bool(causal), 0)
    assert S0 == S1


def test_plan_wave_specialized_rounds(stvmod):
    """The wave-specialized kernel's split plan with the fixed MI355X figure
    used when no device answers (256 CUs, one work-group each, eight XCDs):
    work items run ceil(items / 8) to an XCD, a round costs its tiles plus 12
    tile steps, and the plan takes the cheapest split count.  The 64-node tree
    (three row groups per KV head) gets 21 splits at 262K and at 32K: 252
    items, 32 per XCD, one round."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("with a device the plan follows its occupancy")
    for L in (262144, 32768):
        S, _ = stvmod.attention_plan(64, 24, 4, 256, L, False, 0, "b3")
        n_tiles = -(-(L + 64) // 32)

        def cost(s):
            per_xcd = -(-(4 * 3 * s) // 8)
            return -(-per_xcd // 32) * (-(-n_tiles // s) + 12)

        assert S == 21
        assert cost(S) == min(cost(s) for s in range(1, 89))


def test_workspace_bytes(stvmod):
    lib = stvmod.load_library()
    assert stvmod.workspace_bytes(64, 24, 256, 42) == 42 * 64 * 24 * 257 * 4
    assert stvmod.workspace_bytes(1, 24, 256, 1) == 0
    assert lib.stv_last_error() == b""
    for args in ((0, 24, 256, 2), (8, 0, 256, 2), (8, 24, 96, 2), (8, 24, 256, 0),
                 (8, 24, 256, -3), (1 << 30, 4, 256, 2)):
        assert lib.stv_workspace_bytes(*args) == 0
        assert lib.stv_last_error() != b""
        with pytest.raises(stvmod.StvError):
            stvmod.workspace_bytes(*args)


def test_product_path_refuses_to_run_without_the_library(stvmod, monkeypatch, tmp_path):
    monkeypatch.setattr(stvmod, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(stvmod, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        stvmod.load_library()


def test_noalloc_rejects_split_counts_beyond_its_scratch(lib, stvmod):
    """The no-alloc entry point: an explicit split count whose partials do not
    fit the library's scratch array fails with STV_EWORKSPACE on the host."""
    assert lib.stv_noalloc_scratch_bytes() == 64 << 20
    T, hq, d, L = 64, 24, 256, 262144
    layer = _layer(stvmod, hkv=4, d=d, cap=L + T)
    m = np.ascontiguousarray(synth.ancestor_masks(synth.chain_parents(T)))
    per_split = T * hq * (d + 1) * 4
    fit = (64 << 20) // per_split
    rc = lib.stv_verify_attention_noalloc(FAKE, T, hq, ctypes.byref(layer), L, m.ctypes.data,
                                          0.0625, FAKE, None, fit + 1, None)
    assert rc == stvmod.STV_EWORKSPACE
    assert b"no-alloc scratch" in lib.stv_last_error()
    # the usual argument checks come first
    rc = lib.stv_verify_attention_noalloc(FAKE, 65, hq, ctypes.byref(layer), L, None, 0.0625,
                                          FAKE, None, 0, None)
    assert rc == stvmod.STV_EINVAL
