"""CPU oracle for verify-round attention over a 3-bit KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may use it; the product path never does.  The arithmetic lives
in ``stv_oracle.c`` (plain C, int64 integer logits, fp64 softmax and P.V);
this module builds it with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "stv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.orc_code_get.argtypes = [P, i32]
        lib.orc_code_get.restype = i32
        lib.orc_code_set.argtypes = [P, i32, i32]
        lib.orc_code_set.restype = None
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_f64.restype = ctypes.c_double
        lib.orc_quantize_q_row.argtypes = [P, i32, P, P]
        lib.orc_quantize_q_row.restype = None
        lib.orc_quantize_kv_block.argtypes = [P, P]
        lib.orc_quantize_kv_block.restype = ctypes.c_uint16
        for fn in (lib.orc_k_quant_pack, lib.orc_v_quant_pack):
            fn.argtypes = [P, i32, i32, P, P, i32, i32, i32]
            fn.restype = None
        lib.orc_attention.argtypes = [P, i32, i32, P, P, P, P, i32, i32, i32, i32, P,
                                      ctypes.c_double, i32, i32, P, i32, P, P, P, P, P]
        lib.orc_attention.restype = i32
        lib.orc_set_threads.argtypes = [i32]
        lib.orc_set_threads.restype = i32
        lib.orc_merge.argtypes = [P, P, i32, i32, i32, P, P]
        lib.orc_merge.restype = None
        lib.orc_tree_accept.argtypes = [P, i32, P, P, P, P]
        lib.orc_tree_accept.restype = i32
        lib.orc_kv_commit.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, i32]
        lib.orc_kv_commit.restype = i32
        lib.orc_lookup_draft.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P]
        lib.orc_lookup_draft.restype = None
        lib.orc_quantize_kv4_row.argtypes = [P, i32, P]
        lib.orc_quantize_kv4_row.restype = ctypes.c_uint16
        for fn in (lib.orc_k4_quant_pack, lib.orc_v4_quant_pack):
            fn.argtypes = [P, i32, i32, P, P, i32, i32, i32]
            fn.restype = None
        lib.orc_attention_i4.argtypes = lib.orc_attention.argtypes
        lib.orc_attention_i4.restype = i32
        lib.orc_kv4_commit.argtypes = lib.orc_kv_commit.argtypes
        lib.orc_kv4_commit.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int = 0) -> int:
    """Set (n > 0) and return the number of threads the row loop uses."""
    return int(_load().orc_set_threads(int(n)))


# ------------------------------------------------------------------ format

def code_get(words, e: int) -> int:
    w = _c(words, np.uint32)
    assert w.shape == (3,)
    return _load().orc_code_get(_ptr(w), e)


def pack_block(codes) -> np.ndarray:
    """32 integer codes in [0, 7] -> 3 words (oracle's own packer)."""
    codes = list(codes)
    assert len(codes) == 32
    w = np.zeros(3, dtype=np.uint32)
    lib = _load()
    for e, c in enumerate(codes):
        lib.orc_code_set(_ptr(w), e, int(c))
    return w


def unpack_block(words) -> np.ndarray:
    w = _c(words, np.uint32)
    lib = _load()
    return np.array([lib.orc_code_get(_ptr(w), e) for e in range(32)], dtype=np.int64)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., NB, 3] words -> [..., NB*32] codes (slow; small inputs only)."""
    c = _c(codes, np.uint32)
    lead = c.shape[:-2]
    nb = c.shape[-2]
    flat = c.reshape(-1, nb, 3)
    out = np.empty((flat.shape[0], nb * 32), dtype=np.int64)
    for i in range(flat.shape[0]):
        for b in range(nb):
            out[i, 32 * b:32 * b + 32] = unpack_block(flat[i, b])
    return out.reshape(*lead, nb * 32)


def f32_to_f16_bits(x: float) -> int:
    return int(_load().orc_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f64(h: int) -> float:
    return float(_load().orc_f16_to_f64(int(h)))


# -------------------------------------------------------------- quantizers

def quantize_q_row(q) -> tuple[np.ndarray, np.float32]:
    q = _c(q, np.float32)
    qi = np.empty(q.shape[0], dtype=np.int8)
    sq = np.empty(1, dtype=np.float32)
    _load().orc_quantize_q_row(_ptr(q), q.shape[0], _ptr(qi), _ptr(sq))
    return qi, sq[0]


def quantize_kv_block(x) -> tuple[np.ndarray, int]:
    x = _c(x, np.float32)
    assert x.shape == (32,)
    w = np.zeros(3, dtype=np.uint32)
    s = _load().orc_quantize_kv_block(_ptr(x), _ptr(w))
    return w, int(s)


def kv_quant_pack(x, pos0: int, codes: np.ndarray, scales: np.ndarray, which: str) -> None:
    """x: [n_tok][Hkv][D] fp32, written in place into codes/scales of the K
    (token-major) or V (key-transposed) layout; which is "k" or "v"."""
    x = _c(x, np.float32)
    n_tok, hkv, d = x.shape
    nb = d // 32
    assert codes.dtype == np.uint32 and codes.flags.c_contiguous
    assert scales.dtype == np.uint16 and scales.flags.c_contiguous
    if which == "k":
        cap = codes.shape[1]
        assert codes.shape == (hkv, cap, nb, 3) and scales.shape == (hkv, cap, nb)
        fn = _load().orc_k_quant_pack
    elif which == "v":
        ng = codes.shape[1]
        cap = 32 * ng
        assert codes.shape == (hkv, ng, d, 3) and scales.shape == (hkv, ng, nb, 32)
        fn = _load().orc_v_quant_pack
    else:
        raise ValueError(which)
    assert 0 <= pos0 and pos0 + n_tok <= cap
    fn(_ptr(x), n_tok, pos0, _ptr(codes), _ptr(scales), hkv, d, cap)


def v_values(kv, head: int, key: int) -> np.ndarray:
    """Dequantized V row (fp64) of one key, read through the V layout."""
    d = kv.head_dim
    ng = kv.v_codes.shape[1]
    lib = _load()
    out = np.empty(d)
    grp, e = divmod(key, 32)
    for b in range(d // 32):
        s = f16_bits_to_f64(int(kv.v_scales[head, grp, b, e]))
        for i in range(32):
            w = _c(kv.v_codes[head, grp, 32 * b + i], np.uint32)
            out[32 * b + i] = s * (lib.orc_code_get(_ptr(w), e) - 4)
    return out


# --------------------------------------------------------------- attention

def attention(q, kv, ctx_len: int, mask=None, scale: float | None = None,
              k_begin: int = 0, k_end: int | None = None, rows=None,
              want_logits: bool = False):
    """See attention_fmt; kv is the 3-bit cache, or the 4-bit per-token-head
    cache when it has `fmt == "i4"`."""
    return attention_fmt(q, kv, ctx_len, mask, scale, k_begin, k_end, rows, want_logits,
                         getattr(kv, "fmt", "b3"))


def attention_fmt(q, kv, ctx_len: int, mask=None, scale: float | None = None,
                  k_begin: int = 0, k_end: int | None = None, rows=None,
                  want_logits: bool = False, fmt: str = "b3"):
    """The oracle's attention for the rows listed (flattened t*Hq + h).

    kv: an object with k_codes, k_scales, v_codes, v_scales, n_kv_heads,
    head_dim, capacity (K token-major, V key-transposed; see stv_oracle.c).  mask: uint64 [T] ancestor masks, or None for the
    causal chunk rule.  Returns dict(out fp64 [n][D], lse fp64 [n],
    qi8 int8 [n][D], sq fp32 [n], logits int64 [n][L+T][NB] (3-bit) or
    [n][L+T] (4-bit), or None).  fmt: "b3" (3-bit, per-block scales) or "i4"
    (4-bit, per token-head scales).
    """
    q = _c(q, np.float32)
    T, hq, d = q.shape
    assert d == kv.head_dim
    n_keys = ctx_len + T
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if k_end is None:
        k_end = n_keys
    rows_arr = None
    n = T * hq
    if rows is not None:
        rows_arr = _c(rows, np.int32)
        n = rows_arr.shape[0]
    m = None if mask is None else _c(mask, np.uint64)
    out = np.empty((n, d), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    qi8 = np.empty((n, d), dtype=np.int8)
    sq = np.empty(n, dtype=np.float32)
    lshape = (n, n_keys, d // 32) if fmt == "b3" else (n, n_keys)
    logits = np.empty(lshape, dtype=np.int64) if want_logits else None
    kc = _c(kv.k_codes, np.uint32)
    ks = _c(kv.k_scales, np.uint16)
    vc = _c(kv.v_codes, np.uint32)
    vs = _c(kv.v_scales, np.uint16)
    fn = _load().orc_attention if fmt == "b3" else _load().orc_attention_i4
    rc = fn(_ptr(q), T, hq, _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                               kv.n_kv_heads, d, kv.capacity, ctx_len, _ptr(m),
                               float(scale), k_begin, k_end, _ptr(rows_arr),
                               n if rows is not None else 0, _ptr(out), _ptr(lse),
                               _ptr(logits), _ptr(qi8), _ptr(sq))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"out": out, "lse": lse, "qi8": qi8, "sq": sq, "logits": logits}


def merge(part_o, part_lse):
    """part_o [S][rows][D], part_lse [S][rows] -> (out fp64, lse fp64)."""
    po = _c(part_o, np.float64)
    pl = _c(part_lse, np.float64)
    S, rows, d = po.shape
    assert pl.shape == (S, rows)
    out = np.empty((rows, d), dtype=np.float64)
    lse = np.empty(rows, dtype=np.float64)
    _load().orc_merge(_ptr(po), _ptr(pl), S, rows, d, _ptr(out), _ptr(lse))
    return out, lse


# ------------------------------------------------------ tree acceptance

def tree_accept(mask, draft, target):
    """Greedy tree acceptance (see orc_tree_accept).  mask: uint64 [T]
    ancestor masks; draft, target: int32 [T] token ids.  Returns
    (n, path int32 [T] with -1 past n, bonus)."""
    m = _c(np.asarray(mask, dtype=np.uint64), np.uint64)
    T = m.size
    dr = _c(np.asarray(draft, dtype=np.int32), np.int32)
    tg = _c(np.asarray(target, dtype=np.int32), np.int32)
    assert dr.size == T and tg.size == T
    path = np.empty(T, dtype=np.int32)
    bonus = np.zeros(1, dtype=np.int32)
    n = _load().orc_tree_accept(_ptr(m), T, _ptr(dr), _ptr(tg), _ptr(path), _ptr(bonus))
    if n < 1:
        raise ValueError("bad tree_accept arguments")
    return int(n), path, int(bonus[0])


def kv_commit(kv, ctx_len: int, T: int, path, n: int) -> None:
    """In-place accepted-path commit on a host cache (see orc_kv_commit)."""
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        a = getattr(kv, name)
        assert a.flags["C_CONTIGUOUS"], name
    p = _c(np.asarray(path, dtype=np.int32), np.int32)
    fn = _load().orc_kv_commit if getattr(kv, "fmt", "b3") == "b3" else _load().orc_kv4_commit
    rc = fn(_ptr(kv.k_codes), _ptr(kv.k_scales), _ptr(kv.v_codes),
                               _ptr(kv.v_scales), kv.n_kv_heads, kv.head_dim, kv.capacity,
                               ctx_len, T, _ptr(p), n)
    if rc != 0:
        raise ValueError("bad kv_commit arguments")


# ------------------------------------------------------- lookup drafting

def lookup_draft(history, lengths, n_min: int = 6, n_max: int = 12, k: int = 8):
    """Lookup drafting (see orc_lookup_draft).  history: int32 [B][stride];
    lengths: int32 [B].  Returns dict(tokens [B][k], count, match, pos)."""
    h = _c(np.atleast_2d(np.asarray(history, dtype=np.int32)), np.int32)
    B, stride = h.shape
    ln = _c(np.asarray(lengths, dtype=np.int32).reshape(B), np.int32)
    tokens = np.empty((B, k), dtype=np.int32)
    count = np.empty(B, dtype=np.int32)
    match = np.empty(B, dtype=np.int32)
    pos = np.empty(B, dtype=np.int32)
    _load().orc_lookup_draft(_ptr(h), _ptr(ln), B, stride, n_min, n_max, k, _ptr(tokens),
                             _ptr(count), _ptr(match), _ptr(pos))
    return {"tokens": tokens, "count": count, "match": match, "pos": pos}


# ------------------------------------------- 4-bit per-token-head format

def quantize_kv4_row(x) -> tuple[np.ndarray, int]:
    """(D/8 code words, fp16 scale bits) of one row (see orc_quantize_kv4_row)."""
    x = _c(x, np.float32)
    w = np.empty(x.size // 8, dtype=np.uint32)
    s = _load().orc_quantize_kv4_row(_ptr(x), x.size, _ptr(w))
    return w, int(s)


def kv4_quant_pack(x, pos0: int, codes: np.ndarray, scales: np.ndarray, which: str) -> None:
    """In-place 4-bit pack of x [n_tok][Hkv][D] at positions pos0.. into the
    K (which="k") or V (which="v") arrays of the 4-bit cache."""
    x = _c(x, np.float32)
    n_tok, hkv, d = x.shape
    assert codes.dtype == np.uint32 and scales.dtype == np.uint16
    assert codes.flags["C_CONTIGUOUS"] and scales.flags["C_CONTIGUOUS"]
    cap = scales.shape[1]
    fn = _load().orc_k4_quant_pack if which == "k" else _load().orc_v4_quant_pack
    fn(_ptr(x), n_tok, pos0, _ptr(codes), _ptr(scales), hkv, d, cap)
