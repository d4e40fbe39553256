"""Speculative tree-verify attention over a quantized KV cache (3-bit blocks
or 4-bit per token-head), for MI355X.

Thin ctypes binding of ``libstv.so`` (hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/stv.h``).  This module only checks and
marshals arguments; PyTorch supplies device memory and the current stream.
Every step of the computation runs in the library's kernels, and nothing
here falls back to another implementation: if the library is missing, the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstv.so")

STV_OK = 0
STV_EINVAL = -1
STV_EMASK = -2
STV_ECAPACITY = -3
STV_EWORKSPACE = -4
STV_EHIP = -5

__all__ = [
    "StvError", "KVCache", "load_library", "kv_quant_pack", "attention_plan", "workspace_bytes",
    "verify_attention", "verify_attention_fp16acc", "verify_attention_noalloc",
    "noalloc_scratch_bytes", "prefill_attention",
    "attention_partials", "context_plan", "context_partials", "split_merge", "tree_accept", "kv_commit", "lookup_plan",
    "lookup_draft", "STV_OK", "STV_EINVAL", "STV_EMASK", "STV_ECAPACITY", "STV_EWORKSPACE",
    "STV_EHIP", "STV_KV_3BIT", "STV_KV_4BIT_TOKEN",
]


class StvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"stv error {code}: {msg}")
        self.code = code


class _KVLayer(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("kv_format", ctypes.c_int32)]


STV_KV_3BIT = 0
STV_KV_4BIT_TOKEN = 1
_FORMATS = {"b3": STV_KV_3BIT, "i4": STV_KV_4BIT_TOKEN}


_lib = None
ABI_VERSION = 5      # the argument lists below follow this version of include/stv.h


def load_library():
    """Load libstv.so; raises if it has not been built or was built from
    another version of the ABI than this binding's."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m "
                               "speculative_tree_verify_amd.build_lib` first")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.stv_last_error.restype = ctypes.c_char_p
        lib.stv_last_error.argtypes = []
        lib.stv_abi_version.restype = i32
        lib.stv_abi_version.argtypes = []
        if lib.stv_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} implements ABI version {lib.stv_abi_version()}, "
                               f"this binding expects {ABI_VERSION}: rebuild the library")
        lib.stv_kv_quant_pack.restype = ctypes.c_int
        lib.stv_kv_quant_pack.argtypes = [P, i32, i32, i32, P, P, i32, i32, i32, P]
        lib.stv_workspace_bytes.restype = ctypes.c_size_t
        lib.stv_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.stv_attention_plan.restype = ctypes.c_int
        lib.stv_attention_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                           ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_size_t)]
        lib.stv_verify_attention.restype = ctypes.c_int
        lib.stv_verify_attention.argtypes = [P, i32, i32, ctypes.POINTER(_KVLayer), i32, P,
                                             ctypes.c_float, P, P, P, ctypes.c_size_t, i32,
                                             P, P, P, P]
        lib.stv_verify_attention_fp16acc.restype = ctypes.c_int
        lib.stv_verify_attention_fp16acc.argtypes = [P, i32, i32, ctypes.POINTER(_KVLayer), i32,
                                                     P, ctypes.c_float, P, P, P, ctypes.c_size_t,
                                                     i32, P]
        lib.stv_verify_attention_noalloc.restype = ctypes.c_int
        lib.stv_verify_attention_noalloc.argtypes = [P, i32, i32, ctypes.POINTER(_KVLayer), i32,
                                                     P, ctypes.c_float, P, P, i32, P]
        lib.stv_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.stv_noalloc_scratch_bytes.argtypes = []
        lib.stv_context_plan.restype = ctypes.c_int
        lib.stv_context_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                         ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_size_t)]
        lib.stv_context_partials.restype = ctypes.c_int
        lib.stv_context_partials.argtypes = [P, i32, i32, ctypes.POINTER(_KVLayer), i32,
                                             ctypes.c_float, i32, P, P, P]
        lib.stv_prefill_attention.restype = ctypes.c_int
        lib.stv_prefill_attention.argtypes = [P, i32, i32, ctypes.POINTER(_KVLayer), i32,
                                              ctypes.c_float, P, P, P, ctypes.c_size_t, i32,
                                              P, P, P, P]
        lib.stv_attention_partials.restype = ctypes.c_int
        lib.stv_attention_partials.argtypes = [P, i32, i32, ctypes.POINTER(_KVLayer), i32, P,
                                               ctypes.c_float, i32, P, P, P]
        lib.stv_split_merge.restype = ctypes.c_int
        lib.stv_split_merge.argtypes = [P, P, i32, i32, i32, P, P, P]
        lib.stv_tree_accept.restype = ctypes.c_int
        lib.stv_tree_accept.argtypes = [P, i32, P, P, P, P, P, P]
        lib.stv_kv_commit.restype = ctypes.c_int
        lib.stv_kv_commit.argtypes = [ctypes.POINTER(_KVLayer), i32, i32, P, P, P]
        lib.stv_lookup_plan.restype = ctypes.c_int
        lib.stv_lookup_plan.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_size_t)]
        lib.stv_lookup_draft.restype = ctypes.c_int
        lib.stv_lookup_draft.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P,
                                         ctypes.c_size_t, P]
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != STV_OK:
        raise StvError(rc, load_library().stv_last_error().decode())


def _torch():
    import torch
    return torch


def _dev_ptr(t, dtype, name, shape=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


STV_K = 0
STV_V = 1
STV_K4 = 2
STV_V4 = 3


@dataclass
class KVCache:
    """One layer's quantized cache on the GPU (layouts as in include/stv.h).

    fmt "b3" (3-bit, per-32-element scales): k_codes int32 [Hkv][cap][D/32][3],
    k_scales float16 [Hkv][cap][D/32], v_codes int32 [Hkv][ng][D][3],
    v_scales float16 [Hkv][ng][D/32][32].  fmt "i4" (4-bit, per-token-head
    scales): k_codes int32 [Hkv][cap][D/8], k_scales float16 [Hkv][cap],
    v_codes int32 [Hkv][ng][D][4], v_scales float16 [Hkv][cap].
    ng = ceil(cap / 32); the capacity is that of the K arrays.
    """
    k_codes: "object"
    k_scales: "object"
    v_codes: "object"
    v_scales: "object"
    fmt: str = "b3"

    @property
    def n_kv_heads(self) -> int:
        return int(self.k_codes.shape[0])

    @property
    def capacity(self) -> int:
        return int(self.k_codes.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k_codes.shape[2]) * (32 if self.fmt == "b3" else 8)

    @classmethod
    def empty(cls, n_kv_heads: int, head_dim: int, capacity: int, device="cuda", fmt="b3"):
        torch = _torch()
        nb = head_dim // 32
        ng = (capacity + 31) // 32
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
        if fmt == "i4":
            return cls(z((n_kv_heads, capacity, head_dim // 8), torch.int32),
                       z((n_kv_heads, capacity), torch.float16),
                       z((n_kv_heads, ng, head_dim, 4), torch.int32),
                       z((n_kv_heads, capacity), torch.float16), "i4")
        return cls(z((n_kv_heads, capacity, nb, 3), torch.int32),
                   z((n_kv_heads, capacity, nb), torch.float16),
                   z((n_kv_heads, ng, head_dim, 3), torch.int32),
                   z((n_kv_heads, ng, nb, 32), torch.float16))

    @classmethod
    def from_host(cls, host, device="cuda"):
        """Copy host arrays (uint32 codes, uint16 fp16-bit scales) to the GPU;
        the format is host.fmt when present, else "b3"."""
        torch = _torch()

        def up(a, view):
            return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(device)
        return cls(up(host.k_codes, np.int32), up(host.k_scales, np.float16),
                   up(host.v_codes, np.int32), up(host.v_scales, np.float16),
                   getattr(host, "fmt", "b3"))

    def _layer(self) -> _KVLayer:
        torch = _torch()
        hkv, cap, d = self.n_kv_heads, self.capacity, self.head_dim
        nb, ng = d // 32, (cap + 31) // 32
        if self.fmt == "i4":
            shapes = ((hkv, cap, d // 8), (hkv, cap), (hkv, ng, d, 4), (hkv, cap))
        else:
            shapes = ((hkv, cap, nb, 3), (hkv, cap, nb), (hkv, ng, d, 3), (hkv, ng, nb, 32))
        return _KVLayer(_dev_ptr(self.k_codes, torch.int32, "k_codes", shapes[0]),
                        _dev_ptr(self.k_scales, torch.float16, "k_scales", shapes[1]),
                        _dev_ptr(self.v_codes, torch.int32, "v_codes", shapes[2]),
                        _dev_ptr(self.v_scales, torch.float16, "v_scales", shapes[3]),
                        hkv, d, cap, _FORMATS[self.fmt])


def kv_quant_pack(x, pos0: int, cache: KVCache, which: str):
    """Quantize x [n_tok][Hkv][D] fp32 into positions pos0.. of the cache's K
    (which="k") or V (which="v") arrays."""
    torch = _torch()
    n_tok, hkv, d = x.shape
    if which not in ("k", "v"):
        raise ValueError("which must be 'k' or 'v'")
    layer = cache._layer()
    if hkv != cache.n_kv_heads or d != cache.head_dim:
        raise ValueError("x does not match the cache's heads or head_dim")
    codes, scales = (cache.k_codes, cache.k_scales) if which == "k" else (cache.v_codes, cache.v_scales)
    code = {("k", "b3"): STV_K, ("v", "b3"): STV_V, ("k", "i4"): STV_K4,
            ("v", "i4"): STV_V4}[(which, cache.fmt)]
    rc = load_library().stv_kv_quant_pack(
        _dev_ptr(x, torch.float32, "x"), n_tok, pos0, code,
        codes.data_ptr(), scales.data_ptr(), hkv, d, cache.capacity, _stream(x.device))
    _check(rc)
    del layer


def attention_plan(T: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ctx_len: int,
                   causal: bool, n_splits: int = 0, fmt: str = "b3") -> tuple[int, int]:
    """(effective split count, workspace bytes) of a call with these sizes."""
    s = ctypes.c_int32()
    ws = ctypes.c_size_t()
    _check(load_library().stv_attention_plan(T, n_q_heads, n_kv_heads, head_dim, ctx_len,
                                             int(bool(causal)), _FORMATS[fmt], n_splits,
                                             ctypes.byref(s), ctypes.byref(ws)))
    return int(s.value), int(ws.value)


def workspace_bytes(T: int, n_q_heads: int, head_dim: int, n_splits: int) -> int:
    """Workspace bytes of a call with split count n_splits (0 when it is 1)."""
    lib = load_library()
    n = int(lib.stv_workspace_bytes(T, n_q_heads, head_dim, n_splits))
    if n == 0 and lib.stv_last_error():
        raise StvError(STV_EINVAL, lib.stv_last_error().decode())
    return n


def _attention(q, kv: KVCache, ctx_len: int, mask, softmax_scale, out, out_lse, workspace,
               n_splits, debug, causal, fp16acc=False):
    torch = _torch()
    T, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
    S, ws_bytes = attention_plan(T, hq, kv.n_kv_heads, d, ctx_len, causal, n_splits, kv.fmt)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = None
    ws_len = 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, torch.uint8, "workspace")
        ws_len = workspace.numel()
    dbg = None
    dbg_ptrs = (None, None, None)
    if debug:
        names = ("logits", "q8", "qscale") if debug is True else tuple(debug)
        lshape = (T, hq, ctx_len + T, d // 32) if kv.fmt == "b3" else (T, hq, ctx_len + T)
        shapes = {"logits": (lshape, torch.int32),
                  "q8": ((T, hq, d), torch.int8), "qscale": ((T, hq), torch.float32)}
        dbg = {k: torch.zeros(shapes[k][0], dtype=shapes[k][1], device=q.device) for k in names}
        dbg_ptrs = tuple(dbg[k].data_ptr() if k in dbg else None
                         for k in ("logits", "q8", "qscale"))
    layer = kv._layer()
    lib = load_library()
    common = (_dev_ptr(out, torch.float32, "out", (T, hq, d)),
              _dev_ptr(out_lse, torch.float32, "out_lse", (T, hq)))
    if causal:
        rc = lib.stv_prefill_attention(
            _dev_ptr(q, torch.float32, "q"), T, hq, ctypes.byref(layer), ctx_len,
            float(softmax_scale), *common, ws_ptr, ws_len, n_splits, *dbg_ptrs,
            _stream(q.device))
    else:
        m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint64))
        if m.shape != (T,):
            raise ValueError(f"anc_mask must have shape ({T},)")
        if fp16acc:
            rc = lib.stv_verify_attention_fp16acc(
                _dev_ptr(q, torch.float32, "q"), T, hq, ctypes.byref(layer), ctx_len,
                m.ctypes.data, float(softmax_scale), *common, ws_ptr, ws_len, n_splits,
                _stream(q.device))
        else:
            rc = lib.stv_verify_attention(
                _dev_ptr(q, torch.float32, "q"), T, hq, ctypes.byref(layer), ctx_len,
                m.ctypes.data, float(softmax_scale), *common, ws_ptr, ws_len, n_splits,
                *dbg_ptrs, _stream(q.device))
    _check(rc)
    # keep host/device buffers alive until the enqueued work has consumed them
    # (the mask is copied into kernel arguments at launch; the workspace is
    # owned by the caller's allocator and stream-ordered)
    return (out, dbg) if debug else out


def verify_attention(q, kv: KVCache, ctx_len: int, anc_mask, softmax_scale=None, out=None,
                     out_lse=None, workspace=None, n_splits: int = 0, debug: bool = False):
    """Tree-verify attention: q [T][Hq][D] fp32 over kv, rows masked by anc_mask [T] uint64.

    Returns out [T][Hq][D], and with debug a dict of debug tensors: debug=True
    asks for all of "logits" (int32 per-block Q.K^T sums), "q8" and "qscale";
    a tuple of those names asks for a subset."""
    return _attention(q, kv, ctx_len, anc_mask, softmax_scale, out, out_lse, workspace,
                      n_splits, debug, causal=False)


def verify_attention_fp16acc(q, kv: KVCache, ctx_len: int, anc_mask, softmax_scale=None,
                             out=None, out_lse=None, workspace=None, n_splits: int = 0):
    """verify_attention with P.V accumulated in fp16 (3-bit caches only)."""
    return _attention(q, kv, ctx_len, anc_mask, softmax_scale, out, out_lse, workspace,
                      n_splits, False, causal=False, fp16acc=True)


def verify_attention_noalloc(q, kv: KVCache, ctx_len: int, anc_mask, softmax_scale=None,
                             out=None, out_lse=None, n_splits: int = 0):
    """verify_attention whose split partials go to the library's fixed
    per-GPU scratch array (the call allocates nothing on the device; `out`
    is allocated here only when the caller passes none).  Calls that overlap
    on one GPU race on that array."""
    torch = _torch()
    T, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
    m = np.ascontiguousarray(np.asarray(anc_mask, dtype=np.uint64))
    if m.shape != (T,):
        raise ValueError(f"anc_mask must have shape ({T},)")
    layer = kv._layer()
    _check(load_library().stv_verify_attention_noalloc(
        _dev_ptr(q, torch.float32, "q"), T, hq, ctypes.byref(layer), ctx_len, m.ctypes.data,
        float(softmax_scale), _dev_ptr(out, torch.float32, "out", (T, hq, d)),
        _dev_ptr(out_lse, torch.float32, "out_lse", (T, hq)), n_splits, _stream(q.device)))
    return out


def noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU array verify_attention_noalloc uses."""
    return int(load_library().stv_noalloc_scratch_bytes())


def prefill_attention(q, kv: KVCache, ctx_len: int, softmax_scale=None, out=None,
                      out_lse=None, workspace=None, n_splits: int = 0, debug: bool = False):
    """Chunked-prefill attention: row t sees keys 0 .. ctx_len + t."""
    return _attention(q, kv, ctx_len, None, softmax_scale, out, out_lse, workspace,
                      n_splits, debug, causal=True)


def attention_partials(q, kv: KVCache, ctx_len: int, anc_mask=None, softmax_scale=None,
                       n_splits: int = 0, part_o=None, part_lse=None):
    """Split phase only: returns (part_o [S][T][Hq][D], part_lse [S][T][Hq]).

    anc_mask None selects the causal chunk rule (prefill)."""
    torch = _torch()
    T, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    S, _ = attention_plan(T, hq, kv.n_kv_heads, d, ctx_len, anc_mask is None, n_splits, kv.fmt)
    if part_o is None:
        part_o = torch.empty((S, T, hq, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((S, T, hq), dtype=torch.float32, device=q.device)
    m_ptr = None
    if anc_mask is not None:
        m = np.ascontiguousarray(np.asarray(anc_mask, dtype=np.uint64))
        if m.shape != (T,):
            raise ValueError(f"anc_mask must have shape ({T},)")
        m_ptr = m.ctypes.data
    layer = kv._layer()
    rc = load_library().stv_attention_partials(
        _dev_ptr(q, torch.float32, "q"), T, hq, ctypes.byref(layer), ctx_len, m_ptr,
        float(softmax_scale), n_splits, _dev_ptr(part_o, torch.float32, "part_o", (S, T, hq, d)),
        _dev_ptr(part_lse, torch.float32, "part_lse", (S, T, hq)), _stream(q.device))
    _check(rc)
    return part_o, part_lse


def context_plan(T: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_keys: int,
                 n_splits: int = 0, fmt: str = "b3") -> tuple[int, int]:
    """(split count, workspace bytes) of a context-slice call (no tree keys)."""
    s = ctypes.c_int32()
    ws = ctypes.c_size_t()
    _check(load_library().stv_context_plan(T, n_q_heads, n_kv_heads, head_dim, n_keys,
                                           _FORMATS[fmt], n_splits, ctypes.byref(s),
                                           ctypes.byref(ws)))
    return int(s.value), int(ws.value)


def context_partials(q, kv: KVCache, n_keys: int, softmax_scale=None, n_splits: int = 0,
                     part_o=None, part_lse=None):
    """Split phase over keys 0 .. n_keys-1 of kv for all T rows (a context
    slice without tree keys): returns (part_o [S][T][Hq][D], part_lse [S][T][Hq])."""
    torch = _torch()
    T, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    S, _ = context_plan(T, hq, kv.n_kv_heads, d, n_keys, n_splits, kv.fmt)
    if part_o is None:
        part_o = torch.empty((S, T, hq, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((S, T, hq), dtype=torch.float32, device=q.device)
    layer = kv._layer()
    rc = load_library().stv_context_partials(
        _dev_ptr(q, torch.float32, "q"), T, hq, ctypes.byref(layer), n_keys, float(softmax_scale),
        n_splits, _dev_ptr(part_o, torch.float32, "part_o", (S, T, hq, d)),
        _dev_ptr(part_lse, torch.float32, "part_lse", (S, T, hq)), _stream(q.device))
    _check(rc)
    return part_o, part_lse


def split_merge(part_o, part_lse, out=None, out_lse=None):
    """Log-sum-exp merge of part_o [S][rows][D] with part_lse [S][rows]."""
    torch = _torch()
    S, rows, d = part_o.shape
    if out is None:
        out = torch.empty((rows, d), dtype=torch.float32, device=part_o.device)
    rc = load_library().stv_split_merge(
        _dev_ptr(part_o, torch.float32, "part_o"),
        _dev_ptr(part_lse, torch.float32, "part_lse", (S, rows)), S, rows, d,
        _dev_ptr(out, torch.float32, "out", (rows, d)),
        _dev_ptr(out_lse, torch.float32, "out_lse", (rows,)), _stream(part_o.device))
    _check(rc)
    return out


def tree_accept(anc_mask, draft, target, path=None, n_accepted=None, bonus=None):
    """Greedy acceptance over the draft tree (see include/stv.h).

    anc_mask: uint64 [T] host masks; draft, target: int32 [T] GPU tensors.
    Returns (path int32 [T], n_accepted int32 [1], bonus int32 [1]) GPU
    tensors; path holds the committed nodes, then -1.
    """
    torch = _torch()
    m = np.ascontiguousarray(np.asarray(anc_mask, dtype=np.uint64))
    T = m.size
    dev = draft.device
    if path is None:
        path = torch.empty(T, dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty(1, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(1, dtype=torch.int32, device=dev)
    rc = load_library().stv_tree_accept(
        m.ctypes.data if T else None, T, _dev_ptr(draft, torch.int32, "draft", (T,)),
        _dev_ptr(target, torch.int32, "target", (T,)), _dev_ptr(path, torch.int32, "path", (T,)),
        _dev_ptr(n_accepted, torch.int32, "n_accepted", (1,)),
        _dev_ptr(bonus, torch.int32, "bonus", (1,)), _stream(dev))
    _check(rc)
    return path, n_accepted, bonus


def kv_commit(kv: KVCache, ctx_len: int, path, n_accepted):
    """Move the committed tree tokens' K/V to positions ctx_len.. (in place)."""
    torch = _torch()
    T = int(path.numel())
    layer = kv._layer()
    rc = load_library().stv_kv_commit(ctypes.byref(layer), ctx_len, T,
                                      _dev_ptr(path, torch.int32, "path", (T,)),
                                      _dev_ptr(n_accepted, torch.int32, "n_accepted", (1,)),
                                      _stream(path.device))
    _check(rc)


def lookup_plan(batch: int, stride: int) -> int:
    """Workspace bytes of a lookup_draft call."""
    ws = ctypes.c_size_t()
    _check(load_library().stv_lookup_plan(batch, stride, ctypes.byref(ws)))
    return int(ws.value)


def lookup_draft(history, lengths, n_min: int = 6, n_max: int = 12, k: int = 8, workspace=None,
                 out=None):
    """Lookup drafting (see include/stv.h).  history: int32 [B][stride] GPU
    tensor; lengths: int32 [B] GPU tensor.  Returns dict(tokens [B][k],
    count, match, pos) of GPU tensors (`out`, when given, is filled)."""
    torch = _torch()
    B, stride = history.shape
    dev = history.device
    ws_bytes = lookup_plan(B, stride)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = {"tokens": torch.empty((B, k), dtype=torch.int32, device=dev),
               "count": torch.empty(B, dtype=torch.int32, device=dev),
               "match": torch.empty(B, dtype=torch.int32, device=dev),
               "pos": torch.empty(B, dtype=torch.int32, device=dev)}
    rc = load_library().stv_lookup_draft(
        _dev_ptr(history, torch.int32, "history"), _dev_ptr(lengths, torch.int32, "lengths", (B,)),
        B, stride, n_min, n_max, k, _dev_ptr(out["tokens"], torch.int32, "tokens", (B, k)) if k else None,
        _dev_ptr(out["count"], torch.int32, "count", (B,)),
        _dev_ptr(out["match"], torch.int32, "match", (B,)),
        _dev_ptr(out["pos"], torch.int32, "pos", (B,)),
        _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(dev))
    _check(rc)
    return out
