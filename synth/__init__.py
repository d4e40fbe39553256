"""Seeded synthetic inputs for the verify-attention path.

This module only draws random numbers.  It holds none of the method's
arithmetic: no quantizer, no packing, no attention.  Both the CPU oracle
and the GPU path read what it returns.

Why raw random words stand in for packed codes: a 3-bit code block stores
32 codes in exactly 96 bits, so 96 uniformly random bits are 32 independent
codes uniform on [0, 7], whatever bit layout each side later reads them
with.  The workload statement (codes uniform in [0, 7]) is therefore met
without any packing code here.

Workload recipe (shapes from the verify round on the elpis pages, "Setup"
/ "Recipe" and the 8-row tree of "How"; distributions from the workload
statement):
  * K and V codes: uniform random 32-bit words, 3 words per 32 elements;
  * K and V scales: U(0.01, 0.1) rounded to fp16, one per 32 elements of
    one (token, KV head) row;
  * Q: standard normal fp32;
  * tree: node 0 is the root; node i > 0 takes a uniformly random parent
    among earlier nodes whose depth is below the depth cap.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Geometry", "CONFIGS", "EXTRA_CONFIGS", "KVCache",
    "make_kv", "make_q", "make_tree_parents", "ancestor_masks",
    "chain_parents", "all_tree_shapes", "make_new_rows",
]


@dataclass(frozen=True)
class Geometry:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int          # L: keys already in the cache before the new rows
    n_rows: int           # T: new query tokens (tree nodes or prefill chunk)
    kind: str             # "tree", "chain" or "prefill"
    max_depth: int        # depth cap for random trees (1 = root only)
    seed: int

    @property
    def n_keys(self) -> int:
        return self.ctx_len + self.n_rows


# The five workload configurations, in order: tiny parity case, single-token
# decode, 64-node tree at 32K, 64-node tree at 262K, 4,096-token prefill.
CONFIGS = [
    Geometry("tiny", 4, 1, 64, 512, 8, "chain", 8, 0),
    Geometry("decode_8k", 24, 4, 256, 8192, 1, "tree", 1, 1),
    Geometry("tree64_32k", 24, 4, 256, 32768, 64, "tree", 8, 2),
    Geometry("tree64_262k", 24, 4, 256, 262144, 64, "tree", 8, 3),
    Geometry("prefill_4k_32k", 24, 4, 256, 32768, 4096, "prefill", 0, 4),
]

# Shapes where streaming the cache, not the matrix pipe, bounds the call:
# the pages' own 8-row tree at 262K, and one query token at 262K.
EXTRA_CONFIGS = [
    Geometry("tree8_262k", 24, 4, 256, 262144, 8, "tree", 8, 5),
    Geometry("decode_262k", 24, 4, 256, 262144, 1, "tree", 1, 6),
]


@dataclass
class KVCache:
    """Host arrays of one layer's quantized K/V cache.

    K, token-major:    k_codes uint32 [Hkv][capacity][D/32][3],
                       k_scales uint16 (fp16 bits) [Hkv][capacity][D/32]
    V, key-transposed: v_codes uint32 [Hkv][ng][D][3],
                       v_scales uint16 (fp16 bits) [Hkv][ng][D/32][32]
    with ng = ceil(capacity / 32) groups of 32 keys.  K positions >= n_filled
    are zero; V groups past the one holding key n_filled - 1 are zero (the
    rest of that last group holds random data, which no call reads).
    """
    k_codes: np.ndarray
    k_scales: np.ndarray
    v_codes: np.ndarray
    v_scales: np.ndarray
    n_kv_heads: int
    head_dim: int
    capacity: int
    n_filled: int
    fmt: str = "b3"


def _scales(rng: np.random.Generator, shape) -> np.ndarray:
    s = rng.uniform(0.01, 0.1, size=shape)
    return s.astype(np.float16).view(np.uint16)


def make_kv(rng: np.random.Generator, n_kv_heads: int, head_dim: int,
            n_filled: int, capacity: int | None = None) -> KVCache:
    if capacity is None:
        capacity = n_filled
    assert head_dim % 32 == 0 and 0 <= n_filled <= capacity
    nb = head_dim // 32
    k_codes = np.zeros((n_kv_heads, capacity, nb, 3), dtype=np.uint32)
    k_scales = np.zeros((n_kv_heads, capacity, nb), dtype=np.uint16)
    k_codes[:, :n_filled] = rng.integers(0, 2**32, size=(n_kv_heads, n_filled, nb, 3),
                                         dtype=np.uint32)
    k_scales[:, :n_filled] = _scales(rng, (n_kv_heads, n_filled, nb))
    ng = (capacity + 31) // 32
    ng_filled = (n_filled + 31) // 32
    v_codes = np.zeros((n_kv_heads, ng, head_dim, 3), dtype=np.uint32)
    v_scales = np.zeros((n_kv_heads, ng, nb, 32), dtype=np.uint16)
    v_codes[:, :ng_filled] = rng.integers(0, 2**32, size=(n_kv_heads, ng_filled, head_dim, 3),
                                          dtype=np.uint32)
    v_scales[:, :ng_filled] = _scales(rng, (n_kv_heads, ng_filled, nb, 32))
    return KVCache(k_codes, k_scales, v_codes, v_scales, n_kv_heads, head_dim, capacity, n_filled)


def make_q(rng: np.random.Generator, n_rows: int, n_q_heads: int, head_dim: int) -> np.ndarray:
    return rng.standard_normal((n_rows, n_q_heads, head_dim), dtype=np.float32)


def make_tree_parents(rng: np.random.Generator, n_nodes: int, max_depth: int) -> np.ndarray:
    """Parent array of a random tree: parent[0] = -1, parent[i] < i.

    Node 0 (the root) has depth 1; a node may only hang below a node whose
    depth is under max_depth, so no node is deeper than max_depth.
    """
    parent = np.full(n_nodes, -1, dtype=np.int64)
    depth = np.zeros(n_nodes, dtype=np.int64)
    if n_nodes == 0:
        return parent
    depth[0] = 1
    for i in range(1, n_nodes):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(rng.choice(cand))
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def chain_parents(n_nodes: int) -> np.ndarray:
    p = np.arange(-1, n_nodes - 1, dtype=np.int64)
    return p


def ancestor_masks(parent: np.ndarray) -> np.ndarray:
    """The input format of the verify call: bit a of mask[i] is set iff node a
    is node i or one of its ancestors (parent[i] < i for every node)."""
    n = len(parent)
    assert n <= 64
    m = np.zeros(n, dtype=np.uint64)
    for i in range(n):
        own = np.uint64(1) << np.uint64(i)
        m[i] = own if parent[i] < 0 else (m[parent[i]] | own)
    return m


def all_tree_shapes(n_nodes: int):
    """Every parent array with parent[0] = -1 and parent[i] in [0, i):
    (n_nodes - 1)! shapes (5,040 for the pages' 8-row tree)."""
    def rec(prefix):
        i = len(prefix)
        if i == n_nodes:
            yield np.array(prefix, dtype=np.int64)
            return
        for p in range(i):
            yield from rec(prefix + [p])
    if n_nodes == 0:
        return
    yield from rec([-1])


def make_new_rows(rng: np.random.Generator, n_tok: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """fp32 K or V rows of the new tokens, before they enter the 3-bit cache."""
    return rng.standard_normal((n_tok, n_kv_heads, head_dim), dtype=np.float32)


def make_tree_tokens(rng: np.random.Generator, parent: np.ndarray, vocab: int,
                     p_follow: float = 0.6) -> tuple[np.ndarray, np.ndarray]:
    """Draft tokens of the tree nodes and the target's greedy token at every
    tree row, for acceptance tests and benchmarks.

    Draft tokens are uniform over [0, vocab).  The target token of row i is,
    with probability p_follow, the draft token of one of i's children picked
    uniformly (so some draft paths are followed for a while), else uniform.
    """
    n = len(parent)
    draft = rng.integers(0, vocab, size=n).astype(np.int32)
    target = rng.integers(0, vocab, size=n).astype(np.int32)
    for i in range(n):
        kids = [c for c in range(n) if parent[c] == i]
        if kids and rng.random() < p_follow:
            target[i] = draft[int(rng.choice(kids))]
    return draft, target


def make_lookup_history(rng: np.random.Generator, n_tokens: int, vocab: int, copy_len: int,
                        n_decoys: int = 16) -> np.ndarray:
    """A token history for lookup-drafting tests and benchmarks.

    Tokens are uniform over [0, vocab).  The last copy_len tokens repeat an
    earlier span (so the history's tail occurs earlier), and n_decoys shorter
    copies of the tail's last 1..copy_len-1 tokens are planted at random
    earlier places.
    """
    h = rng.integers(0, vocab, size=n_tokens).astype(np.int32)
    if copy_len > 0 and n_tokens > 2 * copy_len + 1:
        p = int(rng.integers(0, n_tokens - 2 * copy_len))
        h[n_tokens - copy_len:] = h[p:p + copy_len]
        for _ in range(n_decoys):
            j = int(rng.integers(1, copy_len))
            q = int(rng.integers(0, n_tokens - copy_len - j))
            if q + j > p and q < p + copy_len:
                continue                      # keep the planted span whole
            h[q:q + j] = h[n_tokens - j:]
    return h


def make_kv4(rng: np.random.Generator, n_kv_heads: int, head_dim: int,
             n_filled: int, capacity: int | None = None) -> KVCache:
    """A 4-bit per-token-head cache (fmt "i4"):

    K, token-major:    k_codes uint32 [Hkv][capacity][D/8] (8 codes per word),
                       k_scales uint16 (fp16 bits) [Hkv][capacity]
    V, key-transposed: v_codes uint32 [Hkv][ng][D][4] (32 keys per row),
                       v_scales uint16 (fp16 bits) [Hkv][capacity]
    Codes uniform in [0, 15], scales U(0.01, 0.1); positions past n_filled
    (K) and groups past the last filled key (V) are zero.
    """
    if capacity is None:
        capacity = n_filled
    assert head_dim % 32 == 0 and 0 <= n_filled <= capacity
    ng = (capacity + 31) // 32
    kc = np.zeros((n_kv_heads, capacity, head_dim // 8), dtype=np.uint32)
    ks = np.zeros((n_kv_heads, capacity), dtype=np.uint16)
    vc = np.zeros((n_kv_heads, ng, head_dim, 4), dtype=np.uint32)
    vs = np.zeros((n_kv_heads, capacity), dtype=np.uint16)
    kc[:, :n_filled] = rng.integers(0, 2**32, size=(n_kv_heads, n_filled, head_dim // 8),
                                    dtype=np.uint32)
    ks[:, :n_filled] = _scales(rng, (n_kv_heads, n_filled))
    g_used = (n_filled + 31) // 32
    vc[:, :g_used] = rng.integers(0, 2**32, size=(n_kv_heads, g_used, head_dim, 4),
                                  dtype=np.uint32)
    vs[:, :n_filled] = _scales(rng, (n_kv_heads, n_filled))
    return KVCache(kc, ks, vc, vs, n_kv_heads, head_dim, capacity, n_filled, "i4")
