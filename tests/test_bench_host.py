"""CPU: the benchmark's host logic -- the one-GPU guard, the algorithmic
byte and MAC counts its rates divide by (checked against a brute-force count
over the masks), the call and kernel timing split, the kernel it names for
each workload, and the gate that reports counter-measured traffic only for
the kernel sources it was measured at."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _geom(**kw):
    base = dict(name="t", n_q_heads=8, n_kv_heads=2, head_dim=64, ctx_len=100, n_rows=5,
                kind="tree", max_depth=8, seed=0)
    base.update(kw)
    return synth.Geometry(**base)


@pytest.mark.parametrize("masks", [None, "chain", "tree"])
def test_work_counts_match_a_brute_force_count(masks):
    g = _geom()
    T, L, hq, d = g.n_rows, g.ctx_len, g.n_q_heads, g.head_dim
    rng = np.random.default_rng(7)
    if masks == "chain":
        m = synth.ancestor_masks(synth.chain_parents(T))
    elif masks == "tree":
        m = synth.ancestor_masks(synth.make_tree_parents(rng, T, 3))
    else:
        m = None
    w = bench.work_of(g, m)
    # visible keys per (row, query head): the context, then the row's own
    # visible new keys (causal: itself and the ones before it)
    vis = 0
    for t in range(T):
        own = (t + 1) if m is None else sum(1 for u in range(T) if (int(m[t]) >> u) & 1)
        vis += (L + own) * hq
    assert w["qk_ops"] == 2 * vis * d and w["pv_ops"] == 2 * vis * d
    # 3-bit cache: per key and KV head, K and V each hold D/32 blocks of 12
    # code bytes and a 2-byte scale
    n_keys = L + T
    assert w["kv_bytes"] == n_keys * g.n_kv_heads * 2 * (d // 32) * 14
    assert w["q_bytes"] == w["out_bytes"] == T * hq * d * 4
    assert w["attn_bytes"] == w["kv_bytes"] + w["q_bytes"] + w["out_bytes"]
    w4 = bench.work_of(g, m, "i4")
    assert w4["kv_bytes"] == n_keys * g.n_kv_heads * 2 * (d // 2 + 2)


def test_a_chain_and_causal_rows_see_the_same_keys():
    g = _geom(n_rows=7)
    chain = synth.ancestor_masks(synth.chain_parents(g.n_rows))
    assert bench.work_of(g, chain)["qk_ops"] == bench.work_of(g, None)["qk_ops"]


class _FakeWorkload:
    def __init__(self, g):
        self.work = bench.work_of(g, None)
        self.S = 3
        self.images = False


def test_call_time_comes_from_the_steps_without_a_middle_event():
    g = _geom()
    r = {"wall_s": 0.01, "attn_ms": [0.100, 0.110], "merge_ms": [0.020, 0.020],
         "call_ms": [0.115, 0.125]}
    s = bench.summarize(_FakeWorkload(g), r, 4)
    assert s["attn_kernel_us"] == pytest.approx(105.0)
    assert s["merge_kernel_us"] == pytest.approx(20.0)
    assert s["us_per_call"] == pytest.approx(120.0)
    assert s["us_per_call_median"] == pytest.approx(120.0)
    assert s["ms_per_step"] == pytest.approx(2.5)
    assert s["hbm_gbs"] == pytest.approx(_FakeWorkload(g).work["attn_bytes"] / 120e-6 / 1e9)


@pytest.mark.parametrize("name,fmt,kernel", [
    ("decode_262k", "b3", "attn_dec_kernel"),        # 6 rows per KV head
    ("tree8_262k", "b3", "attn_split16_kernel"),     # 48 rows
    ("tree8_262k", "i4", "attn_dec_kernel"),         # the 4-bit few-row kernel takes up to 64
    ("tree64_262k", "b3", "attn_ws_kernel"),         # 384 rows, 3-bit, head_dim 256
    ("tree64_262k", "i4", "attn_split_kernel"),
    ("prefill_4k_32k", "b3", "attn_split_kernel"),   # causal
])
def test_kernel_named_for_each_workload(name, fmt, kernel):
    g = [x for x in synth.CONFIGS + synth.EXTRA_CONFIGS if x.name == name][0]
    assert bench.attention_kernel_of(g, fmt, g.kind == "prefill") == kernel


def test_traffic_is_reported_only_at_the_measured_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = tmp_path / "profiles" / "hbm_traffic_attn_ws_kernel_tree64_262k.md"
    assert bench.measured_traffic("attn_ws_kernel", "tree64_262k") is None
    f.write_text("# summary\n\ntraffic_bytes_per_launch: 123456\n"
                 f"kernel_source_sha256: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic("attn_ws_kernel", "tree64_262k") == 123456
    f.write_text("traffic_bytes_per_launch: 123456\nkernel_source_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("attn_ws_kernel", "tree64_262k") is None
