#!/usr/bin/env python3
"""Benchmark of the verify-round attention path on one MI355X.

One step is one pass of the whole hot path for one layer of a verify round:
  1. append the T new rows' K and V to the 3-bit cache (kv_quant_pack x2),
  2. the split attention kernel (int8 Q.K^T, fp32 online softmax, P.V),
  3. the log-sum-exp merge of the split partials.
The headline workload is the 64-node draft tree over a 262,144-token context
(24 query / 4 KV heads, head_dim 256).  Four distinct caches are rotated so
every step streams its cache from HBM rather than from the 256 MB Infinity
Cache.  Inputs are seeded synthetic data already resident on the GPU.

Prints one JSON line (see the keys below).  Extra workloads (the prefill
chunk, the pages' 8-row tree and one query token at 262K, the 8K decode and
the 32K tree) are reported under "extra".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "µs/verify-round attn + HBM GB/s (% peak) at 262K ctx; prefill int8 MFMA %"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0          # dense int8 MFMA
FP16_PEAK_TFLOPS = 2500.0        # dense fp16 MFMA
N_BUFFERS = 4                    # 4 x 235 MB > 256 MB Infinity Cache
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_tree_verify_amd", "csrc", f)
                  for f in ("stv_kernels.hip", "stv_internal.h", "stv_codes.h")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary for this kernel and workload, or None when
    there is none or the kernel sources changed after the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`")
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_kernel_of(geom: synth.Geometry, fmt: str, causal: bool) -> str:
    """The attention kernel the library's plan runs for a workload (the same
    row-count thresholds as the plan)."""
    rows = geom.n_rows * (geom.n_q_heads // geom.n_kv_heads)
    if rows <= (64 if fmt == "i4" else 16):
        return "attn_dec_kernel"
    if fmt == "b3" and rows <= 64:
        return "attn_split16_kernel"
    row_tiles = (rows + 31) // 32
    if fmt == "b3" and not causal and geom.head_dim == 256 and row_tiles >= 4:
        return "attn_ws_kernel"
    return "attn_split_kernel"


def work_of(geom: synth.Geometry, masks, fmt: str = "b3"):
    """Algorithmic bytes and operations of one step (see the design notes)."""
    T, hq, hkv, d, L = geom.n_rows, geom.n_q_heads, geom.n_kv_heads, geom.head_dim, geom.ctx_len
    nb = d // 32
    n_keys = L + T
    # codes + fp16 scales per (key, KV head), K and V
    per_key_head = 2 * nb * (12 + 2) if fmt == "b3" else 2 * (d // 2 + 2)
    kv_bytes = n_keys * hkv * per_key_head
    q_bytes = T * hq * d * 4
    out_bytes = T * hq * d * 4
    append_bytes = 2 * T * hkv * d * 4 + T * hkv * per_key_head
    if masks is None:
        visible = sum(L + t + 1 for t in range(T)) * hq
    else:
        visible = sum(L + bin(int(m)).count("1") for m in masks) * hq
    macs = visible * d                                     # per product (Q.K^T, and P.V)
    return {
        "kv_bytes": kv_bytes, "q_bytes": q_bytes, "out_bytes": out_bytes,
        "append_bytes": append_bytes,
        "attn_bytes": kv_bytes + q_bytes + out_bytes,
        "step_bytes": kv_bytes + q_bytes + out_bytes + append_bytes,
        "qk_ops": 2 * macs, "pv_ops": 2 * macs,
    }


class Workload:
    def __init__(self, geom: synth.Geometry, torch, stv, n_buffers=N_BUFFERS, fmt="b3",
                 pv16=False):
        self.g = geom
        self.torch = torch
        self.stv = stv
        self.fmt = fmt
        # pv16: the fp16-accumulated P.V variant, one call (its merge included)
        self.pv16 = pv16
        rng = np.random.default_rng(geom.seed)
        make = synth.make_kv if fmt == "b3" else synth.make_kv4
        host = make(rng, geom.n_kv_heads, geom.head_dim, geom.n_keys)
        self.host = host
        self.q_host = synth.make_q(rng, geom.n_rows, geom.n_q_heads, geom.head_dim)
        self.causal = geom.kind == "prefill"
        self.mask = None
        if not self.causal:
            parents = (synth.chain_parents(geom.n_rows) if geom.kind == "chain"
                       else synth.make_tree_parents(rng, geom.n_rows, geom.max_depth))
            self.mask = synth.ancestor_masks(parents)
            self.parents = parents
        knew = synth.make_new_rows(rng, geom.n_rows, geom.n_kv_heads, geom.head_dim)
        vnew = synth.make_new_rows(rng, geom.n_rows, geom.n_kv_heads, geom.head_dim)
        dev = "cuda"
        base = stv.KVCache.from_host(host, device=dev)
        self.caches = [base] + [stv.KVCache(base.k_codes.clone(), base.k_scales.clone(),
                                            base.v_codes.clone(), base.v_scales.clone(), fmt)
                                for _ in range(n_buffers - 1)]
        self.q = torch.from_numpy(self.q_host).to(dev)
        self.knew = torch.from_numpy(knew).to(dev)
        self.vnew = torch.from_numpy(vnew).to(dev)
        self.scale = 1.0 / math.sqrt(geom.head_dim)
        self.S, self.ws_bytes = stv.attention_plan(geom.n_rows, geom.n_q_heads, geom.n_kv_heads,
                                                   geom.head_dim, geom.ctx_len, self.causal, 0,
                                                   fmt)
        T, hq, d = geom.n_rows, geom.n_q_heads, geom.head_dim
        # the plan asks for more than the partials when a causal chunk unpacks
        # its tiles once into images in the workspace
        self.images = self.ws_bytes > stv.workspace_bytes(T, hq, d, self.S)
        self.part_o = self.part_lse = None
        if self.S > 1:
            self.part_o = torch.empty((self.S, T, hq, d), dtype=torch.float32, device=dev)
            self.part_lse = torch.empty((self.S, T, hq), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, hq, d), dtype=torch.float32, device=dev)
        self.out_lse = torch.empty((T, hq), dtype=torch.float32, device=dev)
        self.work = work_of(geom, self.mask, fmt)
        self._prepare_calls()

    def _prepare_calls(self):
        """Marshals every C-ABI call of a step once per cache, so that a step
        costs the host a few microseconds and the launches queue up ahead of
        the GPU (the events then time the kernels, not host gaps).  The calls
        are the ones the package's Python functions make."""
        import ctypes
        stv, g, torch = self.stv, self.g, self.torch
        lib = stv.load_library()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        T, hq, d = g.n_rows, g.n_q_heads, g.head_dim
        codes = {"b3": (stv.STV_K, stv.STV_V), "i4": (stv.STV_K4, stv.STV_V4)}[self.fmt]
        self._mask_arr = (None if self.mask is None
                          else np.ascontiguousarray(np.asarray(self.mask, dtype=np.uint64)))
        mask_ptr = None if self._mask_arr is None else self._mask_arr.ctypes.data
        self._layers = [kv._layer() for kv in self.caches]
        self._calls = []
        for kv, layer in zip(self.caches, self._layers):
            pack = [(lib.stv_kv_quant_pack, (x.data_ptr(), T, g.ctx_len, code, c.data_ptr(),
                                            sc.data_ptr(), g.n_kv_heads, d, kv.capacity, stream))
                    for x, code, c, sc in ((self.knew, codes[0], kv.k_codes, kv.k_scales),
                                           (self.vnew, codes[1], kv.v_codes, kv.v_scales))]
            lref = ctypes.byref(layer)
            if self.pv16:
                if not hasattr(self, "_ws"):
                    self._ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8,
                                           device="cuda")
                attn = (lib.stv_verify_attention_fp16acc,
                        (self.q.data_ptr(), T, hq, lref, g.ctx_len, mask_ptr, self.scale,
                         self.out.data_ptr(), self.out_lse.data_ptr(), self._ws.data_ptr(),
                         self.ws_bytes, 0, stream))
                merge = None
            elif self.images:
                # the causal chunk with tile images: the whole call (image
                # pre-pass, attention and merge) is one ABI call, timed as the
                # attention phase
                if not hasattr(self, "_ws"):
                    self._ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
                attn = (lib.stv_prefill_attention,
                        (self.q.data_ptr(), T, hq, lref, g.ctx_len, self.scale,
                         self.out.data_ptr(), self.out_lse.data_ptr(), self._ws.data_ptr(),
                         self.ws_bytes, 0, None, None, None, stream))
                merge = None
            elif self.S == 1:
                # one split: the attention kernel writes the output itself
                if self.causal:
                    attn = (lib.stv_prefill_attention,
                            (self.q.data_ptr(), T, hq, lref, g.ctx_len, self.scale,
                             self.out.data_ptr(), self.out_lse.data_ptr(), None, 0, 0, None,
                             None, None, stream))
                else:
                    attn = (lib.stv_verify_attention,
                            (self.q.data_ptr(), T, hq, lref, g.ctx_len, mask_ptr, self.scale,
                             self.out.data_ptr(), self.out_lse.data_ptr(), None, 0, 0, None,
                             None, None, stream))
                merge = None
            else:
                attn = (lib.stv_attention_partials,
                        (self.q.data_ptr(), T, hq, lref, g.ctx_len, mask_ptr, self.scale, 0,
                         self.part_o.data_ptr(), self.part_lse.data_ptr(), stream))
                merge = (lib.stv_split_merge,
                         (self.part_o.data_ptr(), self.part_lse.data_ptr(), self.S, T * hq, d,
                          self.out.data_ptr(), self.out_lse.data_ptr(), stream))
            self._calls.append((pack, attn, merge))

    def step(self, i, ev=None, mid=True):
        """One step; with events, ev[0] before the attention call and ev[2]
        after the merge, and ev[1] between the two only when mid is set (an
        event between the launches adds about 2 us to the pair)."""
        check = self.stv._check
        pack, attn, merge = self._calls[i % len(self._calls)]
        for fn, args in pack:
            check(fn(*args))
        if ev is not None:
            ev[0].record()
        check(attn[0](*attn[1]))
        if ev is not None and mid:
            ev[1].record()
        if merge is not None:
            check(merge[0](*merge[1]))
        if ev is not None:
            ev[2].record()

    def run(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        # Even steps time the attention kernel and the merge apart (an event
        # between them); odd steps time the call, attention then merge, with
        # no event between the launches.
        for i in range(steps):
            self.step(warmup + i, evs[i], mid=(i % 2 == 0))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        attn_ms = [e[0].elapsed_time(e[1]) for e in evs[0::2]]
        merge_ms = [e[1].elapsed_time(e[2]) for e in evs[0::2]]
        call_ms = [e[0].elapsed_time(e[2]) for e in evs[1::2]]
        if not call_ms:
            call_ms = [a + m for a, m in zip(attn_ms, merge_ms)]
        return {"wall_s": wall, "attn_ms": attn_ms, "merge_ms": merge_ms, "call_ms": call_ms}


def accept_commit_bench(wl: Workload, steps: int):
    """Times the end of a verify round on the workload's tree: greedy
    acceptance then the accepted-path commit of the 3-bit K/V (one call
    each, device-side path and count)."""
    torch, stv, g = wl.torch, wl.stv, wl.g
    rng = np.random.default_rng(g.seed + 100)
    draft, target = synth.make_tree_tokens(rng, wl.parents, vocab=2, p_follow=0.9)
    d = torch.from_numpy(draft).cuda()
    t = torch.from_numpy(target).cuda()
    path = torch.empty(g.n_rows, dtype=torch.int32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    bonus = torch.empty(1, dtype=torch.int32, device="cuda")
    for i in range(3):
        stv.tree_accept(wl.mask, d, t, path, n, bonus)
        stv.kv_commit(wl.caches[i % len(wl.caches)], g.ctx_len, path, n)
    torch.cuda.synchronize()
    # the same C-ABI calls, marshalled once (see Workload._prepare_calls)
    import ctypes
    lib = stv.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    T = g.n_rows
    accept = (wl._mask_arr.ctypes.data, T, d.data_ptr(), t.data_ptr(), path.data_ptr(),
              n.data_ptr(), bonus.data_ptr(), stream)
    commits = [(ctypes.byref(layer), g.ctx_len, T, path.data_ptr(), n.data_ptr(), stream)
               for layer in wl._layers]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(steps):
        stv._check(lib.stv_tree_accept(*accept))
        stv._check(lib.stv_kv_commit(*commits[i % len(commits)]))
    ev[1].record()
    torch.cuda.synchronize()
    n_acc = int(n.item())
    return {"us_per_call": round(ev[0].elapsed_time(ev[1]) * 1e3 / steps, 2),
            "n_accepted": n_acc, "tree_nodes": g.n_rows,
            "moved_bytes": n_acc * g.n_kv_heads * 2 * (g.head_dim // 32) * 14}


def lookup_bench(torch, stv, batch: int, n_tokens: int, steps: int, n_buffers: int = 1):
    """Lookup drafting over `batch` histories of n_tokens tokens each (vocab
    151,936, the tail copied from earlier in the history), rotating n_buffers
    distinct batches; the scan reads every token once, so its algorithmic
    bytes are batch * n_tokens * 4 per call."""
    rng = np.random.default_rng(7)
    bufs = []
    for _ in range(n_buffers):
        hist = np.stack([synth.make_lookup_history(rng, n_tokens, 151936, 12)
                         for _ in range(batch)])
        bufs.append(torch.from_numpy(hist).cuda())
    ln = torch.full((batch,), n_tokens, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(stv.lookup_plan(batch, n_tokens), 1), dtype=torch.uint8, device="cuda")
    out = {"tokens": torch.empty((batch, 8), dtype=torch.int32, device="cuda"),
           "count": torch.empty(batch, dtype=torch.int32, device="cuda"),
           "match": torch.empty(batch, dtype=torch.int32, device="cuda"),
           "pos": torch.empty(batch, dtype=torch.int32, device="cuda")}
    for i in range(3):
        stv.lookup_draft(bufs[i % n_buffers], ln, 6, 12, 8, workspace=ws, out=out)
    torch.cuda.synchronize()
    # the same C-ABI call, marshalled once (see Workload._prepare_calls)
    import ctypes
    lib = stv.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = [(b.data_ptr(), ln.data_ptr(), batch, n_tokens, 6, 12, 8, out["tokens"].data_ptr(),
              out["count"].data_ptr(), out["match"].data_ptr(), out["pos"].data_ptr(),
              ws.data_ptr(), ws.numel(), stream) for b in bufs]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(steps):
        stv._check(lib.stv_lookup_draft(*calls[i % n_buffers]))
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    nbytes = batch * n_tokens * 4
    return {"us_per_call": round(us, 2), "batch": batch, "tokens_per_history": n_tokens,
            "buffers_rotated": n_buffers,
            "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "match_len": int(out["match"][0].item())}


def summarize(wl: Workload, r, steps):
    w = wl.work
    ms_step = r["wall_s"] * 1e3 / steps
    attn = float(np.mean(r["attn_ms"]))
    merge = float(np.mean(r["merge_ms"]))
    call_us = float(np.mean(r["call_ms"])) * 1e3
    call_med_us = float(np.median(r["call_ms"])) * 1e3
    mfma_s = w["qk_ops"] / (INT8_PEAK_TOPS * 1e12) + w["pv_ops"] / (FP16_PEAK_TFLOPS * 1e12)
    return {
        "ms_per_step": ms_step,
        "attn_kernel_us": attn * 1e3,
        "merge_kernel_us": merge * 1e3,
        "us_per_call": call_us,
        "us_per_call_median": call_med_us,
        "splits": wl.S,
        # what attn_kernel_us covers
        "attn_timed": ("tile-image pre-pass + attention + merge (one call)" if wl.images
                       else "attention kernel"),
        "hbm_gbs": w["attn_bytes"] / (call_us * 1e-6) / 1e9,
        "hbm_frac": w["attn_bytes"] / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "kernel_hbm_gbs": w["attn_bytes"] / (attn * 1e-3) / 1e9,
        "int8_mfma_frac": w["qk_ops"] / (attn * 1e-3) / (INT8_PEAK_TOPS * 1e12),
        "matrix_pipe_frac": mfma_s / (attn * 1e-3),
        "ideal_mfma_us": mfma_s * 1e6,
        "ideal_hbm_us": w["attn_bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6,
    }


def cpu_baseline(wl: Workload, n_rows: int):
    import oracle
    g = wl.g
    total = g.n_rows * g.n_q_heads
    n_rows = min(n_rows, total)
    rows = np.linspace(0, total - 1, n_rows).round().astype(np.int32)
    threads = oracle.set_threads(len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    oracle.attention(wl.q_host, wl.host, g.ctx_len, wl.mask, wl.scale, rows=rows)
    el = time.perf_counter() - t0
    full_s = el * total / n_rows
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": wl.work["attn_bytes"] / full_s / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": model,
            "sample": f"{n_rows} of {total} query rows of {g.name} (full context), {el:.1f} s; "
                      f"scaled to the whole call: {full_s * 1e6:.0f} us"}


def parse_workload(name: str):
    """'tree8_262k_i4' -> ('tree8_262k', 'i4', False); '_pv16' -> fp16-accumulated P.V."""
    if name.endswith("_i4"):
        return name[:-3], "i4", False
    if name.endswith("_pv16"):
        return name[:-5], "b3", True
    return name, "b3", False


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tree64_262k")
    ap.add_argument("--extra", default="prefill_4k_32k,tree8_262k,decode_262k,decode_8k,tree64_32k,"
                                       "tree64_262k_i4,prefill_4k_32k_i4,tree8_262k_i4,decode_262k_i4,"
                                       "tree8_262k_pv16,decode_262k_pv16",
                    help="comma-separated extra workloads ('' for none); suffix _i4: the 4-bit "
                         "per-token-head cache; _pv16: fp16-accumulated P.V (whole call)")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--no-lookup", dest="lookup", action="store_false",
                    help="skip the lookup-drafting lines under extra")
    ap.add_argument("--cpu-rows", type=int, default=128, help="oracle sample size (0: skip)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the run, launch an elementwise copy (torch.neg) of this many MiB "
                         "three times: the reference for scaling HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import speculative_tree_verify_amd as stv
    stv.load_library()
    geoms = {g.name: g for g in synth.CONFIGS + synth.EXTRA_CONFIGS}
    wbase, wfmt, wpv16 = parse_workload(args.workload)
    wl = Workload(geoms[wbase], torch, stv, fmt=wfmt, pv16=wpv16)
    r = wl.run(args.steps, args.warmup)
    s = summarize(wl, r, args.steps)
    g = wl.g
    w = wl.work
    total_ops = w["qk_ops"] + w["pv_ops"]
    blended_peak = total_ops / (w["qk_ops"] / INT8_PEAK_TOPS + w["pv_ops"] / FP16_PEAK_TFLOPS)
    achieved = total_ops / (s["attn_kernel_us"] * 1e-6) / 1e12
    kernel_name = attention_kernel_of(g, wl.fmt, wl.causal)
    line = {
        "metric": METRIC,
        "value": round(w["step_bytes"] / (s["ms_per_step"] * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi8->i32, f16xf16->f32, f32",
        "data": "synthetic (seeded; 3-bit codes uniform, fp16 scales U(0.01,0.1), Q N(0,1))",
        "config": {"workload": g.name, "ctx_len": g.ctx_len, "tree_nodes": g.n_rows,
                   "q_heads": g.n_q_heads, "kv_heads": g.n_kv_heads, "head_dim": g.head_dim,
                   "kv_bits": 3, "splits": wl.S, "kv_buffers_rotated": N_BUFFERS},
        "us_per_verify_call": round(s["us_per_call"], 2),
        "us_per_verify_call_median": round(s["us_per_call_median"], 2),
        "hbm_gbs_per_call": round(s["hbm_gbs"], 1),
        "hbm_frac_per_call": round(s["hbm_frac"], 4),
        "roofline": {
            "kernel": kernel_name,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(blended_peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / blended_peak, 4),
            "traffic": measured_traffic(kernel_name, g.name),
            "kernel_us": round(s["attn_kernel_us"], 2),
            "ideal_mfma_us": round(s["ideal_mfma_us"], 2),
            "ideal_hbm_us": round(s["ideal_hbm_us"], 2),
        },
    }
    extra = {}
    if wl.mask is not None and wl.fmt == "b3":
        extra[f"accept_commit_{g.name}"] = accept_commit_bench(wl, args.extra_steps)
    for name in [n for n in args.extra.split(",") if n]:
        del wl
        torch.cuda.empty_cache()
        base, fmt, pv16 = parse_workload(name)
        wl = Workload(geoms[base], torch, stv, fmt=fmt, pv16=pv16)
        rr = wl.run(args.extra_steps, 2)
        se = summarize(wl, rr, args.extra_steps)
        extra[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in se.items()}
    if args.lookup:
        extra["lookup_1x262k"] = lookup_bench(torch, stv, 1, 262144, args.extra_steps)
        extra["lookup_256x262k"] = lookup_bench(torch, stv, 256, 262144, args.extra_steps,
                                                n_buffers=2)
    if extra:
        line["extra"] = extra
    if args.calib_copy_mb > 0:
        del wl
        torch.cuda.empty_cache()
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        line["calib_copy"] = {"kernel": "torch.neg (fp32, contiguous)", "read_bytes": 4 * n,
                              "write_bytes": 4 * n}
        del src, dst
        torch.cuda.empty_cache()
        wl = None
    if args.cpu_rows > 0:
        del wl
        torch.cuda.empty_cache()
        wl = Workload(geoms[wbase], torch, stv, n_buffers=1, fmt=wfmt, pv16=wpv16)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
