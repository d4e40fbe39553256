"""GPU: verify attention captured in a HIP graph and replayed (the pages
test their verify kernel over repeated graph replays, bit for bit:
elpis-lossless, "Proofs and tests").

Each case captures one verify call (attention kernel, and the merge when
the plan has several splits) into a graph, then replays it several times
with eager work and synchronizations between the replays, on the captured
inputs and on new inputs copied into the same buffers; every replay must
equal an eager call on the same inputs bit for bit.  The library's
launches record no memset nodes (buffers are written in full by kernels).
"""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_tree_verify_amd as stv
    stv.load_library()
    return stv, torch


CASES = [
    # name, hq, hkv, d, L, T, fmt (few-row, 16-row and 32-row kernels; 4-bit few-row)
    ("one_token", 24, 4, 256, 3000, 1, "b3"),
    ("tree8", 24, 4, 256, 3000, 8, "b3"),
    ("tree64", 24, 4, 256, 2000, 64, "b3"),
    ("tree8_4bit", 24, 4, 256, 3000, 8, "i4"),
]


@pytest.mark.parametrize("name,hq,hkv,d,L,T,fmt", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(gpu, name, hq, hkv, d, L, T, fmt):
    stv, torch = gpu
    rng = np.random.default_rng(400 + T)
    make = synth.make_kv if fmt == "b3" else synth.make_kv4
    host = make(rng, hkv, d, L + T)
    kv = stv.KVCache.from_host(host)
    mask = synth.ancestor_masks(synth.make_tree_parents(rng, T, 8) if T > 1
                                else synth.chain_parents(1))
    scale = 1.0 / math.sqrt(d)
    qs = [torch.from_numpy(synth.make_q(rng, T, hq, d)).cuda() for _ in range(3)]
    _, ws_bytes = stv.attention_plan(T, hq, hkv, d, L, False, 0, fmt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    q_static = qs[0].clone()
    out_static = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
    lse_static = torch.empty((T, hq), dtype=torch.float32, device="cuda")

    def eager(q):
        lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
        o = stv.verify_attention(q, kv, L, mask, scale, out_lse=lse, workspace=ws)
        return o.clone(), lse.clone()

    # warm the plan cache and the kernels before capture
    ref = [eager(q) for q in qs]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            stv.verify_attention(q_static, kv, L, mask, scale, out=out_static,
                                 out_lse=lse_static, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % 3
        q_static.copy_(qs[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static, ref[i][0]), f"replay {rep} differs from eager"
        assert torch.equal(lse_static, ref[i][1])
        # eager work between replays, on the same buffers the graph reads
        again = eager(qs[(i + 1) % 3])
        torch.cuda.synchronize()
        assert torch.equal(again[0], ref[(i + 1) % 3][0])


def test_graph_replays_prefill_with_tile_images(gpu):
    """A prefill chunk large enough for tile images (the pre-pass, the
    attention kernel reading images, the merge) captured and replayed."""
    stv, torch = gpu
    hq, hkv, d, L, T = 24, 4, 256, 1000, 200
    rng = np.random.default_rng(410)
    kv = stv.KVCache.from_host(synth.make_kv(rng, hkv, d, L + T))
    scale = 1.0 / math.sqrt(d)
    qs = [torch.from_numpy(synth.make_q(rng, T, hq, d)).cuda() for _ in range(3)]
    S, ws_bytes = stv.attention_plan(T, hq, hkv, d, L, True, 0, "b3")
    assert ws_bytes > stv.workspace_bytes(T, hq, d, S), "the plan uses tile images"
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    q_static = qs[0].clone()
    out_static = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
    lse_static = torch.empty((T, hq), dtype=torch.float32, device="cuda")

    def eager(q):
        lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
        o = stv.prefill_attention(q, kv, L, scale, out_lse=lse, workspace=ws)
        return o.clone(), lse.clone()

    ref = [eager(q) for q in qs]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            stv.prefill_attention(q_static, kv, L, scale, out=out_static, out_lse=lse_static,
                                  workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % 3
        q_static.copy_(qs[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static, ref[i][0]), f"replay {rep} differs from eager"
        assert torch.equal(lse_static, ref[i][1])
