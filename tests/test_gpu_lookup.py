"""GPU parity of lookup drafting against the oracle (integers, bit-exact)."""
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


def _check(gpu, orc, hist, lengths, n_min, n_max, k):
    stv, torch = gpu
    r = stv.lookup_draft(torch.from_numpy(hist).cuda(),
                         torch.from_numpy(np.asarray(lengths, dtype=np.int32)).cuda(),
                         n_min, n_max, k)
    torch.cuda.synchronize()
    w = orc.lookup_draft(hist, lengths, n_min, n_max, k)
    for key in ("tokens", "count", "match", "pos"):
        assert np.array_equal(r[key].cpu().numpy(), w[key]), key


def test_short_histories_small_vocab(gpu, orc):
    rng = np.random.default_rng(61)
    for trial in range(40):
        B = int(rng.integers(1, 50))
        stride = int(rng.integers(1, 5000))
        hist = rng.integers(0, int(rng.integers(1, 4)), size=(B, stride)).astype(np.int32)
        lengths = rng.integers(-2, stride + 3, size=B).astype(np.int32)
        n_min = int(rng.integers(1, 9))
        n_max = int(rng.integers(n_min, 65))
        k = int(rng.integers(0, 20))
        _check(gpu, orc, hist, lengths, n_min, n_max, k)


def test_long_histories_with_planted_copies(gpu, orc):
    rng = np.random.default_rng(62)
    B, stride = 4, 262144
    hist = np.stack([synth.make_lookup_history(rng, stride, 151936, c) for c in (12, 9, 5, 0)])
    lengths = np.array([stride, stride, stride - 1000, stride], dtype=np.int32)
    _check(gpu, orc, hist, lengths, 6, 12, 8)


def test_chunk_boundaries(gpu, orc):
    """Matches that straddle the 4,096-position chunks of the scan."""
    rng = np.random.default_rng(63)
    for stride in (4095, 4096, 4097, 8193, 12289):
        for shift in (0, 1, 5, 11):
            h = rng.integers(0, 1000, size=stride).astype(np.int32)
            e = min(4095 + shift, stride - 20)
            h[stride - 12:] = h[e - 11:e + 1]
            _check(gpu, orc, h[None], [stride], 6, 12, 8)
