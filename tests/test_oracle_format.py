"""Pins for the oracle's 3-bit block layout, fp16 rounding and quantizers.

The layout and the quantizer rules are readings (the pages fix neither);
these tests pin the oracle to hand-worked examples of those readings, to a
structural property (the layout is a bijection of 32 x 3 bits onto 96
bits), and to numpy's IEEE binary16 conversion.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line


def test_pack_golden_worked_examples(orc):
    n = 0
    for line in _golden_lines("pack_blocks.txt"):
        tok = line.split()
        if tok[0] == "single":
            e, code = int(tok[1]), int(tok[2])
            codes = [0] * 32
            codes[e] = code
        else:
            codes = [int(tok[1])] * 32
        want = np.array([int(t, 16) for t in tok[-3:]], dtype=np.uint32)
        got = orc.pack_block(codes)
        assert np.array_equal(got, want), (line, [hex(x) for x in got])
        assert list(orc.unpack_block(want)) == codes
        n += 1
    assert n == 14


def test_layout_is_a_bijection_onto_96_bits(orc):
    # Each (element, code bit) owns exactly one of the 96 bits.
    seen = {}
    for e in range(32):
        for k in range(3):
            codes = [0] * 32
            codes[e] = 1 << k
            w = orc.pack_block(codes)
            bits = [(wi, b) for wi in range(3) for b in range(32) if (int(w[wi]) >> b) & 1]
            assert len(bits) == 1
            assert bits[0] not in seen
            seen[bits[0]] = (e, k)
    assert len(seen) == 96


def test_every_code_at_every_position_round_trips(orc):
    rng = np.random.default_rng(123)
    for e in range(32):
        for v in range(8):
            codes = list(rng.integers(0, 8, size=32))
            codes[e] = v
            w = orc.pack_block(codes)
            back = orc.unpack_block(w)
            assert list(back) == codes


def test_random_words_decode_to_uniform_codes(orc):
    # 96 random bits are 32 independent uniform codes under any bijection.
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2**32, size=(400, 3), dtype=np.uint32)
    codes = np.concatenate([orc.unpack_block(w) for w in words])
    counts = np.bincount(codes, minlength=8)
    assert counts.sum() == 400 * 32
    assert np.all(np.abs(counts / counts.sum() - 1 / 8) < 0.01)


def test_f16_rounding_matches_numpy(orc):
    rng = np.random.default_rng(1)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 70000.0, 2.0**-14, 2.0**-24,
            2.0**-25, 2.0**-25 * 1.0000001, 3 * 2.0**-26, 2.0**-26, 1e-9, 0.1, 1 / 3,
            1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11, 2048.5, 2049.0, 1000.25, np.inf, -np.inf]
    vals += list(rng.uniform(-1e5, 1e5, 2000)) + list(rng.standard_normal(2000) * 1e-5)
    vals += list(np.exp(rng.uniform(-25, 12, 3000)) * rng.choice([-1, 1], 3000))
    for v in vals:
        f = np.float32(v)
        want = int(np.array([f], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
        got = orc.f32_to_f16_bits(f)
        assert got == want, (float(f), hex(got), hex(want))
        if not np.isinf(f):
            back = orc.f16_bits_to_f64(got)
            assert back == float(np.array([want], dtype=np.uint16).view(np.float16)[0])
    assert np.isnan(orc.f16_bits_to_f64(orc.f32_to_f16_bits(np.nan)))


def test_q_quantizer_worked_example(orc):
    for line in _golden_lines("quant_examples.txt"):
        tok = line.split()
        if tok[0] != "qrow":
            continue
        bar = tok.index("|")
        q = np.array([float(t) for t in tok[1:bar]], dtype=np.float32)
        want = [int(t) for t in tok[bar + 1:]]
        qi, sq = orc.quantize_q_row(q)
        assert list(qi) == want
        assert sq == np.float32(1.0) / np.float32(127.0)


def test_q_quantizer_properties(orc):
    rng = np.random.default_rng(2)
    for trial in range(300):
        d = int(rng.choice([32, 64, 256]))
        q = (rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        qi, sq = orc.quantize_q_row(q)
        amax = np.max(np.abs(q))
        assert np.max(np.abs(qi.astype(np.int64))) == 127
        assert qi[np.argmax(np.abs(q))] == (127 if q[np.argmax(np.abs(q))] > 0 else -127)
        assert np.all(np.sign(qi) * np.sign(q) >= 0)
        assert abs(float(sq) - float(amax) / 127.0) <= float(amax) / 127.0 * 2.0**-23
        err = np.abs(q.astype(np.float64) - float(sq) * qi)
        assert np.all(err <= float(sq) * (0.5 + 1e-5))
    qi, sq = orc.quantize_q_row(np.zeros(64, dtype=np.float32))
    assert sq == 0.0 and not np.any(qi)


def _kv_examples():
    for line in _golden_lines("quant_examples.txt"):
        tok = line.split("|")
        head = tok[0].split()
        if head[0] != "kvblock":
            continue
        s16 = int(head[1], 16)
        xs, cs = tok[1].strip(), tok[2].strip()
        e = np.arange(32)
        if "e" in xs:
            x = eval(xs, {"e": e}).astype(np.float32)        # noqa: S307 (fixture formula)
            c = eval(cs, {"e": e})                           # noqa: S307
        else:
            x = np.zeros(32, dtype=np.float32)
            v = [float(t) for t in xs.split()]
            x[:len(v)] = v
            c = np.full(32, 4)
            cv = [int(t) for t in cs.split()]
            c[:len(cv)] = cv
        yield s16, x, np.asarray(c)


def test_kv_quantizer_worked_examples(orc):
    n = 0
    for s16, x, codes in _kv_examples():
        w, s = orc.quantize_kv_block(x)
        assert s == s16, (hex(s), hex(s16))
        assert list(orc.unpack_block(w)) == list(codes)
        n += 1
    assert n == 2


def test_kv_quantizer_properties(orc):
    rng = np.random.default_rng(3)
    for trial in range(500):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        w, s16 = orc.quantize_kv_block(x)
        s = orc.f16_bits_to_f64(s16)
        codes = orc.unpack_block(w)
        assert codes.min() >= 1          # symmetric rule never emits code 0
        xhat = s * (codes - 4)
        inrange = np.abs(x) <= 3.0 * s
        assert np.all(np.abs(x[inrange] - xhat[inrange]) <= s * (0.5 + 1e-6))
        # clamped elements (amax slightly above 3s after fp16 rounding) sit at +-3s
        assert np.all(np.abs(xhat[~inrange]) == 3.0 * s)
    w, s16 = orc.quantize_kv_block(np.zeros(32, dtype=np.float32))
    assert s16 == 0 and list(orc.unpack_block(w)) == [4] * 32
    w, s16 = orc.quantize_kv_block(np.full(32, 1e-9, dtype=np.float32))
    assert s16 == 0 and list(orc.unpack_block(w)) == [4] * 32
    w, s16 = orc.quantize_kv_block(np.full(32, 1e6, dtype=np.float32))
    assert s16 == 0x7BFF and list(orc.unpack_block(w)) == [7] * 32


def test_kv_quant_pack_writes_only_its_positions(orc):
    rng = np.random.default_rng(4)
    hkv, d, cap = 2, 64, 70
    nb = d // 32
    x = rng.standard_normal((5, hkv, d)).astype(np.float32)
    pos0 = 29                                   # straddles V groups 0 and 1
    # K, token-major
    codes = rng.integers(0, 2**32, size=(hkv, cap, nb, 3), dtype=np.uint32)
    scales = rng.integers(0, 2**16, size=(hkv, cap, nb), dtype=np.uint16)
    c0, s0 = codes.copy(), scales.copy()
    orc.kv_quant_pack(x, pos0, codes, scales, "k")
    keep = np.ones(cap, bool)
    keep[pos0:pos0 + 5] = False
    assert np.array_equal(codes[:, keep], c0[:, keep])
    assert np.array_equal(scales[:, keep], s0[:, keep])
    for t in range(5):
        for g in range(hkv):
            for b in range(nb):
                w, s = orc.quantize_kv_block(x[t, g, 32 * b:32 * b + 32])
                assert np.array_equal(codes[g, pos0 + t, b], w)
                assert scales[g, pos0 + t, b] == s
    # V, key-transposed: element d of key j is code j % 32 of block (j // 32, d)
    ng = (cap + 31) // 32
    vcodes = rng.integers(0, 2**32, size=(hkv, ng, d, 3), dtype=np.uint32)
    vscales = rng.integers(0, 2**16, size=(hkv, ng, nb, 32), dtype=np.uint16)
    vc0, vs0 = vcodes.copy(), vscales.copy()
    orc.kv_quant_pack(x, pos0, vcodes, vscales, "v")
    for g in range(hkv):
        for j in range(ng * 32):
            grp, e = divmod(j, 32)
            new = pos0 <= j < pos0 + 5
            for b in range(nb):
                if new:
                    w, s = orc.quantize_kv_block(x[j - pos0, g, 32 * b:32 * b + 32])
                    assert vscales[g, grp, b, e] == s
                    want = orc.unpack_block(w)
                else:
                    assert vscales[g, grp, b, e] == vs0[g, grp, b, e]
                for i in range(32):
                    got = orc.code_get(vcodes[g, grp, 32 * b + i], e)
                    ref = want[i] if new else orc.code_get(vc0[g, grp, 32 * b + i], e)
                    assert got == ref
