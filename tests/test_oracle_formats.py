"""Pins of the oracle's format decoders and encoders against values fixed outside
the oracle: the pages' printed formulas and codebook, hand-worked values, torch's
float8_e4m3fn conversion (a library routine) and brute-force nearest-code search."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formats.json")))


def test_e2m1_table():
    want = GOLD["e2m1_table"]["codes_0_to_15"]
    got = [O.e2m1(c) for c in range(16)]
    assert got == want
    assert [math.copysign(1, g) for g in got] == [math.copysign(1, w) for w in want]


def test_e8m0_pairs_and_all_bytes():
    for b, v in GOLD["e8m0"]["pairs"]:
        assert O.e8m0(b) == v
    # every finite byte is a power of two, strictly increasing by one binade per step
    vals = [O.e8m0(b) for b in range(255)]
    assert all(vals[i + 1] == 2 * vals[i] for i in range(254))
    assert math.isnan(O.e8m0(255))


def test_e4m3_all_bytes_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    for byte, v in GOLD["e4m3"]["pairs"]:
        assert O.e4m3(byte) == v


def _e4m3_values():
    return np.array([O.e4m3(c) for c in range(127)])  # codes 0..126 (0x7F is NaN)


def _brute_e4m3(v):
    """Nearest E4M3 code by exhaustive search (ties to the even code), saturating."""
    vals = _e4m3_values()
    a = min(abs(v), 448.0)
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if len(best) == 1 else int([x for x in best if x % 2 == 0][0])
    return c | (0x80 if math.copysign(1, v) < 0 else 0)


def test_e4m3_encode_vs_torch_in_range_and_ties():
    rng = np.random.default_rng(7)
    vals = _e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties between neighbours
    xs = np.concatenate([rng.uniform(-448, 448, 2000), rng.uniform(-1, 1, 2000),
                         rng.uniform(-0.02, 0.02, 2000), mids, -mids, vals, -vals])
    xs = xs.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(xs.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(x) for x in xs], dtype=np.uint8)
    # -0.0 and +0.0 are both zero; compare values, then codes where nonzero
    assert np.array_equal(got & 0x7F, ref & 0x7F)
    nz = (ref & 0x7F) != 0
    assert np.array_equal(got[nz], ref[nz])


def test_e4m3_encode_saturates_and_brute_force():
    for v in [448.0, 449.0, 464.0, 480.0, 511.9, 1e6, -500.0]:
        assert O.e4m3_encode(v) == _brute_e4m3(v)
        assert O.e4m3_encode(v) & 0x7F == 0x7E
    rng = np.random.default_rng(3)
    for v in rng.uniform(-520, 520, 300):
        assert O.e4m3_encode(v) == _brute_e4m3(v)


def test_mxfp8_hand_blocks():
    for case in GOLD["mxfp8_blocks"]["cases"]:
        blk = np.zeros((1, 32), np.float32)
        for i, v in case["values"].items():
            blk[0, int(i)] = v
        q, s = O.mxfp8_quantize_f32(blk)
        assert s[0, 0] == case["scale_byte"]
        for i, c in case["codes"].items():
            assert q[0, int(i)] == c
        # untouched zeros stay zero codes
        others = [i for i in range(32) if str(i) not in case["values"]]
        assert all(q[0, i] & 0x7F == 0 for i in others)


def test_mxfp8_block_properties():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal((64, 32)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    v[0] = 0.0
    q, s = O.mxfp8_quantize_f32(v)
    vals = _e4m3_values()
    for r in range(64):
        E = int(s[r, 0]) - 127
        amax = float(np.abs(v[r].astype(np.float64)).max())
        if amax == 0:
            assert E == -127 and np.all(q[r] & 0x7F == 0)
            continue
        # the block maximum lands in E4M3's top binade [256, 512) after scaling
        assert 256.0 <= amax * 2.0 ** -E < 512.0
        for i in range(32):
            assert q[r, i] == _brute_e4m3(float(v[r, i]) * 2.0 ** -E)
        # idempotence: re-quantising the dequantised block reproduces it
        deq = np.array([O.e4m3(c) for c in q[r]]) * 2.0 ** E
        q2, s2 = O.mxfp8_quantize_f32(deq[None, :].astype(np.float32))
        if np.abs(deq).max() > 0 and amax * 2.0 ** -E < 448:
            assert s2[0, 0] == s[r, 0] and np.array_equal(q2[0], q[r])


def test_mxfp8_bf16_matches_f32_path():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    from block_scaled_fp4_histogram_amd.inputs import bf16_bits_from_f32
    xb = bf16_bits_from_f32(x)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    q1, s1 = O.mxfp8_quantize_bf16(xb)
    q2, s2 = O.mxfp8_quantize_f32(xf)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_mxfp4_row_hand_value():
    g = GOLD["mxfp4_row"]
    w = np.zeros((1, 16), np.uint8)
    w[0, 0] = g["byte"]
    s = np.full((1, 1), g["scale_byte"], np.uint8)
    row = O.dequant(O.FMT_MXFP4, w, s, 32)
    assert list(row[0, :2]) == g["first_two_values"]
    assert np.all(row[0, 2:] == 0)


def test_nvfp4_row():
    # E2M1 x E4M3(per 16) x global; scale bytes 0x38 (1.0) and 0x40 (2.0), global 0.75
    w = np.array([[0x21] * 16], np.uint8)  # codes 1 (0.5) low, 2 (1.0) high
    s = np.array([[0x38, 0x40]], np.uint8)
    row = O.dequant(O.FMT_NVFP4, w, s, 32, g=0.75)
    assert list(row[0, :2]) == [0.375, 0.75]
    assert list(row[0, 16:18]) == [0.75, 1.5]


def test_nf3_codebook_and_packing():
    g = GOLD["nf3"]
    assert [O.nf3(c) for c in range(8)] == [float(np.float32(v)) for v in g["codebook"]]
    for pk in g["packs"]:
        w = np.zeros((1, 12), np.uint8)
        w[0, :3] = pk["bytes"]
        s = np.array([[0x38]], np.uint8)  # 1.0
        row = O.dequant(O.FMT_NF3, w, s, 32)
        want = [float(np.float32(g["codebook"][c])) for c in pk["codes"]]
        assert list(row[0, :8]) == want


def test_bf16_rounding():
    assert O.bf16_from_float(1.0) == 0x3F80
    assert O.bf16_from_float(1.0 + 2 ** -8) == 0x3F80          # tie -> even
    assert O.bf16_from_float(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert O.bf16_from_float(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert O.bf16_from_float(-2.5) == 0xC020
    rng = np.random.default_rng(1)
    xs = rng.standard_normal(2000).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([O.bf16_from_float(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)
