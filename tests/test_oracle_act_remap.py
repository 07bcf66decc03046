"""Pins of the oracle's activation step and of its EP id remap (CPU only).

The activation values are hand-worked (tests/golden/formats.json) and are run
through the scalar the oracle's layer itself calls (orc_act), and through a
whole one-expert layer whose one-hot weights copy each (gate, up) pair into the
GEMM1 results and each h into the output, so a mistake in either the scalar or
in how the layer wires it fails here. A planted mistake in the oracle's source
(compiled here on the CPU) must fail the same values.
"""
import ctypes as C
import json
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "formats.json")))
REMAP = json.load(open(os.path.join(HERE, "golden", "ep_remap.json")))


def test_swiglu_limit_hand_values():
    for gate, up, h in GOLD["swiglu_limit7"]["cases"]:
        assert O.act(O.ACT_SWIGLU, gate, up, 7.0) == pytest.approx(h, rel=1e-7, abs=1e-12), (gate, up)


def test_swiglu_without_limit_is_silu_times_up():
    # no clamp: (10, -10) gives silu(10) * -10, not the clamped -48.96
    s10 = 10.0 / (1.0 + math.exp(-10.0))
    assert O.act(O.ACT_SWIGLU, 10.0, -10.0, None) == pytest.approx(-10.0 * s10, rel=1e-12)


def test_situ_hand_values_and_limits():
    for gate, up, h in GOLD["situ"]["cases"]:
        assert O.act(O.ACT_SITU, gate, up) == pytest.approx(h, rel=1e-7, abs=1e-12), (gate, up)
    # small arguments: tanh(x / b) * b = x (1 + O(x^2)), so SiTU meets the unclamped SwiGLU
    for gate, up in ((1e-3, 2e-3), (-5e-4, 1e-3), (2e-3, -1e-3)):
        plain = O.act(O.ACT_SWIGLU, gate, up, None)
        assert O.act(O.ACT_SITU, gate, up) == pytest.approx(plain, rel=1e-5)
    # odd in up; bounded by the caps
    for gate, up in ((1.5, 3.0), (-2.0, 40.0), (9.0, -0.25)):
        assert O.act(O.ACT_SITU, gate, -up) == -O.act(O.ACT_SITU, gate, up)
        assert abs(O.act(O.ACT_SITU, gate, up)) < 4.0 * 25.0


def test_relu2_hand_values():
    for z, h in GOLD["relu2_no_mul"]["cases"]:
        assert O.act(O.ACT_RELU2_NO_MUL, 123.0, z) == h


def _onehot_layer(pairs, act_kind, limit):
    """One NVFP4 expert, K = 256, N = 32, top-1 with weight 1: w13 up row n reads x[n],
    gate row n reads x[N + n] (E2M1 code 2 = 1.0, scale E4M3 0x38 = 1.0, global 1),
    w2 row c reads h[c].  Returns (x, acc) with acc[c] = bf16(h[c]) for the pairs."""
    K, N = 256, 32
    xs = np.zeros(K, np.float32)
    for n, (gate, up) in enumerate(pairs):
        xs[n], xs[N + n] = up, gate
    w13_rows = N if act_kind == O.ACT_RELU2_NO_MUL else 2 * N
    w13 = np.zeros((1, w13_rows, K // 2), np.uint8)
    for r in range(w13_rows):
        col = r   # up row n -> column n; gate row n (row N + n) -> column N + n
        w13[0, r, col // 2] = 2 if col % 2 == 0 else 0x20
    s13 = np.full((1, w13_rows, K // 16), 0x38, np.uint8)
    w2 = np.zeros((1, K, N // 2), np.uint8)
    for c in range(N):
        w2[0, c, c // 2] = 2 if c % 2 == 0 else 0x20
    s2 = np.full((1, K, N // 16), 0x38, np.uint8)
    g = np.ones(1, np.float32)
    tier = I.Tier(I.FMT_NVFP4, 1, {"w13": w13, "s13": s13, "g13": g, "w2": w2, "s2": s2, "g2": g}, None)
    x = I.bf16_bits_from_f32(xs[None, :])
    acc, _ = O.moe(1, K, N, 1, limit, [tier], x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                   act_kind=act_kind)
    return acc[0]


def _bf16(v):
    return O.bf16_to_float(O.bf16_from_float(v))


@pytest.mark.parametrize("kind,key,limit", [(O.ACT_SWIGLU, "swiglu_limit7", 7.0), (O.ACT_SITU, "situ", None)])
def test_layer_routes_gate_and_up_through_the_activation(kind, key, limit):
    cases = [c for c in GOLD[key]["cases"] if abs(c[0]) < 1e5 and abs(c[1]) < 1e5]   # bf16-exact inputs
    if kind == O.ACT_SITU:
        cases += [[60.0, 1000.0, GOLD["situ"]["cases"][0][2] * math.tanh(40.0) * math.tanh(15.0)]]
    acc = _onehot_layer([(g, u) for g, u, _ in cases], kind, limit)
    for n, (_, _, h) in enumerate(cases):
        assert acc[n] == pytest.approx(_bf16(h), rel=2 ** -8, abs=1e-30), (n, cases[n])
    assert np.all(acc[len(cases):] == 0.0)


def test_layer_relu2_reads_n_rows():
    cases = GOLD["relu2_no_mul"]["cases"]
    acc = _onehot_layer([(0.0, z) for z, _ in cases], O.ACT_RELU2_NO_MUL, None)
    for n, (_, h) in enumerate(cases):
        assert acc[n] == h


def test_activation_variants_refused_where_the_page_refuses_them():
    t = I.make_problem("tiny")
    c = t.cfg
    with pytest.raises(ValueError):   # ReLU^2 without the multiply: not with W4A8
        O.moe(c.E, c.K, c.N, c.topk, None, t.tiers, t.x, t.ids, t.wts, act_kind=O.ACT_RELU2_NO_MUL)
    with pytest.raises(ValueError):   # SiTU takes no limit
        O.moe(c.E, c.K, c.N, c.topk, 7.0, t.tiers, t.x, t.ids, t.wts, act_kind=O.ACT_SITU)
    O.moe(c.E, c.K, c.N, c.topk, None, t.tiers, t.x, t.ids, t.wts, act_kind=O.ACT_SITU)   # SiTU runs with W4A8


# Each replacement plants a plausible mistake in the oracle's activation; the golden values must catch it.
PLANTED = [
    ("if (gate > limit) gate = limit;", "if (gate < -limit) gate = -limit;"),      # clamp on the wrong side
    ("if (up < -limit) up = -limit;", ""),                                          # up not clamped from below
    ("if (gate > limit) gate = limit;", "if (gate > limit) gate = limit; if (gate < -limit) gate = -limit;"),
    ("return gate / (1.0 + exp(-alpha * gate)) * (up + beta);",
     "{ double h = gate / (1.0 + exp(-alpha * gate)) * (up + beta); if (!isnan(limit)) { if (h > limit) h = limit; "
     "if (h < -limit) h = -limit; } return h; }"),                                  # clamp on h
    ("double g = 4.0 * tanh(gate / 4.0), u = 25.0 * tanh(up / 25.0);",
     "double g = 4.0 * tanh(gate / 4.0), u = up;"),                                 # linear branch uncapped
    ("double g = 4.0 * tanh(gate / 4.0), u = 25.0 * tanh(up / 25.0);",
     "double g = 25.0 * tanh(gate / 25.0), u = 4.0 * tanh(up / 4.0);"),             # caps swapped
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("i", range(len(PLANTED)))
def test_planted_activation_mistakes_fail_the_golden_values(i):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "moe_oracle.c")).read()
    old, new = PLANTED[i]
    assert old in src
    with tempfile.TemporaryDirectory() as d:
        c_path, so_path = os.path.join(d, "m.c"), os.path.join(d, "m.so")
        open(c_path, "w").write(src.replace(old, new, 1))
        subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", c_path, "-o", so_path, "-lm"], check=True)
        L = C.CDLL(so_path)
        L.orc_act.restype = C.c_double
        L.orc_act.argtypes = [C.c_int, C.c_double, C.c_double, C.c_double, C.c_double, C.c_double]
        wrong = 0
        for key, kind, lim in (("swiglu_limit7", 0, 7.0), ("situ", 1, math.nan)):
            for gate, up, h in GOLD[key]["cases"]:
                got = L.orc_act(kind, gate, up, lim, 1.0, 0.0)
                wrong += not math.isclose(got, h, rel_tol=1e-7, abs_tol=1e-12)
        assert wrong > 0, f"planted mistake {i} passed the golden values"


@pytest.mark.parametrize("case", range(len(REMAP["cases"])))
def test_ep_remap_hand_worked(case):
    c = REMAP["cases"][case]
    ids, w = O.ep_remap(np.array(c["ids"], np.int32), np.array(c["w"], np.float32), c["offset"], c["num_local"])
    assert ids.tolist() == c["out_ids"]
    assert w.tolist() == c["out_w"]


def test_ep_remap_invariants():
    rng = np.random.default_rng(5)
    for trial in range(20):
        T, k = int(rng.integers(1, 40)), int(rng.integers(1, 9))
        num_local, offset = int(rng.integers(1, 64)), int(rng.integers(0, 200))
        ids = rng.integers(-1, offset + 2 * num_local, size=(T, k)).astype(np.int32)
        w = rng.random((T, k)).astype(np.float32)
        oi, ow = O.ep_remap(ids, w, offset, num_local)
        lid = ids.astype(np.int64) - offset
        ok = (lid >= 0) & (lid < num_local)
        assert np.array_equal(oi[ok], lid[ok]) and np.array_equal(ow[ok], w[ok])
        assert np.all(ow[~ok] == 0.0)
        assert np.all((oi >= 0) & (oi < num_local))
        if ok.any():
            # every slot names an expert some valid slot of the batch already reads
            assert set(oi.ravel().tolist()) <= set(lid[ok].ravel().tolist())
