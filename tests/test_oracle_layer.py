"""Pins of the oracle's layer and route planner: numpy float64 brute force on small
shapes, the invariants the pages state, and a numpy stable sort for routing."""
import dataclasses

import numpy as np
import pytest

import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

import bruteforce as BF


def _small(fmt, E=4, K=64, N=32, topk=2, T=5, limit=None, seed=1, hybrid=0):
    cfg = I.Config("small", T=T, E=E, K=K, N=N, topk=topk, limit=limit, fmt=fmt, hybrid_nvfp4=hybrid)
    return I.make_problem(cfg, seed=seed)


CASES = {
    "tiny_mxfp4": lambda: I.make_problem("tiny"),
    "mxfp4_k3": lambda: _small(I.FMT_MXFP4, E=5, K=128, N=64, topk=3, T=6, limit=7.0, seed=2),
    "nvfp4": lambda: _small(I.FMT_NVFP4, E=4, K=64, N=32, topk=2, T=5, seed=3),
    "nf3": lambda: _small(I.FMT_NF3, E=3, K=64, N=64, topk=3, T=4, seed=4),
    "hybrid": lambda: _small(I.FMT_NVFP4, E=6, K=64, N=32, topk=3, T=5, seed=5, hybrid=2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_oracle_matches_float64_bruteforce(name):
    p = CASES[name]()
    acc, out = O.moe_problem(p)
    ref = BF.moe(p)
    assert np.allclose(acc, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    # out is acc rounded to bf16
    back = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(back - acc) <= np.abs(acc) * 2.0 ** -8 + 1e-30)


def test_gate_up_stacking_flag():
    p = CASES["mxfp4_k3"]()
    acc, _ = O.moe_problem(p, gate_up=True)
    assert np.allclose(acc, BF.moe(p, gate_up=True), rtol=1e-9, atol=1e-9)
    acc0, _ = O.moe_problem(p, gate_up=False)
    assert not np.allclose(acc, acc0)  # the stacking order matters


def test_duplicate_ids_in_a_row_count_twice():
    p = CASES["nvfp4"]()
    p.ids[:, :] = p.ids[:, :1]  # every slot of a row routes to the same expert
    acc, _ = O.moe_problem(p)
    assert np.allclose(acc, BF.moe(p), rtol=1e-9, atol=1e-9)


def test_k1_weight1_is_single_expert_mlp():
    p = CASES["mxfp4_k3"]()
    c = dataclasses.replace(p.cfg, topk=1)
    ids = np.array([[3], [0], [4], [1], [2], [3]], np.int32)
    w = np.ones((6, 1), np.float32)
    q = I.Problem(c, p.x, ids, w, p.tiers)
    acc, _ = O.moe_problem(q)
    t = p.tiers[0]
    for r in range(6):
        y = BF.expert_mlp(t.fmt, t.weights, int(ids[r, 0]), p.x[r], c.K, c.N, c.limit)
        assert np.allclose(acc[r], y, rtol=1e-10, atol=1e-10 * np.abs(y).max())


@pytest.mark.parametrize("name", ["tiny_mxfp4", "nf3", "hybrid"])
def test_zero_weight_and_invalid_slots_change_nothing(name):
    p = CASES[name]()
    E = p.cfg.E
    acc0, out0 = O.moe_problem(p)
    # 1) a slot with weight 0 is bit-identical to the same slot marked -1
    q = I.Problem(p.cfg, p.x, p.ids.copy(), p.wts.copy(), p.tiers)
    q.wts[:, -1] = 0.0
    r = I.Problem(p.cfg, p.x, p.ids.copy(), p.wts.copy(), p.tiers)
    r.ids[:, -1] = -1
    a1, _ = O.moe_problem(q)
    a2, _ = O.moe_problem(r)
    assert np.array_equal(a1, a2)
    # 2) every out-of-range id behaves like -1
    for bad in (E, E + 7, -5, np.iinfo(np.int32).min, np.iinfo(np.int32).max):
        s = I.Problem(p.cfg, p.x, r.ids.copy(), p.wts.copy(), p.tiers)
        s.ids[:, -1] = bad
        a3, _ = O.moe_problem(s)
        assert np.array_equal(a3, a2)
    # 3) rows with no valid slot are exactly zero
    z = I.Problem(p.cfg, p.x, p.ids.copy(), p.wts.copy(), p.tiers)
    z.ids[1, :] = -1
    a4, o4 = O.moe_problem(z)
    assert np.all(a4[1] == 0) and np.all(o4[1] == 0)
    assert np.array_equal(a4[0], acc0[0])


def test_linear_in_router_weights_and_slot_order():
    p = CASES["mxfp4_k3"]()
    acc, _ = O.moe_problem(p)
    q = I.Problem(p.cfg, p.x, p.ids, p.wts * 2.0, p.tiers)
    acc2, _ = O.moe_problem(q)
    assert np.array_equal(acc2, 2.0 * acc)  # power-of-two scaling is exact
    perm = np.array([2, 0, 1])
    r = I.Problem(p.cfg, p.x, np.ascontiguousarray(p.ids[:, perm]), np.ascontiguousarray(p.wts[:, perm]), p.tiers)
    acc3, _ = O.moe_problem(r)
    assert np.allclose(acc3, acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())


def test_hybrid_is_sum_of_tiers():
    p = CASES["hybrid"]()
    acc, _ = O.moe_problem(p)
    parts = []
    for t in p.tiers:
        q = I.Problem(p.cfg, p.x, p.ids, p.wts, [t])
        parts.append(O.moe_problem(q)[0])
    assert np.allclose(acc, parts[0] + parts[1], rtol=1e-12, atol=1e-12 * np.abs(acc).max())
    assert np.abs(parts[0]).max() > 0 and np.abs(parts[1]).max() > 0


def _np_route(ids, E_global, tiers):
    flat = ids.ravel()
    U = sum(t.E for t in tiers)
    u = np.full(flat.shape, -1, np.int64)
    base = 0
    for t in tiers:
        ok = (flat >= 0) & (flat < E_global)
        loc = np.full(flat.shape, -1, np.int64)
        if t.emap is None:
            loc[ok] = flat[ok]
        else:
            loc[ok] = t.emap[flat[ok]]
        take = (u < 0) & (loc >= 0) & (loc < t.E)
        u[take] = base + loc[take]
        base += t.E
    valid = np.flatnonzero(u >= 0)
    perm = valid[np.argsort(u[valid], kind="stable")]
    cnt = np.bincount(u[valid], minlength=U)
    inv = np.full(flat.shape, -1, np.int64)
    inv[perm] = np.arange(len(perm))
    return cnt, np.concatenate([[0], np.cumsum(cnt)]), perm, inv


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_vs_numpy_stable_sort(seed):
    rng = np.random.default_rng(seed)
    E = 37
    ids = rng.integers(-3, E + 3, size=(50, 6)).astype(np.int32)
    ids[4] = -1
    tiers = [I.Tier(I.FMT_MXFP4, E, {})]
    got = O.route(ids, E, tiers)
    want = _np_route(ids, E, tiers)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)
    # two tiers through expert maps
    ea, eb = I.make_tier_split(E, 10, seed)
    tiers2 = [I.Tier(I.FMT_NVFP4, 10, {}, ea), I.Tier(I.FMT_NF3, E - 10, {}, eb)]
    got = O.route(ids, E, tiers2)
    want = _np_route(ids, E, tiers2)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_quantised_layer_envelope_vs_unquantised():
    """W4A8 against the same weights with exact activations: a few percent rel-L2, as the
    sglang adapter reports for its W4A8 path against an fp32 reference (4.67 %)."""
    p = I.make_problem(dataclasses.replace(I.CONFIGS["decode"], T=3, pad_rows=0))
    acc, _ = O.moe_problem(p)
    t = p.tiers[0]
    c = p.cfg
    rel = []
    for r in range(3):
        ref = np.zeros(c.K)
        for j in range(c.topk):
            e = int(p.ids[r, j])
            W13 = BF.dequant(t.fmt, t.weights["w13"][e], t.weights["s13"][e])
            W2 = BF.dequant(t.fmt, t.weights["w2"][e], t.weights["s2"][e])
            x = (p.x[r].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            z = W13 @ x
            up, gate = np.clip(z[:c.N], -c.limit, c.limit), np.minimum(z[c.N:], c.limit)
            ref += float(p.wts[r, j]) * (W2 @ (gate / (1 + np.exp(-gate)) * up))
        rel.append(np.linalg.norm(acc[r] - ref) / np.linalg.norm(ref))
    assert 0.005 < np.mean(rel) < 0.10, rel


# Router weight on the input (vLLM "fused_moe/b12x" page, apply_router_weight_on_input,
# 16-bit activation formats only): out[t] = sum_j W2 act(W13 (w_j x_t)).
@pytest.mark.parametrize("name", ["nvfp4", "nf3", "hybrid"])
def test_weight_on_input_matches_float64_bruteforce(name):
    p = CASES[name]()
    acc, _ = O.moe_problem(p, weight_on_input=True)
    ref = BF.moe(p, weight_on_input=True)
    assert np.allclose(acc, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    assert not np.allclose(acc, O.moe_problem(p)[0])   # the activation is not linear: it matters where w goes


def test_weight_on_input_is_per_slot_scaled_input():
    """With power-of-two router weights the scaled bf16 input is exact, so the layer equals
    the sum over slots of one-slot layers with weight 1 run on w_j * x."""
    p = CASES["nf3"]()
    T, k = p.ids.shape
    rng = np.random.default_rng(7)
    p.wts[:] = 2.0 ** rng.integers(-3, 3, size=(T, k))
    acc, _ = O.moe_problem(p, weight_on_input=True)
    xf = (p.x.astype(np.uint32) << 16).view(np.float32)
    total = np.zeros_like(acc)
    for j in range(k):
        xj = (xf * p.wts[:, j:j + 1]).astype(np.float32)
        xb = (xj.view(np.uint32) >> 16).astype(np.uint16)   # exact: power-of-two scaling of bf16 values
        assert np.array_equal((xb.astype(np.uint32) << 16).view(np.float32), xj)
        q = I.Problem(dataclasses.replace(p.cfg, topk=1), xb, p.ids[:, j:j + 1].copy(),
                      np.ones((T, 1), np.float32), p.tiers)
        total += O.moe_problem(q)[0]
    assert np.allclose(acc, total, rtol=1e-12, atol=1e-12 * np.abs(total).max())


def test_weight_on_input_refused_for_mxfp8_activations():
    with pytest.raises(ValueError):
        O.moe_problem(CASES["mxfp4_k3"](), weight_on_input=True)


# SwiGLU-OAI (vLLM "fused_moe/b12x" page, _swiglu_params: limit, alpha and beta for the
# swigluoai activation; refused with W4A8).  The formula is not printed there; the oracle
# takes h = gate * sigmoid(alpha gate) * (up + beta) after the clamps.
OAI_CASES = {
    "nvfp4": lambda: _small(I.FMT_NVFP4, E=4, K=64, N=32, topk=2, T=5, limit=7.0, seed=13),
    "nf3": lambda: _small(I.FMT_NF3, E=3, K=64, N=64, topk=3, T=4, limit=7.0, seed=14),
    "hybrid": lambda: _small(I.FMT_NVFP4, E=6, K=64, N=32, topk=3, T=5, limit=7.0, seed=15, hybrid=2),
}


def test_swiglu_oai_alpha1_beta0_is_swiglu():
    p = OAI_CASES["nf3"]()
    a0, o0 = O.moe_problem(p)
    a1, o1 = O.moe_problem(p, alpha=1.0, beta=0.0)
    assert np.array_equal(a0, a1) and np.array_equal(o0, o1)


@pytest.mark.parametrize("name", list(OAI_CASES))
def test_swiglu_oai_matches_float64_bruteforce(name):
    alpha, beta = 1.702, 1.0
    p = OAI_CASES[name]()
    acc, _ = O.moe_problem(p, alpha=alpha, beta=beta)
    ref = BF.moe(p, act=lambda g, u: g * (1.0 / (1.0 + np.exp(-alpha * g))) * (u + beta))
    assert np.allclose(acc, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    assert not np.allclose(acc, O.moe_problem(p)[0], rtol=1e-3)
    # each parameter on its own moves the result
    assert not np.allclose(acc, O.moe_problem(p, alpha=alpha)[0], rtol=1e-3)
    assert not np.allclose(acc, O.moe_problem(p, beta=beta)[0], rtol=1e-3)


def test_swiglu_oai_large_alpha_is_relu_gate():
    """alpha -> inf turns the sigmoid into a step: h = relu(gate) (up + beta)."""
    p = OAI_CASES["nvfp4"]()
    acc, _ = O.moe_problem(p, alpha=1e4, beta=0.5)
    ref = BF.moe(p, act=lambda g, u: np.maximum(g, 0.0) * (u + 0.5))
    assert np.allclose(acc, ref, rtol=0, atol=2e-3 * np.abs(ref).max())
    silu = BF.moe(p, act=lambda g, u: g / (1.0 + np.exp(-g)) * (u + 0.5))
    assert not np.allclose(silu, ref, rtol=0, atol=2e-2 * np.abs(ref).max())


def test_swiglu_oai_refused_for_mxfp8_activations():
    with pytest.raises(ValueError):
        O.moe_problem(CASES["mxfp4_k3"](), alpha=1.702, beta=1.0)
