"""Bit-exact GPU stages against the oracle: MXFP8 quantiser, route planner and the
weight repacker's round trip. All calls go through the C ABI."""
import dataclasses

import numpy as np
import pytest
import torch

import block_scaled_fp4_histogram_amd as M
import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import DeviceLayer, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(8, 7168), (5, 256), (1, 32), (37, 6144)])
def test_quant_bf16_bitexact(rows, cols):
    x = I.make_x(rows, cols, seed=rows)
    q, s = M.debug_quant_mxfp8(dev(x, torch.bfloat16))
    torch.cuda.synchronize()
    qo, so = O.mxfp8_quantize_bf16(x)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy(), so)


def _hard_f32(rows, cols, seed):
    """fp32 values across many binades, with exact E4M3 ties, saturating blocks and zeros."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-30, 30, (rows, 1)))).astype(np.float32)
    vals = np.array([O.e4m3(c) for c in range(127)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    for r in range(0, rows, 3):   # a block whose amax is 448 * 2^E plus exact midpoints
        E = int(rng.integers(-20, 20))
        blk = rng.choice(mids, 32).astype(np.float64) * np.sign(rng.standard_normal(32))
        blk[0] = 448.0
        v[r, :32] = (blk * 2.0 ** E).astype(np.float32)
    v[1 % rows, 32:64] = 0.0
    if rows > 2:
        v[2, :32] = np.float32(460.0) * np.exp2(np.float32(-3))  # amax 57.5: block saturates (57.5*2^3=460)
    return v


def test_quant_bf16_hard_and_full_size():
    """The bf16 quantiser (the one every bf16-activation path runs, decode included) on blocks
    with exact E4M3 ties, saturating blocks, zeros and many binades, then on the prefill
    workload's whole activation matrix (4096 x 7168)."""
    hard = torch.from_numpy(_hard_f32(48, 512, seed=7)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x in (hard, I.make_x(4096, 7168, seed=0)):
        q, s = M.debug_quant_mxfp8(dev(x, torch.bfloat16))
        torch.cuda.synchronize()
        qo, so = O.mxfp8_quantize_bf16(x)
        assert np.array_equal(s.cpu().numpy(), so)
        assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("rows,cols", [(16, 576), (64, 512), (3, 96)])
def test_quant_f32_bitexact(rows, cols):
    v = _hard_f32(rows, cols, seed=cols)
    q, s = M.debug_quant_mxfp8(dev(v))
    torch.cuda.synchronize()
    qo, so = O.mxfp8_quantize_f32(v)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


def _route_case(name):
    if name == "decode":
        return I.make_problem("decode")
    if name == "prefill":   # 24,576 routes: the multi-block planner, Zipf loads
        cfg = I.CONFIGS["prefill"]
        ids, wts = I.make_routing(cfg.T, cfg.E, cfg.topk, 0, cfg.zipf_s)
        return I.Problem(cfg, None, ids, wts, [I.Tier(cfg.fmt, cfg.E, {})])
    if name == "hybrid":
        cfg = I.CONFIGS["hybrid"]
        ids, wts = I.make_routing(cfg.T, cfg.E, cfg.topk, 0)
        ea, eb = I.make_tier_split(cfg.E, 64, 0)
        return I.Problem(cfg, None, ids, wts, [I.Tier(I.FMT_NVFP4, 64, {}, ea), I.Tier(I.FMT_NF3, 192, {}, eb)])
    if name == "invalid_ids":   # ragged T, ids outside [0,E) of every kind
        rng = np.random.default_rng(9)
        E = 40
        ids = rng.integers(-2, E + 2, size=(333, 5)).astype(np.int32)
        ids[::7, 2] = np.iinfo(np.int32).min
        ids[::11, 4] = np.iinfo(np.int32).max
        ids[5] = -1
        cfg = I.Config("inv", T=333, E=E, K=256, N=64, topk=5, limit=None, fmt=I.FMT_MXFP4)
        return I.Problem(cfg, None, ids, None, [I.Tier(I.FMT_MXFP4, E, {})])
    if name == "single_block":   # 1,020 routes: one planner block, its last wave ragged
        cfg = I.Config("single", T=170, E=384, K=256, N=64, topk=6, limit=None, fmt=I.FMT_MXFP4)
        ids, wts = I.make_routing(cfg.T, cfg.E, cfg.topk, 3, 1.1)
        return I.Problem(cfg, None, ids, wts, [I.Tier(cfg.fmt, cfg.E, {})])
    raise KeyError(name)


@pytest.mark.parametrize("name", ["decode", "single_block", "prefill", "hybrid", "invalid_ids"])
def test_route_bitexact(name):
    prob = _route_case(name)
    c = prob.cfg
    fmt = prob.tiers[0].fmt
    # the planner depends on E, top_k and the tier sizes only; small K and N keep the weights tiny
    plan = M.Plan(c.E, 256, 64, c.topk, None, M.A_MXFP8 if fmt == I.FMT_MXFP4 else M.A_BF16, max_tokens=c.T)
    small = [I.Tier(t.fmt, t.E, I.make_weights(t.fmt, t.E, 256, 64), t.emap) for t in prob.tiers]
    keep, tiers = [], []
    for t in small:
        w = t.weights
        ts = [dev(w[k]) for k in ("w13", "s13", "w2", "s2")]
        g13 = None if w["g13"] is None else dev(w["g13"])
        g2 = None if w["g2"] is None else dev(w["g2"])
        ex = M.Experts(plan, t.fmt, t.E, *ts, g13, g2)
        emap = None if t.emap is None else dev(t.emap)
        keep += ts + [g13, g2, emap]
        tiers.append((ex, emap))
    cnt, off, perm, inv = M.debug_route(plan, tiers, dev(prob.ids))
    ocnt, ooff, operm, oinv = O.route(prob.ids, c.E, small)
    assert np.array_equal(cnt.cpu().numpy(), ocnt)
    assert np.array_equal(off.cpu().numpy(), ooff)
    assert np.array_equal(perm.cpu().numpy(), operm)
    assert np.array_equal(inv.cpu().numpy(), oinv)


@pytest.mark.parametrize("fmt,gate_up", [(I.FMT_MXFP4, False), (I.FMT_MXFP4, True), (I.FMT_NVFP4, False),
                                         (I.FMT_NF3, False)])
# (E, K, N); N = 896 / 1344: MXFP4 w2 scales with a tail of whole k-tiles after the runs of four
@pytest.mark.parametrize("geom", [(8, 256, 128), (3, 512, 96), (2, 7168, 576), (2, 256, 896), (2, 256, 1344)])
def test_repack_roundtrip_bitexact(fmt, gate_up, geom):
    E, K, N = geom
    w = I.make_weights(fmt, E, K, N, seed=E + K)
    plan = M.Plan(E, K, N, 2, None, M.A_MXFP8 if fmt == I.FMT_MXFP4 else M.A_BF16,
                  M.W13_GATE_UP if gate_up else M.W13_UP_GATE, 16)
    ts = [dev(w[k]) for k in ("w13", "s13", "w2", "s2")]
    g13 = None if w["g13"] is None else dev(w["g13"])
    g2 = None if w["g2"] is None else dev(w["g2"])
    ex = M.Experts(plan, fmt, E, *ts, g13, g2)
    torch.cuda.synchronize()
    changed = [not np.array_equal(t.cpu().numpy(), w[k]) for t, k in zip(ts, ("w13", "s13", "w2", "s2"))]
    assert changed[0] and changed[2], "prepare left the weights in checkpoint layout"
    ex.unpack()
    torch.cuda.synchronize()
    for t, k in zip(ts, ("w13", "s13", "w2", "s2")):
        assert np.array_equal(t.cpu().numpy(), w[k]), k
    # an unpacked handle is refused by moe_run
    x = torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    wts = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.run(plan, [ex], x, ids, wts)
    assert ei.value.code == M.MOE_ENOTPREPARED
