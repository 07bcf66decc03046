"""Layer parity on the GPU (through the C ABI) against the CPU oracle, per row:
rel-L2 <= 1e-2 and rel max-abs <= 2e-2 against the oracle's float64
accumulator; rows with no valid slot exactly zero; deterministic mode bit-stable.
Small configurations are compared on every row, full-size ones on sampled rows."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import block_scaled_fp4_histogram_amd as M
import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import DeviceLayer, assert_rows_match, dev

pytestmark = pytest.mark.gpu

_CACHE = {}


def layer(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _CACHE:
        if name in I.CONFIGS:
            prob = I.make_problem(name)
        else:
            prob = SMALL[name]()
        _CACHE.clear()   # keep at most one large layer resident
        _CACHE[key] = DeviceLayer(prob, **kw)
        if name in SMALL and "prefill" in name:
            # small batches the ladder gives the 16-route kernels: pin the 64-route ones
            _CACHE[key].plan.set_sequence(prob.cfg.T, M.SEQ_PREFILL)
    return _CACHE[key]


SMALL = {
    # ragged T and N with a partial last k-tile in the down GEMM (N % 128 == 96)
    "mxfp4_ragged": lambda: I.make_problem(I.Config("mxfp4_ragged", T=37, E=12, K=512, N=224, topk=3, limit=7.0,
                                                    fmt=I.FMT_MXFP4, e8m0_exp=(-6, -2)), seed=3),
    "nvfp4_small": lambda: I.make_problem(I.Config("nvfp4_small", T=21, E=16, K=256, N=160, topk=4, limit=None,
                                                   fmt=I.FMT_NVFP4), seed=4),
    "nf3_small": lambda: I.make_problem(I.Config("nf3_small", T=19, E=10, K=512, N=96, topk=2, limit=None,
                                                 fmt=I.FMT_NF3), seed=5),
    "hybrid_small": lambda: I.make_problem(I.Config("hybrid_small", T=29, E=24, K=256, N=128, topk=5, limit=None,
                                                    fmt=I.FMT_NVFP4, hybrid_nvfp4=8), seed=6),
    "nvfp4_clamped": lambda: I.make_problem(I.Config("nvfp4_clamped", T=9, E=6, K=256, N=64, topk=2, limit=30.0,
                                                     fmt=I.FMT_NVFP4), seed=7),
    # decode-size batches (T <= 16, T * top_k <= 64): the two-launch path
    "hybrid_decode": lambda: I.make_problem(I.Config("hybrid_decode", T=8, E=256, K=1024, N=512, topk=8, limit=None,
                                                     fmt=I.FMT_NVFP4, hybrid_nvfp4=64), seed=8),
    # ~16 routes per expert at K=7168: the MXFP8 rows are staged through LDS in two passes
    "decode_many_routes": lambda: I.make_problem(I.Config("decode_many_routes", T=16, E=4, K=7168, N=64, topk=4,
                                                          limit=7.0, fmt=I.FMT_MXFP4, e8m0_exp=(-9, -5)), seed=9),
    "nf3_decode": lambda: I.make_problem(I.Config("nf3_decode", T=5, E=40, K=512, N=96, topk=7, limit=None,
                                                  fmt=I.FMT_NF3), seed=10),
    # decode down GEMM split over two blocks per output tile by halves of the k-tiles: uneven halves
    # (256 + 96 columns, 128 + 32 columns), the second ending in a partial k-tile
    "nf3_decode_n352": lambda: I.make_problem(I.Config("nf3_decode_n352", T=6, E=24, K=512, N=352, topk=5,
                                                       limit=None, fmt=I.FMT_NF3), seed=11),
    "nvfp4_decode_n160": lambda: I.make_problem(I.Config("nvfp4_decode_n160", T=12, E=20, K=256, N=160, topk=3,
                                                         limit=None, fmt=I.FMT_NVFP4), seed=12),
    # W4A8 batches on the prefill sequence (pinned in layer(); N % 64 == 0): 64-route tiles streamed through
    # the LDS ring; Zipf-skewed loads give full, ragged and single-tile experts, and
    # N % 128 == 64 leaves a half k-tile in the down GEMM
    "prefill_small": lambda: I.make_problem(I.Config("prefill_small", T=160, E=12, K=512, N=192, topk=4, limit=7.0,
                                                     fmt=I.FMT_MXFP4, e8m0_exp=(-6, -2), zipf_s=1.1,
                                                     pad_rows=3), seed=11),
    # one k-tile in the down GEMM (N = 64), two in the up/gate GEMM (K = 256), no clamp
    "prefill_narrow": lambda: I.make_problem(I.Config("prefill_narrow", T=130, E=3, K=256, N=64, topk=2,
                                                      limit=None, fmt=I.FMT_MXFP4), seed=12),
    # the W4A16 / W3A16 prefill kernels: NVFP4 with a half k-tile in the down GEMM,
    # NF3 with one down k-tile and the clamp, and both tiers in one batch
    "nvfp4_prefill_small": lambda: I.make_problem(I.Config("nvfp4_prefill_small", T=150, E=8, K=256, N=192,
                                                           topk=4, limit=None, fmt=I.FMT_NVFP4, pad_rows=2),
                                                  seed=13),
    "nf3_prefill_small": lambda: I.make_problem(I.Config("nf3_prefill_small", T=130, E=6, K=256, N=64, topk=2,
                                                         limit=10.0, fmt=I.FMT_NF3), seed=14),
    "hybrid_prefill_small": lambda: I.make_problem(I.Config("hybrid_prefill_small", T=140, E=12, K=512, N=128,
                                                            topk=3, limit=None, fmt=I.FMT_NVFP4, hybrid_nvfp4=4),
                                                   seed=15),
    # k-loop shapes of the prefill kernels: W4A8 down GEMM with 3 k-tiles (the last
    # half) requested up front; 6 k-tiles through the register/LDS ring with an
    # up/gate GEMM of 8 k-tiles (two whole ring turns, then closing steps); W4A16
    # down GEMMs with 3 k-tiles (straight-line) and 5 (ring)
    "prefill_n320": lambda: I.make_problem(I.Config("prefill_n320", T=140, E=6, K=256, N=320, topk=2, limit=7.0,
                                                    fmt=I.FMT_MXFP4, e8m0_exp=(-6, -2), zipf_s=1.1), seed=16),
    "prefill_n768": lambda: I.make_problem(I.Config("prefill_n768", T=128, E=4, K=1024, N=768, topk=2, limit=7.0,
                                                    fmt=I.FMT_MXFP4, e8m0_exp=(-7, -3)), seed=17),
    "nvfp4_prefill_n320": lambda: I.make_problem(I.Config("nvfp4_prefill_n320", T=136, E=5, K=256, N=320, topk=2,
                                                          limit=None, fmt=I.FMT_NVFP4), seed=18),
    "nf3_prefill_n640": lambda: I.make_problem(I.Config("nf3_prefill_n640", T=130, E=4, K=768, N=640, topk=2,
                                                        limit=None, fmt=I.FMT_NF3), seed=19),
    # the 16-bit up/gate GEMM on 128-route tiles with Zipf-skewed loads: experts spanning
    # several 128-route tiles with a ragged last one; both tiers in one launch
    "nvfp4_prefill_zipf": lambda: I.make_problem(I.Config("nvfp4_prefill_zipf", T=400, E=16, K=512, N=128, topk=4,
                                                          limit=None, fmt=I.FMT_NVFP4, zipf_s=1.1, pad_rows=3),
                                                 seed=20),
    "hybrid_prefill_zipf": lambda: I.make_problem(I.Config("hybrid_prefill_zipf", T=300, E=24, K=768, N=192, topk=6,
                                                           limit=None, fmt=I.FMT_NVFP4, hybrid_nvfp4=8,
                                                           zipf_s=1.1), seed=21),
}


def _sample_rows(prob, n, seed=0):
    """Rows to compare at full size: spread over the batch, plus every padding row and
    rows routed to the most loaded expert."""
    T = prob.cfg.T
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    ids = prob.ids
    valid = ids[(ids >= 0) & (ids < prob.cfg.E)]
    if valid.size:
        top = np.bincount(valid, minlength=prob.cfg.E).argmax()
        rows |= set(np.flatnonzero((ids == top).any(axis=1))[:4].tolist())
    rows |= set(np.flatnonzero(~((ids >= 0) & (ids < prob.cfg.E)).any(axis=1))[:2].tolist())
    return np.array(sorted(rows), dtype=np.int32)


@pytest.mark.parametrize("name", ["tiny", "mxfp4_ragged", "nvfp4_small", "nf3_small", "hybrid_small",
                                  "nvfp4_clamped", "hybrid_decode", "decode_many_routes", "nf3_decode",
                                  "nf3_decode_n352", "nvfp4_decode_n160", "prefill_small", "prefill_narrow", "nvfp4_prefill_small", "nf3_prefill_small",
                                  "hybrid_prefill_small", "prefill_n320", "prefill_n768", "nvfp4_prefill_n320",
                                  "nf3_prefill_n640", "nvfp4_prefill_zipf", "hybrid_prefill_zipf"])
@pytest.mark.parametrize("deterministic", [False, True])
def test_small_layers_all_rows(name, deterministic):
    L = layer(name)
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(L.prob)
    assert_rows_match(out, acc, label=f"{name} det={deterministic}", prob=L.prob)


@pytest.mark.parametrize("name", ["hybrid_decode", "nf3_decode", "nf3_decode_n352", "nvfp4_decode_n160",
                                  "decode_many_routes"])
def test_decode_cases_take_the_decode_sequence(name):
    L = layer(name)
    assert L.plan.sequence(L.prob.cfg.T) == M.SEQ_DECODE


@pytest.mark.parametrize("deterministic", [False, True])
def test_decode_all_rows(deterministic):
    L = layer("decode")
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(L.prob)
    assert_rows_match(out, acc, label=f"decode det={deterministic}", prob=L.prob)
    assert torch.all(out[6:].view(torch.int16) == 0)   # the two padding rows


@pytest.mark.parametrize("name,nrows", [("prefill", 20), ("nvfp4_decode", 8), ("nvfp4_prefill", 16),
                                        ("hybrid", 16)])
@pytest.mark.parametrize("deterministic", [False, True])
def test_full_size_sampled_rows(name, nrows, deterministic):
    L = layer(name)
    out = L.run(deterministic=deterministic)
    rows = _sample_rows(L.prob, nrows)
    acc, _ = O.moe_problem(L.prob, rows=rows)
    assert_rows_match(out, acc, rows=rows, label=f"{name} det={deterministic}", prob=L.prob)


@pytest.mark.parametrize("name", ["decode", "nvfp4_decode"])
@pytest.mark.parametrize("T", [1, 2, 3, 5])
def test_full_size_decode_smaller_batches(name, T):
    """The full-size decode layers on batches of their first T tokens: each batch size
    is its own capacity rung of the plan (the layer's weights and plan are shared)."""
    L = layer(name)
    p = L.prob
    q = I.Problem(p.cfg, p.x[:T].copy(), p.ids[:T].copy(), p.wts[:T].copy(), p.tiers)
    acc, _ = O.moe_problem(q)
    for det in (False, True):
        out = L.run(x=dev(q.x, torch.bfloat16), ids=dev(q.ids), wts=dev(q.wts), deterministic=det)
        assert out.shape[0] == T
        assert_rows_match(out, acc, label=f"{name} T={T} det={det}", prob=q)


@pytest.mark.parametrize("name", ["decode", "hybrid_small", "prefill", "hybrid_decode", "nf3_decode_n352",
                                  "nvfp4_decode"])
def test_deterministic_bit_stable(name):
    L = layer(name)
    outs = [L.run(deterministic=True).view(torch.int16).clone() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_chunked_batch_matches_single_launch():
    """T above the plan's max_tokens runs in chunks of the top capacity; chunks of the
    same kernel path give the bit-identical deterministic result of one launch."""
    prob = SMALL["mxfp4_ragged"]()   # T = 37
    big = DeviceLayer(prob)
    ref = big.run(deterministic=True)
    chunked = DeviceLayer(SMALL["mxfp4_ragged"](), max_tokens=20)   # chunks of 20 + 17 tokens
    out = chunked.run(deterministic=True)
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
    acc, _ = O.moe_problem(prob)
    assert_rows_match(chunked.run(deterministic=False), acc, label="chunked atomic", prob=prob)
    # chunks small enough for the decode path (8 tokens x 3 slots)
    dec = DeviceLayer(SMALL["mxfp4_ragged"](), max_tokens=8)
    for det in (False, True):
        assert_rows_match(dec.run(deterministic=det), acc, label=f"decode-size chunks det={det}", prob=prob)


@pytest.mark.parametrize("name", ["mxfp4_ragged", "decode"])
def test_invalid_ids_and_zero_weights(name):
    L = layer(name)
    p = L.prob
    E = p.cfg.E
    ids = p.ids.copy()
    wts = p.wts.copy()
    ids[:, 1] = np.array([-1, E, E + 7, np.iinfo(np.int32).min, np.iinfo(np.int32).max] * 8)[: p.cfg.T]
    ids[3, :] = -1                 # a row with no valid slot
    ids[5 % p.cfg.T, 2] = ids[5 % p.cfg.T, 0]   # a duplicate
    wts[4, 0] = 0.0                # a zero-weight slot
    for det in (False, True):
        out = L.run(ids=dev(ids), wts=dev(wts), deterministic=det)
        q = I.Problem(p.cfg, p.x, ids, wts, p.tiers)
        acc, _ = O.moe_problem(q)
        assert_rows_match(out, acc, label=f"{name} invalid ids det={det}", prob=q)
        assert torch.all(out[3].view(torch.int16) == 0)


@pytest.mark.parametrize("name", ["nvfp4_small", "decode", "hybrid_decode"])
def test_duplicate_ids_in_a_row(name):
    L = layer(name)
    p = L.prob
    ids = np.repeat(p.ids[:, :1], p.cfg.topk, axis=1).copy()
    ids[:, -1] = p.ids[:, -1]
    for det in (False, True):
        out = L.run(ids=dev(ids), deterministic=det)
        q = I.Problem(p.cfg, p.x, ids, p.wts, p.tiers)
        acc, _ = O.moe_problem(q)
        assert_rows_match(out, acc, label=f"{name} duplicate ids det={det}", prob=q)


def test_zero_tokens_is_noop_and_all_padding_batch():
    L = layer("tiny")
    c = L.prob.cfg
    x = torch.zeros((0, c.K), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((0, c.topk), dtype=torch.int32, device="cuda")
    wts = torch.zeros((0, c.topk), dtype=torch.float32, device="cuda")
    out = M.run(L.plan, L.tiers, x, ids, wts, scratch=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, c.K)
    for name in ("tiny", "mxfp4_ragged"):   # decode-size and general paths
        L = layer(name)
        c = L.prob.cfg
        ids = torch.full((c.T, c.topk), -1, dtype=torch.int32, device="cuda")
        for det in (False, True):
            out = L.run(ids=ids, deterministic=det)
            assert torch.all(out.view(torch.int16) == 0)


def test_scratch_too_small_is_refused():
    L = layer("tiny")
    c = L.prob.cfg
    need = L.plan.scratch_bytes(c.T, False)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        L.run(scratch=small)
    assert ei.value.code == M.MOE_ESCRATCH


def test_gate_up_layout_flag():
    prob = SMALL["mxfp4_ragged"]()
    L = DeviceLayer(prob, gate_up=True)
    out = L.run()
    acc, _ = O.moe_problem(prob, gate_up=True)
    assert_rows_match(out, acc, label="gate_up")


# Router weight on the input (W4A16 / W3A16 only), on every launch sequence: the general
# 16-route kernels, decode, prefill, and both hybrid tiers in one prefill launch.
@pytest.mark.parametrize("name", ["nvfp4_small", "nf3_small", "hybrid_decode", "nvfp4_prefill_small",
                                  "hybrid_prefill_small"])
@pytest.mark.parametrize("deterministic", [False, True])
def test_router_weight_on_input(name, deterministic):
    L = layer(name, weight_on_input=True)
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(L.prob, weight_on_input=True)
    assert_rows_match(out, acc, label=f"{name} weight-on-input det={deterministic}")


# SwiGLU-OAI activation gate * sigmoid(alpha gate) * (up + beta) (W4A16 / W3A16 only), on
# every launch sequence, with and without the clamp.
@pytest.mark.parametrize("name", ["nvfp4_small", "nf3_small", "nvfp4_clamped", "hybrid_decode",
                                  "nvfp4_prefill_small", "hybrid_prefill_small"])
@pytest.mark.parametrize("deterministic", [False, True])
def test_swiglu_oai(name, deterministic):
    alpha, beta = 1.702, 1.0
    L = layer(name, swiglu_oai=(alpha, beta))
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(L.prob, alpha=alpha, beta=beta)
    assert_rows_match(out, acc, label=f"{name} swiglu-oai det={deterministic}")
    plain, _ = O.moe_problem(L.prob)
    assert not np.allclose(acc, plain, rtol=1e-2), "the parameters must change this case"



# Launch sequences pinned per capacity rung (moe_plan_set_sequence): batches the ladder
# (or the pin above) would send down another sequence must give the same layer on the
# pinned one.
@pytest.mark.parametrize("name,seq", [("prefill_small", M.SEQ_PREFILL_NARROW), ("prefill_n768", M.SEQ_PREFILL_NARROW),
                                      ("nvfp4_clamped", M.SEQ_PREFILL_NARROW), ("hybrid_small", M.SEQ_PREFILL_NARROW),
                                      ("hybrid_decode", M.SEQ_GENERAL), ("hybrid_decode", M.SEQ_PREFILL),
                                      ("nf3_decode", M.SEQ_GENERAL), ("nvfp4_clamped", M.SEQ_PREFILL),
                                      ("decode_many_routes", M.SEQ_PREFILL), ("prefill_small", M.SEQ_GENERAL),
                                      ("hybrid_small", M.SEQ_PREFILL), ("mxfp4_ragged", M.SEQ_GENERAL)])
@pytest.mark.parametrize("deterministic", [False, True])
def test_pinned_sequence(name, seq, deterministic):
    L = layer(name)
    T = L.prob.cfg.T
    before = L.plan.sequence(T)
    L.plan.set_sequence(T, seq)
    try:
        assert L.plan.sequence(T) == seq
        out = L.run(deterministic=deterministic)
    finally:
        L.plan.set_sequence(T, before)
    acc, _ = O.moe_problem(L.prob)
    assert_rows_match(out, acc, label=f"{name} sequence {seq} det={deterministic}", prob=L.prob)


_SLOT_SEQ = (M.SEQ_DECODE, M.SEQ_GENERAL, M.SEQ_GENERAL, M.SEQ_PREFILL, M.SEQ_PREFILL, M.SEQ_PREFILL_NARROW,
             M.SEQ_PREFILL_NARROW)
_SLOT_COMB = (None, M.COMBINE_ATOMIC, M.COMBINE_ROUTE_BUFFER, M.COMBINE_ATOMIC, M.COMBINE_ROUTE_BUFFER,
              M.COMBINE_ATOMIC, M.COMBINE_ROUTE_BUFFER)


def _check_pins(plan, t, us, deterministic):
    times = [v if not math.isnan(v) else float("inf") for v in us]
    k = times.index(min(times))
    assert plan.sequence(t) == _SLOT_SEQ[k]
    if not deterministic and _SLOT_COMB[k] is not None:
        assert plan.combine(t) == _SLOT_COMB[k]


@pytest.mark.parametrize("deterministic", [False, True])
def test_autotune_pins_the_fastest_sequence_and_combine(deterministic):
    L = layer("hybrid_small")          # 29 tokens x 5 slots: general or the prefill ones; 8 tokens: all
    T = L.prob.cfg.T
    try:
        us = L.plan.autotune(L.tiers, [T, 8], deterministic=deterministic, reps=3)
        # no decode slot at 29 tokens; general, prefill and prefill_narrow with the route buffer
        assert math.isnan(us[0][0]) and us[0][2] > 0 and us[0][4] > 0 and us[0][6] > 0
        assert us[1][0] > 0 and us[1][2] > 0 and us[1][4] > 0 and us[1][6] > 0
        if deterministic:   # only the route-buffer combine
            assert all(math.isnan(v) for v in (us[0][1], us[0][3], us[0][5], us[1][1], us[1][3], us[1][5]))
        else:
            assert us[0][1] > 0 and us[0][3] > 0 and us[0][5] > 0
        for i, t in enumerate((T, 8)):
            _check_pins(L.plan, t, us[i], deterministic)
        out = L.run(deterministic=deterministic)
    finally:
        for t in (T, 8):
            L.plan.set_sequence(t, M.SEQ_AUTO)
            L.plan.set_combine(t, M.COMBINE_AUTO)
    acc, _ = O.moe_problem(L.prob)
    assert_rows_match(out, acc, label="hybrid_small after autotune")


@pytest.mark.parametrize("name", ["prefill_small", "nvfp4_prefill_small"])
def test_autotune_on_the_workload_s_own_batch(name):
    """The race at the rung of the caller's batch (Zipf-skewed loads in prefill_small)
    on that batch; the pinned (sequence, combine) runs the layer within tolerance."""
    L = layer(name)
    p = L.prob
    T = p.cfg.T
    x, ids, wts = dev(p.x, torch.bfloat16), dev(p.ids), dev(p.wts)
    before = L.plan.sequence(T)
    try:
        us = L.plan.autotune_batch(L.tiers, x, ids, wts, reps=3)
        a8 = p.tiers[0].fmt == I.FMT_MXFP4
        assert all(v > 0 for v in us[1:])    # every slot but decode, the 64-route up/gate variant included
        _check_pins(L.plan, T, us, False)
        out = L.run(deterministic=False)
    finally:
        L.plan.set_sequence(T, before)
        L.plan.set_combine(T, M.COMBINE_AUTO)
    acc, _ = O.moe_problem(p)
    assert_rows_match(out, acc, label=f"{name} after autotune_batch", prob=p if a8 else None)


@pytest.mark.parametrize("name,T", [("prefill_small", 160), ("mxfp4_ragged", 37), ("nvfp4_prefill_small", 150)])
def test_combine_pins_give_the_same_layer(name, T):
    """deterministic = 0 with the route-buffer combine equals the deterministic run bit for
    bit; with atomics it is within tolerance; both on the pinned or ladder sequence."""
    L = layer(name)
    p = L.prob
    acc, _ = O.moe_problem(p)
    a8 = p.tiers[0].fmt == I.FMT_MXFP4
    det = L.run(deterministic=True)
    try:
        L.plan.set_combine(T, M.COMBINE_ROUTE_BUFFER)
        rb = L.run(deterministic=False)
        assert torch.equal(rb.view(torch.int16), det.view(torch.int16))
        L.plan.set_combine(T, M.COMBINE_ATOMIC)
        at = L.run(deterministic=False)
        assert_rows_match(at, acc, label=f"{name} atomic combine", prob=p if a8 else None)
    finally:
        L.plan.set_combine(T, M.COMBINE_AUTO)


# ---- production rungs at full geometry -------------------------------------------------
# Batches of 11..511 tokens run the 16-route general kernels; at the pages' geometries
# their k-loops are 56 (K = 7168) and 48 (K = 6144) k-tiles long.

def _batch(name, T):
    """The named workload's weights with a batch of T tokens of its own routing recipe."""
    return I.make_problem(name, T=T)


@pytest.mark.parametrize("name,batches", [("decode", ((40, 12), (120, 12))), ("nvfp4_decode", ((40, 10),)),
                                          ("hybrid", ((40, 10),))])
def test_general_sequence_at_full_geometry(name, batches):
    L = layer(name, max_tokens=256)
    for T, nrows in batches:
        q = _batch(name, T)
        assert L.plan.sequence(T) == M.SEQ_GENERAL
        rows = _sample_rows(q, nrows, seed=T)
        acc, _ = O.moe_problem(q, rows=rows)
        for det in (False, True):
            out = L.run(x=dev(q.x, torch.bfloat16), ids=dev(q.ids), wts=dev(q.wts), deterministic=det)
            assert_rows_match(out, acc, rows=rows, label=f"{name} T={T} general det={det}", prob=q)


# The rungs the ladder sends to the prefill kernels below the benchmark's batch, at the
# production geometries: W4A8 with 64-route up/gate tiles while experts average under 32
# routes (from the first prefill rung, 256 tokens: 4 an expert) and 128-route ones from
# there (2048: 32); 16-bit activations with 128-route ones from the first prefill rung (512
# tokens: 16 an expert).
@pytest.mark.parametrize("name,T,seq", [("prefill", 256, M.SEQ_PREFILL_NARROW), ("prefill", 2048, M.SEQ_PREFILL),
                                        ("nvfp4_prefill", 512, M.SEQ_PREFILL), ("hybrid", 1024, M.SEQ_PREFILL)])
def test_ladder_prefill_rungs_at_full_geometry(name, T, seq):
    L = layer(name, max_tokens=T)
    q = _batch(name, T)
    assert L.plan.sequence(T) == seq
    rows = _sample_rows(q, 10, seed=T)
    acc, _ = O.moe_problem(q, rows=rows)
    for det in (False, True):
        out = L.run(x=dev(q.x, torch.bfloat16), ids=dev(q.ids), wts=dev(q.wts), deterministic=det)
        assert_rows_match(out, acc, rows=rows, label=f"{name} T={T} seq={seq} det={det}", prob=q)


def test_hybrid_decode_at_full_geometry():
    """Both tiers (64 NVFP4 + 192 NF3 experts, K = 6144, N = 512, top-8) on the decode
    sequence, every row, both combine modes."""
    L = layer("hybrid", max_tokens=8)
    q = _batch("hybrid", 8)
    assert L.plan.sequence(8) == M.SEQ_DECODE
    acc, _ = O.moe_problem(q)
    for det in (False, True):
        out = L.run(x=dev(q.x, torch.bfloat16), ids=dev(q.ids), wts=dev(q.wts), deterministic=det)
        assert_rows_match(out, acc, label=f"hybrid T=8 decode det={det}")


def _tile_rows(prob, tile=64, hottest=5):
    """Tokens of the first route, a middle tile's route and the last route (the last,
    ragged tile) of the most loaded experts, and of every expert holding one route."""
    c = prob.cfg
    cnt, off, perm, _ = O.route(prob.ids, c.E, prob.tiers)
    rows = set()
    for e in np.argsort(-cnt, kind="stable")[:hottest]:
        n = int(cnt[e])
        tiles = (n + tile - 1) // tile
        for pos in (0, (tiles // 2) * tile + 7, n - 1):
            rows.add(int(perm[off[e] + min(pos, n - 1)]) // c.topk)
    for e in np.flatnonzero(cnt == 1)[:4]:
        rows.add(int(perm[off[e]]) // c.topk)
    return np.array(sorted(rows), dtype=np.int32)


def test_prefill_hot_expert_tiles():
    L = layer("prefill")
    assert L.plan.sequence(L.prob.cfg.T) == M.SEQ_PREFILL
    rows = _tile_rows(L.prob)
    acc, _ = O.moe_problem(L.prob, rows=rows)
    for det in (False, True):
        out = L.run(deterministic=det)
        assert_rows_match(out, acc, rows=rows, label=f"prefill hot tiles det={det}", prob=L.prob)


@pytest.mark.parametrize("name,max_tokens", [("nvfp4_small", 17), ("nf3_small", 17), ("hybrid_small", 24)])
@pytest.mark.parametrize("deterministic", [False, True])
def test_sixteen_bit_plans_with_a_decode_sized_last_chunk(name, max_tokens, deterministic):
    """A top capacity above the decode sizes (the arena is carved for the general
    kernels) and a decode-size last chunk (4, 2 and 5 tokens), whose down GEMM meets
    its two halves in the arena's accumulators."""
    prob = SMALL[name]()
    L = DeviceLayer(prob, max_tokens=max_tokens)
    T = prob.cfg.T
    assert L.plan.sequence(max_tokens) != M.SEQ_DECODE and L.plan.sequence(T % max_tokens) == M.SEQ_DECODE
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(prob)
    assert_rows_match(out, acc, label=f"{name} chunks of {max_tokens} det={deterministic}")


# SiTU, silu(4 tanh(gate/4)) * 25 tanh(up/25), on every launch sequence and both
# activation formats (W4A8 too: the page runs SiTU there): decode (tiny, hybrid_decode),
# general (mxfp4_ragged, nvfp4_small) and prefill (prefill_small, nvfp4_prefill_small,
# hybrid_prefill_small).
@pytest.mark.parametrize("name", ["tiny", "mxfp4_ragged", "prefill_small", "nvfp4_small", "hybrid_decode",
                                  "nvfp4_prefill_small", "hybrid_prefill_small"])
def test_situ(name):
    L = layer(name, act=M.ACT_SITU)
    acc, _ = O.moe_problem(L.prob, act_kind=O.ACT_SITU)
    a8 = L.prob.tiers[0].fmt == I.FMT_MXFP4
    for det in (False, True):
        out = L.run(deterministic=det)
        assert_rows_match(out, acc, label=f"{name} situ det={det}", prob=L.prob if a8 else None,
                          act_kind=O.ACT_SITU)
    plain, _ = O.moe_problem(L.prob)
    assert not np.allclose(acc, plain, rtol=1e-2), "SiTU must change this case"


# ReLU^2 without the gate multiply (16-bit activations): w13 of N rows; every launch
# sequence; NVFP4, NF3 and two tiers.
def _relu2_problem(cfg, seed):
    """A problem whose w13 keeps the first N of its 2N rows (the checkpoint of a
    ReLU^2 layer has N rows)."""
    import dataclasses
    prob = I.make_problem(cfg, seed=seed)
    N = cfg.N
    tiers = []
    for t in prob.tiers:
        w = dict(t.weights)
        w["w13"] = np.ascontiguousarray(w["w13"][:, :N])
        w["s13"] = np.ascontiguousarray(w["s13"][:, :N])
        tiers.append(dataclasses.replace(t, weights=w))
    return dataclasses.replace(prob, tiers=tiers)


RELU2 = {
    "r2_general": (I.Config("r2_general", T=21, E=16, K=256, N=128, topk=4, limit=None, fmt=I.FMT_NVFP4), 31,
                   None),
    "r2_decode_nf3": (I.Config("r2_decode_nf3", T=6, E=20, K=512, N=192, topk=3, limit=None, fmt=I.FMT_NF3), 32,
                      None),
    "r2_prefill": (I.Config("r2_prefill", T=150, E=8, K=256, N=256, topk=4, limit=None, fmt=I.FMT_NVFP4,
                            pad_rows=2), 33, M.SEQ_PREFILL),
    "r2_hybrid_prefill": (I.Config("r2_hybrid_prefill", T=140, E=12, K=512, N=128, topk=3, limit=None,
                                   fmt=I.FMT_NVFP4, hybrid_nvfp4=4), 34, M.SEQ_PREFILL),
    "r2_hybrid_decode": (I.Config("r2_hybrid_decode", T=8, E=256, K=1024, N=512, topk=8, limit=None,
                                  fmt=I.FMT_NVFP4, hybrid_nvfp4=64), 35, None),
}


@pytest.mark.parametrize("name", sorted(RELU2))
def test_relu2_no_mul(name):
    cfg, seed, pin = RELU2[name]
    prob = _relu2_problem(cfg, seed)
    L = DeviceLayer(prob, act=M.ACT_RELU2_NO_MUL)
    if pin is not None:
        L.plan.set_sequence(cfg.T, pin)
    assert L.plan.sequence(cfg.T) == (pin or (M.SEQ_DECODE if "decode" in name else M.SEQ_GENERAL))
    acc, _ = O.moe_problem(prob, act_kind=O.ACT_RELU2_NO_MUL)
    for det in (False, True):
        out = L.run(deterministic=det)
        assert_rows_match(out, acc, label=f"{name} relu2 det={det}")


def test_relu2_repack_round_trip():
    cfg, seed, _ = RELU2["r2_decode_nf3"]
    prob = _relu2_problem(cfg, seed)
    L = DeviceLayer(prob, act=M.ACT_RELU2_NO_MUL)
    ex, _ = L.tiers[0]
    before = [t.cpu().clone() for t in L.keep[:4]]
    ex.unpack()
    torch.cuda.synchronize()
    w = prob.tiers[0].weights
    for t, k in zip(L.keep[:4], ("w13", "s13", "w2", "s2")):
        assert np.array_equal(t.cpu().numpy(), w[k]), k
    assert not torch.equal(before[0], L.keep[0].cpu())   # the tile layout differs from the checkpoint


def _scale_bf16(x, e):
    """bf16 bits times 2^e elementwise (e broadcast to x's shape); exact while the values stay bf16 normals."""
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * np.exp2(e)
    b = f.astype(np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


# E4M3 scale bytes 448, 1, 2^-3 and 2^-6, one per 32-column slice of the intermediate in turn
_SLICE_SCALES = np.array([0x7E, 0x38, 0x20, 0x08], dtype=np.uint8)


def _wide_range_problem(name):
    """A decode-size 16-bit layer whose token rows span 2^-16 .. 2^16 times the generator's values, with the
    four k-tile classes of a row (k-tile index mod 4) a further 2^-8 .. 2^10 apart, and whose w13 scales put
    the intermediate's 32-column slices up to about 2^30 apart within one row."""
    p = SMALL[name]()
    T, K, N = p.cfg.T, p.cfg.K, p.cfg.N
    row_e = np.round(np.linspace(-16, 16, T))[:, None]
    col_e = np.array([-8, -2, 4, 10])[(np.arange(K) // 128) % 4][None, :]
    x = _scale_bf16(p.x, row_e + col_e)
    tiers = []
    for t in p.tiers:
        w = dict(t.weights)
        s13 = w["s13"].copy()
        cls = _SLICE_SCALES[(np.arange(N) // 32) % 4]
        s13[:, :N, :] = cls[None, :, None]   # up rows ([up; gate] stacking)
        s13[:, N:, :] = cls[None, :, None]   # gate rows
        w["s13"] = s13
        tiers.append(dataclasses.replace(t, weights=w))
    return I.Problem(p.cfg, x, p.ids, p.wts, tiers)


@pytest.mark.parametrize("name", ["nvfp4_decode_n160", "nf3_decode_n352", "hybrid_decode"])
@pytest.mark.parametrize("deterministic", [False, True])
def test_decode_fp16_operands_over_wide_ranges(name, deterministic):
    """The 16-bit decode kernels multiply in fp16 on operands scaled by powers of two (per route row and
    wave for the activations, per 32-column slice then per route row for the intermediate): rows far
    outside fp16's range, waves of one row with different exponents, and intermediate slices from equal
    to more than 24 binades apart all stay within the row tolerance of the oracle."""
    prob = _wide_range_problem(name)
    L = DeviceLayer(prob)
    assert L.plan.sequence(prob.cfg.T) == M.SEQ_DECODE
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(prob)
    assert np.all(np.isfinite(acc))
    mags = np.abs(acc).max(axis=1)
    assert mags.max() / mags[mags > 0].min() > 2.0 ** 40   # the rows really span a wide range
    assert_rows_match(out, acc, label=f"{name} wide det={deterministic}", prob=prob)


@pytest.mark.parametrize("name", ["nvfp4_prefill_small", "hybrid_prefill_small", "nvfp4_prefill_zipf"])
@pytest.mark.parametrize("deterministic", [False, True])
def test_prefill_fp16_down_gemm_over_wide_ranges(name, deterministic):
    """The NVFP4 route-buffer down GEMM converts each tile's intermediate rows to fp16 times a power of two
    per route: token rows from 2^-16 to 2^16 times the generator's values (the intermediate then spans
    about 2^64) stay within the row tolerance on the prefill sequence, NF3 tiles (bf16) alongside."""
    prob = _wide_range_problem(name)
    L = DeviceLayer(prob)
    L.plan.set_sequence(prob.cfg.T, M.SEQ_PREFILL)
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(prob)
    assert np.all(np.isfinite(acc))
    mags = np.abs(acc).max(axis=1)
    assert mags.max() / mags[mags > 0].min() > 2.0 ** 40
    assert_rows_match(out, acc, label=f"{name} wide det={deterministic}", prob=prob)


# The prefill GEMMs read copies of the MXFP4 scales stored per row tile in runs of four
# whole k-tiles (a lane's four bytes in one dword), then the whole k-tiles after the
# last run, then a partial last k-tile; NVFP4 layers of the same shapes alongside (their
# two-byte scales keep the tile layout, with odd and partial k-tile counts).  Widths
# with two runs and a partial k-tile (1088), a run and a tail of three (896), and two
# runs, a tail of two and a partial k-tile (1344); hidden sizes with two runs and a tail
# of two (1280), one run and a tail of two (768) and a tail of two alone (256); every
# launch sequence.
@pytest.mark.parametrize("fmt", [I.FMT_MXFP4, I.FMT_NVFP4])
@pytest.mark.parametrize("N,K", [(896, 1280), (1088, 256), (1344, 768)])
@pytest.mark.parametrize("seq", [M.SEQ_DECODE, M.SEQ_GENERAL, M.SEQ_PREFILL, M.SEQ_PREFILL_NARROW])
@pytest.mark.parametrize("deterministic", [False, True])
def test_scale_runs(fmt, N, K, seq, deterministic):
    T = 6 if seq == M.SEQ_DECODE else 96
    extra = {"e8m0_exp": (-7, -3)} if fmt == I.FMT_MXFP4 else {}
    prob = I.make_problem(I.Config(f"scale_runs_{fmt}_n{N}_k{K}", T=T, E=4, K=K, N=N, topk=2, limit=7.0, fmt=fmt,
                                   **extra), seed=N + K + T + fmt)
    L = DeviceLayer(prob)
    L.plan.set_sequence(T, seq)
    assert L.plan.sequence(T) == seq
    out = L.run(deterministic=deterministic)
    acc, _ = O.moe_problem(prob)
    assert_rows_match(out, acc, label=f"fmt {fmt} N={N} sequence {seq} det={deterministic}", prob=prob)
