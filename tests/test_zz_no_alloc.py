"""moe_run_noalloc (the library's static device arena as scratch) against moe_run
with a caller arena, through the C ABI: two calls in a row, the second with a
smaller batch, on the general and decode sequences of a W4A8 and a W4A16 layer;
bit-identical in deterministic mode, within the per-row tolerance of the oracle
in atomic mode. Batches beyond the arena are refused."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_histogram_amd as M
import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import DeviceLayer, assert_rows_match, dev

pytestmark = pytest.mark.gpu


def _sub(prob, T):
    return I.Problem(prob.cfg, prob.x[:T].copy(), prob.ids[:T].copy(), prob.wts[:T].copy(), prob.tiers)


@pytest.mark.parametrize("cfg", [
    I.Config("na_mxfp4", T=37, E=12, K=512, N=224, topk=3, limit=7.0, fmt=I.FMT_MXFP4, e8m0_exp=(-6, -2)),
    I.Config("na_nvfp4", T=30, E=16, K=256, N=160, topk=4, limit=None, fmt=I.FMT_NVFP4),
])
def test_noalloc_matches_moe_run_on_two_calls(cfg):
    prob = I.make_problem(cfg, seed=21)
    L = DeviceLayer(prob)
    a8 = cfg.fmt == I.FMT_MXFP4
    for T in (cfg.T, 5):   # the general sequence, then a smaller decode-size batch
        q = _sub(prob, T)
        x, ids, wts = dev(q.x, torch.bfloat16), dev(q.ids), dev(q.wts)
        acc, _ = O.moe_problem(q)
        for det in (True, False):
            ref = M.run(L.plan, L.tiers, x, ids, wts, deterministic=det)
            out = torch.full_like(ref, float("nan"))
            M.run_noalloc(L.plan, L.tiers, x, ids, wts, out, deterministic=det)
            torch.cuda.synchronize()
            if det:
                assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"T={T}"
            assert_rows_match(out, acc, label=f"{cfg.name} noalloc T={T} det={det}", prob=q if a8 else None)


def test_noalloc_refuses_batches_beyond_its_arena():
    prob = I.make_problem("tiny")
    c = prob.cfg
    T = 65536
    L = DeviceLayer(prob, max_tokens=T)
    assert L.plan.scratch_bytes(T, True) > 64 << 20
    x = torch.zeros((T, c.K), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((T, c.topk), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, c.topk), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(M.MoeError) as ei:
        M.run_noalloc(L.plan, L.tiers, x, ids, wts, out, deterministic=True)
    assert ei.value.code == M.MOE_ESCRATCH and "64 MiB" in str(ei.value)
    M.run_noalloc(L.plan, L.tiers, x[:0], ids[:0], wts[:0], out[:0])   # T = 0: a no-op
