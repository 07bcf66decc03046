"""moe_run captured in a HIP graph: every replay, with the program's own eager work
and synchronisations between replays, must reproduce the eager result."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_histogram_amd as M
import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import DeviceLayer, assert_rows_match, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("deterministic", [True, False])
@pytest.mark.parametrize("name", ["decode_small", "nvfp4_small", "nvfp4_split"])
def test_graph_replays_match_eager(name, deterministic):
    if name == "decode_small":
        cfg = I.Config("decode_small", T=8, E=64, K=1024, N=192, topk=6, limit=7.0, fmt=I.FMT_MXFP4,
                       pad_rows=2, e8m0_exp=(-8, -4))
    elif name == "nvfp4_small":
        cfg = I.Config("nvfp4_small", T=8, E=32, K=512, N=128, topk=8, limit=None, fmt=I.FMT_NVFP4)
    else:
        # two k-tiles: the down GEMM's two blocks per output tile meet through counters and
        # accumulators that the up/gate kernel clears on every replay
        cfg = I.Config("nvfp4_split", T=8, E=32, K=512, N=256, topk=8, limit=None, fmt=I.FMT_NVFP4)
    prob = I.make_problem(cfg, seed=11)
    L = DeviceLayer(prob)
    x = dev(prob.x, torch.bfloat16)
    ids = dev(prob.ids)
    wts = dev(prob.wts)
    out = torch.empty_like(x)
    scratch = M.scratch_for(L.plan, cfg.T, deterministic)
    eager = M.run(L.plan, L.tiers, x, ids, wts, out, deterministic, scratch).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.run(L.plan, L.tiers, x, ids, wts, out, deterministic, scratch)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        M.run(L.plan, L.tiers, x, ids, wts, out, deterministic, scratch)
    acc, _ = O.moe_problem(prob)
    for rep in range(4):
        out.fill_(1.0)                     # eager work between replays
        junk = (x.float() * 2).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if deterministic:
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert_rows_match(out, acc, label=f"{name} replay {rep} det={deterministic}", prob=prob)
        del junk
