"""The EP id remap kernel (moe_ep_remap) against the oracle, bit for bit, and the
layer's view of it: a remapped batch runs the same layer as the batch with the
foreign slots dropped."""
import json
import os

import numpy as np
import pytest
import torch

import block_scaled_fp4_histogram_amd as M
import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import DeviceLayer, assert_rows_match, dev

pytestmark = pytest.mark.gpu

REMAP = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ep_remap.json")))


def _remap(ids, w, offset, num_local):
    oi, ow = M.ep_remap(dev(ids), dev(w), offset, num_local)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ow.cpu().numpy()


@pytest.mark.parametrize("case", range(len(REMAP["cases"])))
def test_hand_worked_cases(case):
    c = REMAP["cases"][case]
    oi, ow = _remap(np.array(c["ids"], np.int32), np.array(c["w"], np.float32), c["offset"], c["num_local"])
    assert oi.tolist() == c["out_ids"] and ow.tolist() == c["out_w"]


@pytest.mark.parametrize("T,k,num_local,offset", [(1, 1, 1, 0), (8, 6, 96, 96), (37, 8, 64, 192),
                                                  (4096, 6, 96, 288), (2048, 8, 32, 0), (3000, 16, 7, 5)])
def test_random_batches_bit_exact(T, k, num_local, offset):
    rng = np.random.default_rng(T + k)
    ids = rng.integers(-1, offset + 2 * num_local + 3, size=(T, k)).astype(np.int32)
    ids[rng.random((T, k)) < 0.01] = np.iinfo(np.int32).min
    ids[rng.random((T, k)) < 0.01] = np.iinfo(np.int32).max
    w = rng.random((T, k)).astype(np.float32)
    ref_i, ref_w = O.ep_remap(ids, w, offset, num_local)
    oi, ow = _remap(ids, w, offset, num_local)
    assert np.array_equal(oi, ref_i) and np.array_equal(ow.view(np.uint32), ref_w.view(np.uint32))


def test_no_local_slot_and_empty_batch():
    ids = np.full((5, 3), 7, np.int32)
    oi, ow = _remap(ids, np.ones((5, 3), np.float32), 100, 4)
    assert np.all(oi == 0) and np.all(ow == 0)
    e = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    oi, ow = M.ep_remap(e, torch.zeros((0, 4), dtype=torch.float32, device="cuda"), 0, 8)
    assert oi.shape == (0, 4) and ow.shape == (0, 4)


@pytest.mark.parametrize("name,rank", [("nvfp4_small", 1), ("mxfp4_ragged", 0), ("hybrid_decode", 1)])
def test_remapped_batch_runs_the_rank_s_share_of_the_layer(name, rank):
    """One rank of a two-rank expert-parallel layer: global ids over 2E experts, this
    rank holding [rank E, rank E + E). The remapped batch (foreign slots: weight 0 on a
    local expert) gives the bit-identical deterministic output of the batch whose
    foreign slots are dropped (-1), up to the sign of zero, and both match the oracle."""
    from test_gpu_layer import SMALL
    prob = SMALL[name]()
    c = prob.cfg
    E = c.E
    rng = np.random.default_rng(rank + 3)
    gids = rng.integers(0, 2 * E, size=(c.T, c.topk)).astype(np.int32)
    gids[-1, :] = -1
    lo = rank * E
    dropped = np.where((gids >= lo) & (gids < lo + E), gids - lo, -1).astype(np.int32)
    L = DeviceLayer(prob)
    ri, rw = M.ep_remap(dev(gids), dev(prob.wts), lo, E)
    q = I.Problem(c, prob.x, dropped, prob.wts, prob.tiers)
    acc, _ = O.moe_problem(q)
    a = L.run(ids=ri, wts=rw, deterministic=True)
    b = L.run(ids=dev(dropped), deterministic=True)
    # the same values (a zero-weight slot may leave -0 where the dropped slot leaves +0)
    assert torch.equal(a.float(), b.float())
    a8 = prob.tiers[0].fmt == I.FMT_MXFP4
    assert_rows_match(a, acc, label=f"{name} rank {rank} remapped", prob=q if a8 else None)
    assert_rows_match(L.run(ids=ri, wts=rw, deterministic=False), acc, label=f"{name} remapped atomic",
                      prob=q if a8 else None)
