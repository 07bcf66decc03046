"""The GPU tests' row check for W4A8 layers lets a row differ from the oracle by a
whole E4M3 step of an intermediate element only where that element sits on a
rounding midpoint (both codes correct up to summation order). These cases pin that
it accepts such a flip and nothing else, with the oracle alone."""
import numpy as np
import torch

import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import _tie_flips, assert_rows_match

# T=520 E=20 K=512 N=128 top-4 MXFP4: token 148's first slot (expert 6) has an
# intermediate element whose scaled value is within 1.2e-6 of the midpoint between
# the E4M3 codes 352 and 384
CFG = I.Config("tie", T=520, E=20, K=512, N=128, topk=4, limit=None, fmt=I.FMT_MXFP4, pad_rows=1,
               e8m0_exp=(-7, -3))
SEED = 38985
ROW = 148


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_midpoint_flip_is_accepted_and_other_errors_are_not():
    prob = I.make_problem(CFG, seed=SEED)
    acc, _ = O.moe_problem(prob, rows=[ROW])
    big = [f for f in _tie_flips(prob, ROW) if np.linalg.norm(f) > 1e-2 * np.linalg.norm(acc[0])]
    assert len(big) == 1 and np.linalg.norm(big[0]) > 0.03 * np.linalg.norm(acc[0])
    flipped = acc + big[0]
    assert_rows_match(_bf16(flipped), acc, rows=None, label="flip", prob=_one_row(prob, ROW))
    try:
        assert_rows_match(_bf16(flipped), acc, label="flip without prob")
    except AssertionError:
        pass
    else:
        raise AssertionError("the flip alone must be outside the plain tolerance")
    d = np.random.default_rng(0).standard_normal(acc.shape)
    for wrong in (acc + d * np.linalg.norm(big[0]) / np.linalg.norm(d), acc * 1.04, acc - big[0]):
        try:
            assert_rows_match(_bf16(wrong), acc, label="planted", prob=_one_row(prob, ROW))
        except AssertionError:
            continue
        raise AssertionError("an error that is not a midpoint flip passed")


def _one_row(prob, r):
    """The problem restricted to token r (the check maps result rows to tokens)."""
    import dataclasses
    cfg = dataclasses.replace(prob.cfg, T=1)
    return dataclasses.replace(prob, cfg=cfg, x=prob.x[r:r + 1], ids=prob.ids[r:r + 1], wts=prob.wts[r:r + 1])


def test_no_flips_for_16_bit_layers_or_ignored_ids():
    """16-bit activation layers round h to bf16, whose steps stay inside the row
    tolerance: no flips are offered. Ids the layer skips offer none either."""
    nv = I.make_problem(I.Config("nv", T=3, E=6, K=256, N=64, topk=2, limit=None, fmt=I.FMT_NVFP4), seed=1)
    assert all(_tie_flips(nv, t) == [] for t in range(3))
    prob = I.make_problem(CFG, seed=SEED)
    one = _one_row(prob, ROW)
    assert len(_tie_flips(one, 0)) > 0
    ids = one.ids.copy()
    ids[0, :] = [-1, CFG.E, CFG.E + 5, np.iinfo(np.int32).min]
    assert _tie_flips(dataclasses_replace(one, ids=ids), 0) == []


def dataclasses_replace(prob, **kw):
    import dataclasses
    return dataclasses.replace(prob, **kw)


def test_more_than_one_flipped_row_fails():
    """At most max(1, 1 %) of the compared rows may pass through flips: the same
    flipped row twice in a two-row comparison is refused."""
    import dataclasses
    import pytest
    prob = I.make_problem(CFG, seed=SEED)
    acc, _ = O.moe_problem(prob, rows=[ROW])
    big = [f for f in _tie_flips(prob, ROW) if np.linalg.norm(f) > 1e-2 * np.linalg.norm(acc[0])]
    two = dataclasses.replace(prob, cfg=dataclasses.replace(prob.cfg, T=2), x=prob.x[[ROW, ROW]],
                              ids=prob.ids[[ROW, ROW]], wts=prob.wts[[ROW, ROW]])
    acc2 = np.concatenate([acc, acc])
    flipped2 = acc2 + big[0]
    with pytest.raises(AssertionError, match="needed midpoint flips"):
        assert_rows_match(_bf16(flipped2), acc2, label="two flipped rows", prob=two)
    one_flipped = np.concatenate([acc + big[0], acc])
    assert_rows_match(_bf16(one_flipped), acc2, label="one flipped row", prob=two)


def test_flips_follow_the_gate_up_layout():
    """With w13 stacked [gate; up] the halves swap: the flips offered for the swapped
    reading of the same weights are those of the oracle run with gate_up."""
    prob = _one_row(I.make_problem(CFG, seed=SEED), ROW)
    a = _tie_flips(prob, 0, gate_up=False)
    b = _tie_flips(prob, 0, gate_up=True)
    assert len(a) > 0
    assert len(a) != len(b) or any(not np.allclose(x, y) for x, y in zip(a, b))
