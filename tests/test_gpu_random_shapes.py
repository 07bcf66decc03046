"""Seeded sweep of random layer shapes through the C ABI, every row against the oracle.

Each case draws the expert count, hidden and intermediate sizes (within the plan's
constraints: K % 256 == 0, N % 32 == 0), top-k, weight format (MXFP4, NVFP4, NF3 or
two tiers), clamp and a batch size that lands on the decode (<= 16 tokens and <= 64
routes), 16-route or 64-route launch sequence, with and without padding rows, and
runs both combine modes. The list is fixed by its two seeds, so a failure names a
reproducible case. Rows are compared with the oracle under the same rule as every
other GPU test, including its allowance for intermediate codes on a rounding
midpoint."""
import numpy as np
import pytest

import oracle as O
from block_scaled_fp4_histogram_amd import inputs as I

from gpu_util import DeviceLayer, assert_rows_match

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ["decode", "general", "prefill"][i % 3]
        fmt = [I.FMT_MXFP4, I.FMT_NVFP4, I.FMT_NF3, "hybrid"][int(rng.integers(0, 4))]
        E = int(rng.integers(2, 41))
        K = 256 * int(rng.integers(1, 4))
        topk = int(rng.integers(1, min(8, E) + 1))
        if kind == "prefill":
            N = 64 * int(rng.integers(1, 4))            # the 64-route kernels take N % 64 == 0
            T = int(rng.integers(512, 561))
            topk = min(topk, 4)
        else:
            N = 32 * int(rng.integers(1, 11))
            T = int(rng.integers(1, 17)) if kind == "decode" else int(rng.integers(17, 200))
            if kind == "decode":
                topk = min(topk, 64 // T)
        hybrid = fmt == "hybrid"
        cfg = I.Config(f"s{seed}_{i}_{kind}", T=T, E=E, K=K, N=N, topk=topk,
                       limit=[None, 7.0, 30.0][int(rng.integers(0, 3))],
                       fmt=I.FMT_NVFP4 if hybrid else fmt,
                       pad_rows=int(rng.integers(0, min(2, T - 1) + 1)) if T > 1 else 0,
                       e8m0_exp=(-7, -3) if K <= 512 else (-8, -4),
                       hybrid_nvfp4=int(rng.integers(1, E)) if hybrid else 0)
        out.append((cfg, int(rng.integers(0, 1 << 16))))
    return out


CASES = _cases(24, 2026) + _cases(24, 7)


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c.name for c, _ in CASES])
def test_random_shape_all_rows(case):
    cfg, seed = CASES[case]
    print(f"case {cfg} seed {seed}", flush=True)
    prob = I.make_problem(cfg, seed=seed)
    L = DeviceLayer(prob)
    acc, _ = O.moe_problem(prob)
    for det in (False, True):
        out = L.run(deterministic=det)
        assert_rows_match(out, acc, label=f"{cfg.name} det={det}", prob=prob)
