"""Helpers shared by the GPU tests: move a seeded problem to the device, run the
layer through the C ABI, and compare against the oracle row by row."""
import numpy as np
import torch

import block_scaled_fp4_histogram_amd as M
from block_scaled_fp4_histogram_amd import inputs as I

A_OF = {I.FMT_MXFP4: M.A_MXFP8, I.FMT_NVFP4: M.A_BF16, I.FMT_NF3: M.A_BF16}

# per-row acceptance: rel-L2 and rel max-abs against the oracle's float64 accumulator
REL_L2 = 1e-2
REL_MAXABS = 2e-2


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


class DeviceLayer:
    """Plan + prepared experts of a Problem, on cuda:0."""

    def __init__(self, prob, max_tokens=None, gate_up=False, weight_on_input=False, swiglu_oai=None):
        c = prob.cfg
        self.prob = prob
        self.plan = M.Plan(c.E, c.K, c.N, c.topk, c.limit, A_OF[prob.tiers[0].fmt],
                           M.W13_GATE_UP if gate_up else M.W13_UP_GATE, max_tokens or max(c.T, 1))
        if weight_on_input:
            self.plan.set_router_weight_on_input(True)
        if swiglu_oai is not None:
            self.plan.set_swiglu_oai(*swiglu_oai)
        self.tiers = []
        self.keep = []
        for t in prob.tiers:
            w = t.weights
            g13 = None if w["g13"] is None else dev(w["g13"])
            g2 = None if w["g2"] is None else dev(w["g2"])
            ts = [dev(w[k]) for k in ("w13", "s13", "w2", "s2")]
            ex = M.Experts(self.plan, t.fmt, t.E, ts[0], ts[1], ts[2], ts[3], g13, g2)
            emap = None if t.emap is None else dev(t.emap)
            self.keep += ts + [g13, g2, emap]
            self.tiers.append((ex, emap))

    def run(self, x=None, ids=None, wts=None, deterministic=False, scratch=None):
        p = self.prob
        x = dev(p.x, torch.bfloat16) if x is None else x
        ids = dev(p.ids) if ids is None else ids
        wts = dev(p.wts) if wts is None else wts
        out = M.run(self.plan, self.tiers, x, ids, wts, deterministic=deterministic, scratch=scratch)
        torch.cuda.synchronize()
        return out


def bf16_to_f64(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16).view(np.float32).astype(np.float64)


def row_errors(got, ref):
    """Per-row (rel-L2, rel max-abs) of got against ref (float64 arrays [n, K])."""
    d = got - ref
    nref = np.linalg.norm(ref, axis=1)
    mref = np.abs(ref).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        l2 = np.where(nref > 0, np.linalg.norm(d, axis=1) / nref, np.where(np.abs(got).max(axis=1) > 0, np.inf, 0.0))
        mx = np.where(mref > 0, np.abs(d).max(axis=1) / mref, np.where(np.abs(got).max(axis=1) > 0, np.inf, 0.0))
    return l2, mx


def assert_rows_match(got_bf16, acc, rows=None, label=""):
    got = bf16_to_f64(got_bf16)
    if rows is not None:
        got = got[rows]
    l2, mx = row_errors(got, acc)
    zero_ref = ~np.any(acc != 0, axis=1)
    assert np.all(got[zero_ref] == 0), f"{label}: rows with no valid slot must be exactly zero"
    bad = np.flatnonzero((l2 > REL_L2) | (mx > REL_MAXABS))
    assert bad.size == 0, (f"{label}: {bad.size} rows out of tolerance; worst rel-L2 {l2.max():.3e} "
                           f"rel-maxabs {mx.max():.3e}; first bad rows {bad[:8]}")
    return float(l2.max()), float(mx.max())
