"""Float64 dense MoE written with numpy, used to pin the oracle.

Independent of the oracle's C code: weights are decoded with numpy from the
golden E2M1 table, the pages' E8M0 formula 2^(b-127), torch's float8_e4m3fn
decode and the pages' NF3 codebook; the GEMMs are numpy matmuls. Where the layer
quantises activations (MXFP8 for W4A8, bf16 for W4A16) it calls the oracle's
quantiser and bf16 rounding, which are pinned on their own in
test_oracle_formats.py.
"""
import json
import os

import numpy as np
import torch

import oracle as O

_G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formats.json")))
E2M1 = np.array(_G["e2m1_table"]["codes_0_to_15"], np.float64)
NF3 = np.array(_G["nf3"]["codebook"], np.float32).astype(np.float64)
E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e8m0(b):
    return np.power(2.0, b.astype(np.float64) - 127.0)


def fp4_codes(w):
    lo = (w & 15).astype(np.int64)
    hi = (w >> 4).astype(np.int64)
    return np.stack([lo, hi], -1).reshape(w.shape[:-1] + (w.shape[-1] * 2,))


def nf3_codes(w):
    g = w.reshape(w.shape[:-1] + (w.shape[-1] // 3, 3)).astype(np.int64)
    w24 = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    c = np.stack([(w24 >> (3 * i)) & 7 for i in range(8)], -1)
    return c.reshape(w.shape[:-1] + (-1,))


def dequant(fmt, w, s, g=1.0):
    if fmt == O.FMT_MXFP4:
        return E2M1[fp4_codes(w)] * np.repeat(e8m0(s), 32, axis=-1)
    if fmt == O.FMT_NVFP4:
        return E2M1[fp4_codes(w)] * np.repeat(E4M3[s], 16, axis=-1) * float(g)
    return NF3[nf3_codes(w)] * np.repeat(E4M3[s], 32, axis=-1)


def _mx_fake(v32):
    q, s = O.mxfp8_quantize_f32(v32[None, :].astype(np.float32))
    return E4M3[q[0]] * np.repeat(e8m0(s[0]), 32)


def _bf16(v):
    return np.array([O.bf16_to_float(O.bf16_from_float(float(a))) for a in v])


def silu_mul(gate, up):
    return gate / (1.0 + np.exp(-gate)) * up


def expert_mlp(fmt, wts, e, x_bf16_row, K, N, limit, gate_up=False, x_scale=1.0, act=silu_mul):
    """One token through one expert, float64, quantisation as the format demands;
    x_scale multiplies the (16-bit) input first; act(gate, up) is the activation
    applied after the clamps."""
    g13 = 1.0 if wts.get("g13") is None else float(wts["g13"][e])
    g2 = 1.0 if wts.get("g2") is None else float(wts["g2"][e])
    W13 = dequant(fmt, wts["w13"][e], wts["s13"][e], g13)
    W2 = dequant(fmt, wts["w2"][e], wts["s2"][e], g2)
    x = (x_bf16_row.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if fmt == O.FMT_MXFP4:
        x = _mx_fake(x.astype(np.float32))
    x = x * x_scale
    z = W13 @ x
    up, gate = (z[N:], z[:N]) if gate_up else (z[:N], z[N:])
    if limit is not None:
        gate = np.minimum(gate, limit)
        up = np.clip(up, -limit, limit)
    h = act(gate, up)
    if fmt == O.FMT_MXFP4:
        h = np.concatenate([_mx_fake(h[i:i + 32].astype(np.float32)) for i in range(0, N, 32)])
    else:
        h = _bf16(h)
    return W2 @ h


def moe(prob, gate_up=False, weight_on_input=False, act=silu_mul):
    c = prob.cfg
    T = prob.x.shape[0]
    acc = np.zeros((T, c.K))
    for t in range(T):
        for j in range(c.topk):
            gid = int(prob.ids[t, j])
            if gid < 0 or gid >= c.E:
                continue
            for tier in prob.tiers:
                e = gid if tier.emap is None else int(tier.emap[gid])
                if 0 <= e < tier.E:
                    w = float(prob.wts[t, j])
                    if weight_on_input:
                        acc[t] += expert_mlp(tier.fmt, tier.weights, e, prob.x[t], c.K, c.N, c.limit, gate_up, w,
                                             act)
                    else:
                        acc[t] += w * expert_mlp(tier.fmt, tier.weights, e, prob.x[t], c.K, c.N, c.limit, gate_up,
                                                 1.0, act)
                    break
    return acc
