"""Seeded synthetic inputs for the routed-MoE layer, shared by the tests, the
oracle's callers and the benchmark.

This module draws random numbers and lays them out in the checkpoint formats
the pages describe; it holds none of the layer's arithmetic (no decode, no
quantisation of activations, no GEMM). Every tensor comes from its own stream
``numpy.random.default_rng([seed, tensor_id])`` so that any one tensor can be
regenerated without the others.

Shapes follow the pages' workloads:

* W4A8, DeepSeek-V4.1 slice (sglang ``moe_b12x_next.py``, module docstring):
  384 experts, intermediate slice N=576 per TP4 rank, top-6; w13 stacked
  [up; gate] (same docstring, "load_up_proj_weight_first"). Checkpoint
  tensors per ``_convert_layer``: w13 [E,2N,K/2] u8 (two E2M1 codes per byte),
  w13 scales [E,2N,K/32] E8M0, w2 [E,K,N/2], w2 scales [E,K,N/32].
* W4A16 / W3A16, GLM-5.2 hybrid (vLLM ``hybrid_loader.py``, ``create_weights``
  and ``_unpack_nf3``): 256 experts, hidden 6144, intermediate 512, top-8;
  NVFP4 = E2M1 + E4M3 per-16 scales + fp32 per-expert global; NF3 = 3-bit
  codes, 8 per 3 bytes, E4M3 per-32 scales.

The hidden size 7168 of the W4A8 workloads and every value distribution are
this module's choices (the pages print neither); they are listed with the
tensor-id table in the design notes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# tensor ids of the per-tensor random streams
TID_X, TID_LOGITS, TID_W13, TID_S13, TID_W2, TID_S2, TID_GLOBAL, TID_ZIPF, TID_TIER = range(9)
TID_TIER_B_OFFSET = 16  # second tier's weight streams: TID_W13 + 16, ...

FMT_MXFP4 = 1  # E2M1 + E8M0 per 32, MXFP8 activations (W4A8)
FMT_NVFP4 = 2  # E2M1 + E4M3 per 16 + fp32 global, bf16 activations (W4A16)
FMT_NF3 = 3    # 3-bit codebook + E4M3 per 32, bf16 activations (W3A16)


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid])


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    E: int
    K: int
    N: int
    topk: int
    limit: Optional[float]          # SwiGLU clamp; None = no clamp
    fmt: int                        # weight format of the (first) tier
    pad_rows: int = 0               # trailing rows whose ids are all -1
    e8m0_exp: tuple = (-4, 0)       # MXFP4 scale exponent range (inclusive)
    zipf_s: Optional[float] = None  # per-expert logit bias -s*ln(rank)
    hybrid_nvfp4: int = 0           # >0: that many experts NVFP4, the rest NF3


CONFIGS = {
    # tiny W4A8 layer, the case the oracle finishes instantly
    "tiny": Config("tiny", T=4, E=8, K=256, N=128, topk=2, limit=7.0, fmt=FMT_MXFP4),
    # one TP4 rank's decode step: 8 rows, the last two CUDA-graph padding rows
    "decode": Config("decode", T=8, E=384, K=7168, N=576, topk=6, limit=7.0, fmt=FMT_MXFP4,
                     pad_rows=2, e8m0_exp=(-9, -5)),
    # prefill on the same geometry with Zipf-skewed expert loads
    "prefill": Config("prefill", T=4096, E=384, K=7168, N=576, topk=6, limit=7.0, fmt=FMT_MXFP4,
                      e8m0_exp=(-9, -5), zipf_s=1.1),
    # NVFP4 W4A16, decode- and prefill-sized batches
    "nvfp4_decode": Config("nvfp4_decode", T=8, E=256, K=6144, N=512, topk=8, limit=None, fmt=FMT_NVFP4),
    "nvfp4_prefill": Config("nvfp4_prefill", T=2048, E=256, K=6144, N=512, topk=8, limit=None, fmt=FMT_NVFP4),
    # hybrid: 64 NVFP4 experts + 192 NF3 experts, one shared id space of 256
    "hybrid": Config("hybrid", T=2048, E=256, K=6144, N=512, topk=8, limit=None, fmt=FMT_NVFP4,
                     hybrid_nvfp4=64),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (input preparation only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def make_x(T: int, K: int, seed: int = 0) -> np.ndarray:
    """Activations: fp32 N(0,1) rounded to bf16; returned as uint16 bit patterns [T,K]."""
    return bf16_bits_from_f32(_rng(seed, TID_X).standard_normal((T, K), dtype=np.float32))


def make_routing(T: int, E: int, topk: int, seed: int = 0, zipf_s: Optional[float] = None,
                 pad_rows: int = 0):
    """Router output: ids = top-k of N(0,1) logits (+ optional Zipf bias), descending,
    ties to the lower id; weights = softmax over the k selected logits.

    Returns (ids int32 [T,k], weights float32 [T,k]). Padding rows get ids -1 and keep
    non-zero weights, so a kernel that failed to skip them would show it.
    """
    logits = _rng(seed, TID_LOGITS).standard_normal((T, E))
    if zipf_s is not None:
        rank = _rng(seed, TID_ZIPF).permutation(E) + 1
        logits = logits + (-zipf_s * np.log(rank))[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(logits, order, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    ids = order.astype(np.int32)
    if pad_rows:
        ids[T - pad_rows:, :] = -1
    return np.ascontiguousarray(ids), np.ascontiguousarray(w.astype(np.float32))


def _bytes(seed, tid, shape):
    return _rng(seed, tid).integers(0, 256, size=shape, dtype=np.uint8)


def make_mxfp4(E: int, K: int, N: int, seed: int = 0, exp_range=(-4, 0), tid_offset: int = 0):
    """MXFP4 checkpoint tensors. E2M1 codes uniform over 16 values (so packed bytes are
    uniform over 256); E8M0 bytes 127+u, u uniform in exp_range (inclusive)."""
    lo, hi = exp_range
    w13 = _bytes(seed, TID_W13 + tid_offset, (E, 2 * N, K // 2))
    s13 = (127 + _rng(seed, TID_S13 + tid_offset).integers(lo, hi + 1, size=(E, 2 * N, K // 32))).astype(np.uint8)
    w2 = _bytes(seed, TID_W2 + tid_offset, (E, K, N // 2))
    s2 = (127 + _rng(seed, TID_S2 + tid_offset).integers(lo, hi + 1, size=(E, K, N // 32))).astype(np.uint8)
    return dict(w13=w13, s13=s13, g13=None, w2=w2, s2=s2, g2=None)


# E4M3 scale bytes 0x18..0x3F: the 40 positive normal codes with exponent -4..0
_E4M3_SCALE_LO, _E4M3_SCALE_HI = 0x18, 0x3F


def _e4m3_scales(seed, tid, shape):
    return _rng(seed, tid).integers(_E4M3_SCALE_LO, _E4M3_SCALE_HI + 1, size=shape).astype(np.uint8)


def make_nvfp4(E: int, K: int, N: int, seed: int = 0, tid_offset: int = 0):
    """NVFP4 checkpoint tensors: uniform E2M1 codes, E4M3 per-16 scales, fp32 globals U(0.5, 2)."""
    w13 = _bytes(seed, TID_W13 + tid_offset, (E, 2 * N, K // 2))
    s13 = _e4m3_scales(seed, TID_S13 + tid_offset, (E, 2 * N, K // 16))
    w2 = _bytes(seed, TID_W2 + tid_offset, (E, K, N // 2))
    s2 = _e4m3_scales(seed, TID_S2 + tid_offset, (E, K, N // 16))
    g = _rng(seed, TID_GLOBAL + tid_offset).uniform(0.5, 2.0, size=(2, E)).astype(np.float32)
    return dict(w13=w13, s13=s13, g13=np.ascontiguousarray(g[0]), w2=w2, s2=s2, g2=np.ascontiguousarray(g[1]))


def make_nf3(E: int, K: int, N: int, seed: int = 0, tid_offset: int = 0):
    """NF3 checkpoint tensors: codes uniform over 8 values packed 8 per 3 bytes (24 uniform
    bits, hence uniform bytes); E4M3 per-32 scales."""
    w13 = _bytes(seed, TID_W13 + tid_offset, (E, 2 * N, K // 8 * 3))
    s13 = _e4m3_scales(seed, TID_S13 + tid_offset, (E, 2 * N, K // 32))
    w2 = _bytes(seed, TID_W2 + tid_offset, (E, K, N // 8 * 3))
    s2 = _e4m3_scales(seed, TID_S2 + tid_offset, (E, K, N // 32))
    return dict(w13=w13, s13=s13, g13=None, w2=w2, s2=s2, g2=None)


def make_weights(fmt: int, E: int, K: int, N: int, seed: int = 0, exp_range=(-4, 0), tid_offset: int = 0):
    if fmt == FMT_MXFP4:
        return make_mxfp4(E, K, N, seed, exp_range, tid_offset)
    if fmt == FMT_NVFP4:
        return make_nvfp4(E, K, N, seed, tid_offset)
    if fmt == FMT_NF3:
        return make_nf3(E, K, N, seed, tid_offset)
    raise ValueError(f"unknown weight format {fmt}")


def make_tier_split(E: int, n_first: int, seed: int = 0):
    """Hybrid tier maps: a seeded sample of n_first global ids (sorted ascending) forms
    tier A, the rest tier B; local ids ascend with the global id. Returns (emap_a, emap_b)
    int32 [E] with -1 where the id belongs to the other tier."""
    sel = np.sort(_rng(seed, TID_TIER).choice(E, size=n_first, replace=False))
    in_a = np.zeros(E, dtype=bool)
    in_a[sel] = True
    emap_a = np.full(E, -1, dtype=np.int32)
    emap_b = np.full(E, -1, dtype=np.int32)
    emap_a[in_a] = np.arange(n_first, dtype=np.int32)
    emap_b[~in_a] = np.arange(E - n_first, dtype=np.int32)
    return emap_a, emap_b


@dataclasses.dataclass
class Tier:
    fmt: int
    E: int
    weights: dict
    emap: Optional[np.ndarray] = None


@dataclasses.dataclass
class Problem:
    cfg: Config
    x: np.ndarray          # uint16 bf16 bits [T,K]
    ids: np.ndarray        # int32 [T,k]
    wts: np.ndarray        # float32 [T,k]
    tiers: list


def make_problem(cfg: Config | str, seed: int = 0, T: Optional[int] = None) -> Problem:
    """Full synthetic layer for a named workload (optionally with another token count)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T, pad_rows=min(cfg.pad_rows, T))
    x = make_x(cfg.T, cfg.K, seed)
    ids, wts = make_routing(cfg.T, cfg.E, cfg.topk, seed, cfg.zipf_s, cfg.pad_rows)
    if cfg.hybrid_nvfp4:
        ea, eb = make_tier_split(cfg.E, cfg.hybrid_nvfp4, seed)
        na, nb = cfg.hybrid_nvfp4, cfg.E - cfg.hybrid_nvfp4
        tiers = [Tier(FMT_NVFP4, na, make_nvfp4(na, cfg.K, cfg.N, seed), ea),
                 Tier(FMT_NF3, nb, make_nf3(nb, cfg.K, cfg.N, seed, TID_TIER_B_OFFSET), eb)]
    else:
        tiers = [Tier(cfg.fmt, cfg.E, make_weights(cfg.fmt, cfg.E, cfg.K, cfg.N, seed, cfg.e8m0_exp))]
    return Problem(cfg, x, ids, wts, tiers)
