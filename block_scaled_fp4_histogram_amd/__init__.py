"""Routed mixture-of-experts with block-scaled 4-bit expert weights on MI355X (gfx950).

Python front end of the C ABI in include/moe.h. PyTorch supplies device memory
and streams; the library's HIP kernels do every step of the layer:

    plan = Plan(E, K, N, top_k, swiglu_limit=7.0, act_format=A_MXFP8, max_tokens=4096)
    experts = Experts(plan, W_MXFP4, E, w13, s13, w2, s2)      # in-place repack
    run(plan, [experts], x, topk_ids, topk_weights, out, deterministic=False)
"""
from __future__ import annotations

import ctypes as C
import math
import os
from typing import Optional, Sequence

from . import _lib

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOTPREPARED, MOE_ESCRATCH, MOE_EHIP = 0, -1, -2, -3, -4, -5
W_MXFP4, W_NVFP4, W_NF3 = 1, 2, 3
A_MXFP8, A_BF16 = 1, 2
W13_UP_GATE, W13_GATE_UP = 0, 1
ACT_SWIGLU, ACT_SITU, ACT_RELU2_NO_MUL = 0, 1, 2
SEQ_AUTO, SEQ_DECODE, SEQ_GENERAL, SEQ_PREFILL, SEQ_PREFILL_NARROW = 0, 1, 2, 3, 4
COMBINE_AUTO, COMBINE_ATOMIC, COMBINE_ROUTE_BUFFER = 0, 1, 2
# race slots of the autotuner: (sequence, combine of deterministic = 0 runs)
RACE_SLOTS = (("decode", None), ("general", "atomic"), ("general", "route_buffer"), ("prefill", "atomic"),
              ("prefill", "route_buffer"), ("prefill_narrow", "atomic"), ("prefill_narrow", "route_buffer"))
NSLOTS = len(RACE_SLOTS)


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, _lib.load().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, name, dtype, device=True, shape=None, numel=None):
    """Dtype, contiguity and device of a tensor the C ABI receives as a raw pointer,
    and its shape or element count: the library cannot check those itself."""
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def weight_bytes(weight_format: int, num_experts: int, K: int, N: int, w13_rows: Optional[int] = None):
    """Bytes of (w13, s13, w2, s2) in the checkpoint layout of include/moe.h for
    num_experts experts: w13 [E, 2N, K] and w2 [E, K, N] codes with their block scales."""
    rows13 = 2 * N if w13_rows is None else w13_rows
    if weight_format == W_MXFP4:
        code, sblk = (lambda n: n // 2), 32
    elif weight_format == W_NVFP4:
        code, sblk = (lambda n: n // 2), 16
    elif weight_format == W_NF3:
        code, sblk = (lambda n: n // 8 * 3), 32
    else:
        raise ValueError(f"unknown weight format {weight_format}")
    E = num_experts
    return (E * rows13 * code(K), E * rows13 * (K // sblk), E * K * code(N), E * K * (N // sblk))


class Plan:
    """One layer geometry (moe_plan)."""

    def __init__(self, E: int, K: int, N: int, top_k: int, swiglu_limit: Optional[float] = None,
                 act_format: int = A_MXFP8, w13_layout: int = W13_UP_GATE, max_tokens: int = 4096):
        L = _lib.load()
        h = C.c_void_p()
        lim = math.nan if swiglu_limit is None else float(swiglu_limit)
        _check(L.moe_plan(E, K, N, top_k, lim, act_format, w13_layout, max_tokens, C.byref(h)))
        self.handle = h
        self.E, self.K, self.N, self.top_k = E, K, N, top_k
        self.act_format, self.w13_layout, self.max_tokens = act_format, w13_layout, max_tokens
        self.act = ACT_SWIGLU

    def scratch_bytes(self, T: int, deterministic: bool = False) -> int:
        return _lib.load().moe_scratch_bytes(self.handle, T, int(bool(deterministic)))

    def capacity(self, T: int):
        rows = C.c_int(0)
        cap = _lib.load().moe_plan_capacity(self.handle, T, C.byref(rows))
        return cap, rows.value

    def set_sequence(self, tokens: int, seq: int):
        """Pin the rung a batch of `tokens` runs at to a launch sequence (SEQ_AUTO: the ladder's choice)."""
        _check(_lib.load().moe_plan_set_sequence(self.handle, int(tokens), int(seq)))

    def sequence(self, tokens: int) -> int:
        """The launch sequence a batch of `tokens` runs with (SEQ_DECODE / SEQ_GENERAL / SEQ_PREFILL /
        SEQ_PREFILL_NARROW)."""
        return _lib.load().moe_plan_sequence(self.handle, int(tokens))

    def set_combine(self, tokens: int, combine: int):
        """Pin the combine of deterministic = 0 runs at the rung of `tokens` (COMBINE_*)."""
        _check(_lib.load().moe_plan_set_combine(self.handle, int(tokens), int(combine)))

    def combine(self, tokens: int) -> int:
        """COMBINE_ATOMIC or COMBINE_ROUTE_BUFFER: how a deterministic = 0 batch of `tokens` combines."""
        return _lib.load().moe_plan_combine(self.handle, int(tokens))

    def autotune(self, tiers, tokens, deterministic: bool = False, reps: int = 5, stream=None):
        """Race, at the rung of each batch size in `tokens`, the eligible (sequence, combine) pairs on a
        synthetic batch and pin the fastest; returns [len(tokens)][7] median microseconds in RACE_SLOTS
        order (NaN where not raced)."""
        tok = [int(t) for t in tokens]
        arr, keep = _tiers(tiers, self)
        ta = (C.c_int * len(tok))(*tok)
        us = (C.c_float * (NSLOTS * len(tok)))()
        _check(_lib.load().moe_plan_autotune(self.handle, arr, len(tiers), ta, len(tok), int(bool(deterministic)),
                                             int(reps), _stream(stream), us))
        return [[us[NSLOTS * i + k] for k in range(NSLOTS)] for i in range(len(tok))]

    def autotune_batch(self, tiers, x, topk_ids, topk_weights, deterministic: bool = False, reps: int = 5,
                       stream=None):
        """The same race at the rung of x's batch, on this batch itself (its own routing); returns the
        7 median times in RACE_SLOTS order."""
        import torch
        T = x.shape[0]
        for device in (False, True):
            _need(x, "x", torch.bfloat16, device, shape=(T, self.K))
            _need(topk_ids, "topk_ids", torch.int32, device, shape=(T, self.top_k))
            _need(topk_weights, "topk_weights", torch.float32, device, shape=(T, self.top_k))
        arr, keep = _tiers(tiers, self)
        us = (C.c_float * NSLOTS)()
        _check(_lib.load().moe_plan_autotune_batch(self.handle, arr, len(tiers), _ptr(x), _ptr(topk_ids),
                                                   _ptr(topk_weights), T, int(bool(deterministic)), int(reps),
                                                   _stream(stream), us))
        return [us[k] for k in range(NSLOTS)]

    def save_tuning(self, path: str):
        _check(_lib.load().moe_plan_save_tuning(self.handle, os.fsencode(path)))

    def load_tuning(self, path: str) -> int:
        """Pin the rungs the file holds for this geometry; returns how many were applied."""
        n = _lib.load().moe_plan_load_tuning(self.handle, os.fsencode(path))
        _check(min(n, 0))
        return n

    def set_swiglu_oai(self, alpha: float, beta: float):
        """Activation gate * sigmoid(alpha gate) * (up + beta) after the clamps (bf16 plans; 1, 0 = plain)."""
        _check(_lib.load().moe_plan_set_swiglu_oai(self.handle, float(alpha), float(beta)))

    def set_activation(self, act: int):
        """ACT_SWIGLU (default), ACT_SITU (silu(4 tanh(gate/4)) * 25 tanh(up/25)) or ACT_RELU2_NO_MUL
        (relu(z)^2 of a w13 with N rows; bf16 plans); SiTU and ReLU^2 on plans without a limit.
        Set before preparing experts for the plan."""
        _check(_lib.load().moe_plan_set_activation(self.handle, int(act)))
        self.act = int(act)

    def set_router_weight_on_input(self, enable: bool = True):
        """Apply each slot's router weight to GEMM1's input instead of the GEMM2 result (bf16 plans)."""
        _check(_lib.load().moe_plan_set_router_weight_on_input(self.handle, int(bool(enable))))

    def enable_stage_timing(self, max_runs: int):
        """Record HIP events between the layer's stages for the next max_runs runs."""
        _check(_lib.load().moe_plan_enable_stage_timing(self.handle, max_runs))

    def stage_times(self):
        """Summed ms of (route, gemm1, gemm2, combine) over the recorded runs, and the run count."""
        ms = (C.c_float * 4)()
        runs = C.c_int(0)
        _check(_lib.load().moe_plan_stage_times(self.handle, ms, 4, C.byref(runs)))
        return [float(v) for v in ms], runs.value

    def close(self):
        if self.handle:
            _lib.load().moe_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Experts:
    """One layer's (or tier's) experts, repacked in place (moe_prepare_weights).

    The tensors are borrowed: they hold the tile layout until unpack().  For MXFP4 the
    handle also owns device copies of s13 and s2 in the prefill GEMMs' order, freed by
    unpack() or when the handle is destroyed."""

    def __init__(self, plan: Plan, weight_format: int, num_experts: int, w13, s13, w2, s2, g13=None, g2=None,
                 stream=None):
        import torch
        sizes = weight_bytes(weight_format, num_experts, plan.K, plan.N,
                             plan.N if plan.act == ACT_RELU2_NO_MUL else None)
        for device in (False, True):   # every size first, then where the tensors live
            for name, t, n in zip(("w13", "s13", "w2", "s2"), (w13, s13, w2, s2), sizes):
                _need(t, name, torch.uint8, device, numel=n)
            for name, t in (("g13", g13), ("g2", g2)):
                if t is not None:
                    _need(t, name, torch.float32, device, numel=num_experts)
        h = C.c_void_p()
        _check(_lib.load().moe_prepare_weights(plan.handle, weight_format, num_experts, _ptr(w13), _ptr(s13),
                                               _ptr(g13), _ptr(w2), _ptr(s2), _ptr(g2), _stream(stream),
                                               C.byref(h)))
        self.handle = h
        self.plan = plan
        self.weight_format, self.num_experts = weight_format, num_experts
        self.tensors = (w13, s13, w2, s2, g13, g2)

    def unpack(self, stream=None):
        _check(_lib.load().moe_unpack_weights(self.handle, _stream(stream)))

    def close(self):
        if self.handle:
            _lib.load().moe_experts_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _tiers(tiers, plan=None):
    arr = (_lib.MoeTier * len(tiers))()
    keep = []
    for i, t in enumerate(tiers):
        ex, emap = (t if isinstance(t, (tuple, list)) else (t, None))
        if emap is not None:
            import torch
            _need(emap, "expert_map", torch.int32, numel=None if plan is None else plan.E)
        keep.append(emap)
        arr[i] = _lib.MoeTier(ex.handle.value, _ptr(emap))
    return arr, keep


def scratch_for(plan: Plan, T: int, deterministic: bool = False, device="cuda"):
    """A scratch tensor large enough for moe_run of T tokens."""
    import torch
    return torch.empty(max(plan.scratch_bytes(T, deterministic), 256), dtype=torch.uint8, device=device)


def run(plan: Plan, tiers: Sequence, x, topk_ids, topk_weights, out=None, deterministic: bool = False,
        scratch=None, stream=None):
    """The layer (moe_run). tiers: Experts, or (Experts, expert_map int32 [E]) pairs."""
    import torch
    if x is None or x.dim() != 2:
        raise ValueError("x must be a [T, K] tensor")
    T = x.shape[0]
    for device in (False, True):   # every shape first, then where the tensors live
        _need(x, "x", torch.bfloat16, device, shape=(T, plan.K))
        _need(topk_ids, "topk_ids", torch.int32, device, shape=(T, plan.top_k))
        _need(topk_weights, "topk_weights", torch.float32, device, shape=(T, plan.top_k))
        if out is not None:
            _need(out, "out", torch.bfloat16, device, shape=(T, plan.K))
    if out is None:
        out = torch.empty_like(x)
    if scratch is None:
        scratch = scratch_for(plan, T, deterministic, x.device)
    _need(scratch, "scratch", torch.uint8)
    arr, keep = _tiers(tiers, plan)
    _check(_lib.load().moe_run(plan.handle, arr, len(tiers), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                               _ptr(out), T, int(bool(deterministic)), _ptr(scratch), scratch.numel(),
                               _stream(stream)))
    return out


def run_noalloc(plan: Plan, tiers: Sequence, x, topk_ids, topk_weights, out, deterministic: bool = False,
                stream=None):
    """The layer with the library's static 64 MiB device arena as scratch (moe_run_noalloc):
    no device allocation by the library or here (out must be given)."""
    import torch
    if x is None or x.dim() != 2:
        raise ValueError("x must be a [T, K] tensor")
    T = x.shape[0]
    for device in (False, True):
        _need(x, "x", torch.bfloat16, device, shape=(T, plan.K))
        _need(topk_ids, "topk_ids", torch.int32, device, shape=(T, plan.top_k))
        _need(topk_weights, "topk_weights", torch.float32, device, shape=(T, plan.top_k))
        _need(out, "out", torch.bfloat16, device, shape=(T, plan.K))
    arr, keep = _tiers(tiers, plan)
    _check(_lib.load().moe_run_noalloc(plan.handle, arr, len(tiers), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                       _ptr(out), T, int(bool(deterministic)), _stream(stream)))
    return out


def ep_remap(topk_ids, topk_weights, offset: int, num_local: int, out_ids=None, out_weights=None, stream=None):
    """Expert-parallel id remap (moe_ep_remap): global top-k ids of [T, k] -> this rank's
    local ids for experts [offset, offset + num_local); other slots get weight 0 and an
    expert the batch already reads. Returns (out_ids int32, out_weights fp32)."""
    import torch
    if topk_ids is None or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be a [T, k] tensor")
    T, k = topk_ids.shape
    if out_ids is None:
        out_ids = torch.empty_like(topk_ids)
    if out_weights is None:
        out_weights = torch.empty((T, k), dtype=torch.float32, device=topk_ids.device)
    for device in (False, True):
        _need(topk_ids, "topk_ids", torch.int32, device, shape=(T, k))
        _need(topk_weights, "topk_weights", torch.float32, device, shape=(T, k))
        _need(out_ids, "out_ids", torch.int32, device, shape=(T, k))
        _need(out_weights, "out_weights", torch.float32, device, shape=(T, k))
    _check(_lib.load().moe_ep_remap(_ptr(topk_ids), _ptr(topk_weights), T, k, int(offset), int(num_local),
                                    _ptr(out_ids), _ptr(out_weights), _stream(stream)))
    return out_ids, out_weights


def debug_route(plan: Plan, tiers: Sequence, topk_ids, scratch=None, stream=None):
    """Route planner alone. Returns (cnt [U], off [U+1], perm [off[U]], inv [T*k]) device tensors."""
    import torch
    if topk_ids is None or topk_ids.dim() != 2 or topk_ids.shape[1] != plan.top_k:
        raise ValueError(f"topk_ids must be a [T, {plan.top_k}] tensor")
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    U = sum((t[0] if isinstance(t, (tuple, list)) else t).num_experts for t in tiers)
    dev = topk_ids.device
    if scratch is None:
        scratch = scratch_for(plan, T, True, dev)
    cnt = torch.empty(U, dtype=torch.int32, device=dev)
    off = torch.empty(U + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    arr, keep = _tiers(tiers, plan)
    _check(_lib.load().moe_debug_route(plan.handle, arr, len(tiers), _ptr(topk_ids), T, _ptr(scratch),
                                       scratch.numel(), _ptr(cnt), _ptr(off), _ptr(perm), _ptr(inv),
                                       _stream(stream)))
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return cnt, off, perm[: int(off[-1].item())], inv


def debug_quant_mxfp8(v, stream=None):
    """MXFP8 quantiser alone on a [rows, cols] bf16 or fp32 device tensor -> (codes, scales)."""
    import torch
    if v.dtype not in (torch.bfloat16, torch.float32) or not v.is_contiguous():
        raise TypeError("expected a contiguous bf16 or fp32 tensor")
    rows, cols = v.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=v.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=v.device)
    fn = _lib.load().moe_debug_quant_mxfp8_bf16 if v.dtype == torch.bfloat16 else _lib.load().moe_debug_quant_mxfp8_f32
    _check(fn(_ptr(v), rows, cols, _ptr(q), _ptr(s), _stream(stream)))
    return q, s
