"""The C-ABI library on the CPU: it loads, exports every function include/moe.h
declares, and its host-side validation returns the documented codes. No call
here launches GPU work."""
import ctypes as C
import math
import os
import re

import pytest

import block_scaled_fp4_histogram_amd as M
from block_scaled_fp4_histogram_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = _lib.load()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures and header disagree"


def test_plan_validation_codes():
    ok = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert ok.scratch_bytes(8) > 0
    bad = [((384, 7000, 576, 6), M.MOE_EUNSUPPORTED),   # K % 256
           ((384, 7168, 570, 6), M.MOE_EUNSUPPORTED),   # N % 32
           ((0, 7168, 576, 6), M.MOE_EUNSUPPORTED),
           ((2000, 7168, 576, 6), M.MOE_EUNSUPPORTED),
           ((384, 7168, 576, 0), M.MOE_EINVAL),
           ((384, 7168, 576, 17), M.MOE_EINVAL)]
    for args, code in bad:
        with pytest.raises(M.MoeError) as ei:
            M.Plan(*args)
        assert ei.value.code == code, args
        assert str(ei.value)  # carries the library's message
    with pytest.raises(M.MoeError) as ei:
        M.Plan(8, 256, 128, 2, None, act_format=7)
    assert ei.value.code == M.MOE_EUNSUPPORTED
    with pytest.raises(M.MoeError) as ei:
        M.Plan(8, 256, 128, 2, None, w13_layout=5)
    assert ei.value.code == M.MOE_EINVAL


def test_capacity_ladder_and_scratch_sizes():
    p = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert p.capacity(1)[0] == 1
    assert p.capacity(6)[0] == 6
    assert p.capacity(9)[0] == 10
    assert p.capacity(100)[0] == 128
    assert p.capacity(4096)[0] == 4096
    assert p.capacity(10000)[0] == 4096          # chunks of the top rung
    # route tile rows of the launch sequence: decode (T <= 16, <= 64 routes) has none
    assert p.capacity(8)[1] == 0
    assert p.capacity(11)[1] == 16                # 66 routes: general kernels
    assert p.capacity(4096)[1] == 64              # prefill (N % 64 == 0)
    q = M.Plan(8, 256, 96, 2, None, M.A_MXFP8, max_tokens=512)
    assert q.capacity(512)[1] == 16               # N % 64 != 0: general kernels
    sizes = [p.scratch_bytes(t) for t in (1, 8, 64, 512, 4096)]
    assert sizes == sorted(sizes)
    assert p.scratch_bytes(10000) == p.scratch_bytes(4096)
    assert p.scratch_bytes(128, True) > p.scratch_bytes(128, False)     # route buffer vs accumulator (general)
    # the prefill sequence combines through the route buffer in both modes (the ladder's choice)
    assert p.scratch_bytes(4096, True) == p.scratch_bytes(4096, False)
    assert p.scratch_bytes(8) % 256 == 0
    L = _lib.load()
    assert L.moe_scratch_bytes(None, 8, 0) == 0


def test_null_and_bad_handles_are_refused_on_the_host():
    L = _lib.load()
    p = M.Plan(8, 256, 128, 2, 7.0, M.A_MXFP8, max_tokens=16)
    h = C.c_void_p()
    # weight format that does not fit the plan's activation format
    rc = L.moe_prepare_weights(p.handle, M.W_NVFP4, 8, 16, 16, None, 16, 16, None, None, C.byref(h))
    assert rc == M.MOE_EUNSUPPORTED
    rc = L.moe_prepare_weights(p.handle, 9, 8, 16, 16, None, 16, 16, None, None, C.byref(h))
    assert rc == M.MOE_EUNSUPPORTED
    rc = L.moe_prepare_weights(p.handle, M.W_MXFP4, 8, None, 16, None, 16, 16, None, None, C.byref(h))
    assert rc == M.MOE_EINVAL
    rc = L.moe_prepare_weights(p.handle, M.W_MXFP4, 8, 17, 16, None, 16, 16, None, None, C.byref(h))
    assert rc == M.MOE_EINVAL                                       # misaligned
    rc = L.moe_prepare_weights(None, M.W_MXFP4, 8, 16, 16, None, 16, 16, None, None, C.byref(h))
    assert rc == M.MOE_EINVAL
    # moe_run with no tiers / a null experts handle
    tiers = (_lib.MoeTier * 1)()
    rc = L.moe_run(p.handle, tiers, 1, 256, 256, 256, 256, 4, 0, 256, 1 << 20, None)
    assert rc == M.MOE_EINVAL
    rc = L.moe_run(p.handle, tiers, 0, 256, 256, 256, 256, 4, 0, 256, 1 << 20, None)
    assert rc == M.MOE_EINVAL
    rc = L.moe_run(None, tiers, 1, 256, 256, 256, 256, 4, 0, 256, 1 << 20, None)
    assert rc == M.MOE_EINVAL
    assert L.moe_last_error().decode() != ""
    # stage timing on a bad plan; debug quantiser shape checks
    assert L.moe_plan_enable_stage_timing(None, 4) == M.MOE_EINVAL
    assert L.moe_debug_quant_mxfp8_f32(16, 4, 33, 16, 16, None) == M.MOE_EINVAL
    assert L.moe_debug_quant_mxfp8_f32(16, 0, 32, 16, 16, None) == M.MOE_OK   # empty is a no-op


def test_destroy_is_safe_on_null():
    L = _lib.load()
    L.moe_plan_destroy(None)
    L.moe_experts_destroy(None)


def test_router_weight_on_input_needs_bf16_activations():
    a8 = M.Plan(8, 256, 128, 2, 7.0, M.A_MXFP8, max_tokens=16)
    with pytest.raises(RuntimeError) as e:
        a8.set_router_weight_on_input(True)
    assert "bf16" in str(e.value)
    a8.set_router_weight_on_input(False)   # the default stays accepted
    a16 = M.Plan(8, 256, 128, 2, None, M.A_BF16, max_tokens=16)
    a16.set_router_weight_on_input(True)
    a16.set_router_weight_on_input(False)


def test_swiglu_oai_needs_bf16_activations():
    a8 = M.Plan(8, 256, 128, 2, 7.0, M.A_MXFP8, max_tokens=16)
    with pytest.raises(RuntimeError) as e:
        a8.set_swiglu_oai(1.702, 1.0)
    assert "bf16" in str(e.value)
    a8.set_swiglu_oai(1.0, 0.0)   # the plain form stays accepted
    a16 = M.Plan(8, 256, 128, 2, 7.0, M.A_BF16, max_tokens=16)
    a16.set_swiglu_oai(1.702, 1.0)
    with pytest.raises(RuntimeError):
        a16.set_swiglu_oai(float("nan"), 1.0)
    with pytest.raises(RuntimeError):
        a16.set_swiglu_oai(1.0, float("inf"))


def test_sequence_pins_and_tuning_file(tmp_path):
    p = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert p.sequence(8) == M.SEQ_DECODE
    assert p.sequence(64) == M.SEQ_GENERAL
    assert p.sequence(4096) == M.SEQ_PREFILL
    p.set_sequence(8, M.SEQ_GENERAL)
    assert p.sequence(8) == M.SEQ_GENERAL and p.capacity(8)[1] == 16
    assert p.sequence(7) == M.SEQ_DECODE              # another rung
    p.set_sequence(64, M.SEQ_PREFILL)
    assert p.sequence(50) == M.SEQ_PREFILL and p.capacity(64)[1] == 64
    with pytest.raises(M.MoeError) as e:
        p.set_sequence(24, M.SEQ_DECODE)              # 24 tokens x 6 slots > 64 routes
    assert e.value.code == M.MOE_EUNSUPPORTED
    with pytest.raises(M.MoeError) as e:
        p.set_sequence(8, 7)
    assert e.value.code == M.MOE_EINVAL
    path = str(tmp_path / "tuning.txt")
    other = M.Plan(8, 256, 96, 2, None, M.A_MXFP8, max_tokens=512)
    with pytest.raises(M.MoeError) as e:
        other.set_sequence(512, M.SEQ_PREFILL)        # N % 64 != 0
    assert e.value.code == M.MOE_EUNSUPPORTED
    other.set_sequence(4, M.SEQ_GENERAL)
    other.save_tuning(path)
    p.save_tuning(path)                               # keeps the other geometry's line
    fresh = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert fresh.load_tuning(path) == 2
    assert fresh.sequence(8) == M.SEQ_GENERAL and fresh.sequence(64) == M.SEQ_PREFILL
    assert fresh.sequence(4096) == M.SEQ_PREFILL
    o2 = M.Plan(8, 256, 96, 2, None, M.A_MXFP8, max_tokens=512)
    assert o2.load_tuning(path) == 1 and o2.sequence(4) == M.SEQ_GENERAL
    p.set_sequence(8, M.SEQ_AUTO)
    assert p.sequence(8) == M.SEQ_DECODE
    p.save_tuning(path)                               # rewrites this geometry's lines only
    again = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert again.load_tuning(path) == 1 and again.sequence(8) == M.SEQ_DECODE
    with pytest.raises(M.MoeError):
        again.load_tuning(str(tmp_path / "missing.txt"))


def test_wrapper_refuses_mis_shaped_tensors_before_the_library_sees_them():
    """The C ABI takes raw pointers and cannot check sizes: the Python wrapper checks
    every tensor against the plan's geometry first (CPU tensors: refused at the shape
    check, before the device check)."""
    import torch
    p = M.Plan(8, 256, 128, 2, 7.0, M.A_MXFP8, max_tokens=16)
    w13, s13, w2, s2 = (torch.zeros(n, dtype=torch.uint8) for n in M.weight_bytes(M.W_MXFP4, 8, 256, 128))
    assert (w13.numel(), s13.numel(), w2.numel(), s2.numel()) == (8 * 256 * 128, 8 * 256 * 8, 8 * 256 * 64,
                                                                   8 * 256 * 4)
    short = torch.zeros(w13.numel() - 1, dtype=torch.uint8)
    for args in ((short, s13, w2, s2), (w13, s13[:-4], w2, s2), (w13, s13, w2, s2[1:])):
        with pytest.raises(ValueError, match="elements"):
            M.Experts(p, M.W_MXFP4, 8, *args)
    with pytest.raises(ValueError, match="elements"):   # globals must hold one value per expert
        M.Experts(p, M.W_MXFP4, 8, w13, s13, w2, s2, g13=torch.ones(7))
    nv = M.weight_bytes(M.W_NVFP4, 3, 512, 64)
    assert nv == (3 * 128 * 256, 3 * 128 * 32, 3 * 512 * 32, 3 * 512 * 4)
    nf = M.weight_bytes(M.W_NF3, 3, 512, 64)
    assert nf == (3 * 128 * 192, 3 * 128 * 16, 3 * 512 * 24, 3 * 512 * 2)

    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    ids = torch.zeros(4, 2, dtype=torch.int32)
    wts = torch.zeros(4, 2, dtype=torch.float32)
    cases = [(torch.zeros(4, 255, dtype=torch.bfloat16), ids, wts, None, "x"),
             (x, torch.zeros(4, 3, dtype=torch.int32), wts, None, "topk_ids"),
             (x, ids, torch.zeros(5, 2, dtype=torch.float32), None, "topk_weights"),
             (x, ids, wts, torch.zeros(3, 256, dtype=torch.bfloat16), "out")]
    for xx, ii, ww, oo, name in cases:
        with pytest.raises(ValueError, match=name):
            M.run(p, [], xx, ii, ww, out=oo, scratch=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="expert_map"):
        M._tiers([(type("E", (), {"handle": C.c_void_p(1)})(), torch.zeros(7, dtype=torch.int32))], p)


def test_combine_pins_follow_the_ladder_scratch_and_tuning_file(tmp_path):
    """deterministic = 0 combines through the route buffer on the prefill sequences and on
    the W4A8 general one from 256 tokens (where a pin puts it), with atomics on the general
    one below unless a rung is pinned; the scratch follows the combine (route buffer 2 R K
    bytes, accumulator 4 T K); pins persist (v2 lines) and sequence-only v1 lines still load."""
    p = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert p.combine(4096) == M.COMBINE_ROUTE_BUFFER and p.combine(100) == M.COMBINE_ATOMIC
    g = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    g.set_sequence(256, M.SEQ_GENERAL)
    assert g.combine(256) == M.COMBINE_ROUTE_BUFFER and g.combine(128) == M.COMBINE_ATOMIC
    assert M.Plan(256, 6144, 512, 8, None, M.A_BF16, max_tokens=4096).combine(256) == M.COMBINE_ATOMIC
    assert p.scratch_bytes(4096, False) == p.scratch_bytes(4096, True)
    atomic_100 = p.scratch_bytes(100, False)
    p.set_combine(100, M.COMBINE_ROUTE_BUFFER)
    assert p.combine(100) == M.COMBINE_ROUTE_BUFFER
    rb_100 = p.scratch_bytes(100, False)
    assert rb_100 - atomic_100 >= 2 * 128 * 6 * 7168 - 4 * 128 * 7168 - 4096
    p.set_combine(4096, M.COMBINE_ATOMIC)
    assert p.combine(4096) == M.COMBINE_ATOMIC and p.scratch_bytes(4096, False) < p.scratch_bytes(4096, True)
    with pytest.raises(M.MoeError) as e:
        p.set_combine(8, 9)
    assert e.value.code == M.MOE_EINVAL
    path = str(tmp_path / "t.txt")
    p.save_tuning(path)
    text = open(path).read()
    assert "moe v2" in text and "comb=2" in text and "comb=1" in text
    q = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert q.load_tuning(path) == 2
    assert q.combine(100) == M.COMBINE_ROUTE_BUFFER and q.combine(4096) == M.COMBINE_ATOMIC
    v1 = str(tmp_path / "v1.txt")
    key = "E=384 K=7168 N=576 topk=6 afmt=1 max_tokens=4096"
    open(v1, "w").write(f"moe v1 {key} cap=8 seq=2\n")
    r = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert r.load_tuning(v1) == 1 and r.sequence(8) == M.SEQ_GENERAL and r.combine(8) == M.COMBINE_ATOMIC


def test_activation_forms_are_validated_on_the_host():
    a8 = M.Plan(8, 256, 128, 2, None, M.A_MXFP8, max_tokens=16)
    a8.set_activation(M.ACT_SITU)                                  # SiTU runs with W4A8
    for plan, code in ((M.Plan(8, 256, 128, 2, None, M.A_MXFP8, max_tokens=16), M.MOE_EUNSUPPORTED),   # W4A8
                       (M.Plan(8, 256, 160, 2, None, M.A_BF16, max_tokens=16), M.MOE_EUNSUPPORTED),    # N % 64
                       (M.Plan(8, 256, 128, 2, 7.0, M.A_BF16, max_tokens=16), M.MOE_EUNSUPPORTED),     # a limit
                       (M.Plan(8, 256, 128, 2, None, M.A_BF16, M.W13_GATE_UP, 16), M.MOE_EUNSUPPORTED)):
        with pytest.raises(M.MoeError) as e:
            plan.set_activation(M.ACT_RELU2_NO_MUL)
        assert e.value.code == code
    with pytest.raises(M.MoeError):
        M.Plan(8, 256, 128, 2, 7.0, M.A_BF16, max_tokens=16).set_activation(M.ACT_SITU)
    with pytest.raises(M.MoeError):
        a8.set_activation(9)
    p = M.Plan(8, 256, 192, 2, None, M.A_BF16, max_tokens=1024)
    p.set_sequence(1024, M.SEQ_PREFILL)
    p.set_activation(M.ACT_RELU2_NO_MUL)               # N = 192: 96 pairs, no prefill kernel
    assert p.sequence(1024) == M.SEQ_GENERAL           # the pin it can no longer take is dropped
    with pytest.raises(M.MoeError):
        p.set_sequence(1024, M.SEQ_PREFILL)
    q = M.Plan(8, 256, 256, 2, None, M.A_BF16, max_tokens=1024)
    q.set_activation(M.ACT_RELU2_NO_MUL)
    q.set_sequence(1024, M.SEQ_PREFILL)
    # the wrapper sizes w13 as N rows under ReLU^2
    import torch
    w13, s13, w2, s2 = (torch.zeros(n, dtype=torch.uint8) for n in M.weight_bytes(M.W_NVFP4, 8, 256, 256, 256))
    assert w13.numel() == 8 * 256 * 128
    with pytest.raises(ValueError, match="device"):    # sizes accepted, then refused for living on the CPU
        M.Experts(q, M.W_NVFP4, 8, w13, s13, w2, s2)
    big = torch.zeros(8 * 512 * 128, dtype=torch.uint8)
    with pytest.raises(ValueError, match="elements"):
        M.Experts(q, M.W_NVFP4, 8, big, s13, w2, s2)


def test_narrow_prefill_sequence_is_a_w4a8_variant(tmp_path):
    p = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    p.set_sequence(4096, M.SEQ_PREFILL_NARROW)
    assert p.sequence(4096) == M.SEQ_PREFILL_NARROW and p.capacity(4096)[1] == 64
    assert p.combine(4096) == M.COMBINE_ROUTE_BUFFER          # a prefill sequence: the ladder's combine
    path = str(tmp_path / "n.txt")
    p.save_tuning(path)
    q = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=4096)
    assert q.load_tuning(path) == 1 and q.sequence(4096) == M.SEQ_PREFILL_NARROW
    a16 = M.Plan(256, 6144, 512, 8, None, M.A_BF16, max_tokens=2048)
    a16.set_sequence(2048, M.SEQ_PREFILL_NARROW)               # 16-bit plans run 128-route up/gate tiles too
    assert a16.sequence(2048) == M.SEQ_PREFILL_NARROW
    odd = M.Plan(256, 6144, 544, 8, None, M.A_BF16, max_tokens=2048)
    with pytest.raises(M.MoeError) as e:
        odd.set_sequence(2048, M.SEQ_PREFILL_NARROW)           # as PREFILL: N % 64 == 0 only
    assert e.value.code == M.MOE_EUNSUPPORTED


def test_ladder_default_sequences():
    """The ladder's own choice per batch size (no pins): decode up to 64 routes, the
    16-route kernels below 256 tokens (W4A8) or 512 (16-bit activations), then the prefill
    kernels: for W4A8 with 64-route up/gate tiles until experts average 32 routes and
    128-route ones from there, for 16-bit activations with 128-route ones throughout."""
    a8 = M.Plan(384, 7168, 576, 6, 7.0, M.A_MXFP8, max_tokens=16384)
    want = {8: M.SEQ_DECODE, 12: M.SEQ_GENERAL, 200: M.SEQ_GENERAL, 255: M.SEQ_GENERAL, 256: M.SEQ_PREFILL_NARROW,
            512: M.SEQ_PREFILL_NARROW, 1024: M.SEQ_PREFILL_NARROW, 2048: M.SEQ_PREFILL, 4096: M.SEQ_PREFILL,
            16384: M.SEQ_PREFILL}
    assert {t: a8.sequence(t) for t in want} == want
    a16 = M.Plan(256, 6144, 512, 8, None, M.A_BF16, max_tokens=4096)
    want = {8: M.SEQ_DECODE, 256: M.SEQ_GENERAL, 511: M.SEQ_GENERAL, 512: M.SEQ_PREFILL,
            1024: M.SEQ_PREFILL, 2048: M.SEQ_PREFILL}
    assert {t: a16.sequence(t) for t in want} == want
    odd = M.Plan(64, 512, 96, 4, None, M.A_BF16, max_tokens=4096)   # N % 64 != 0: no prefill kernels
    assert odd.sequence(4096) == M.SEQ_GENERAL
