"""Host checks of the seeded input generator: the recipe the parity tests and
the benchmark rely on (layouts, seeding, value ranges, bf16 rounding)."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mixture_experts_transformer_router_amd import inputs as I  # noqa: E402
from mixture_experts_transformer_router_amd import workloads as W  # noqa: E402


def _small(w, **kw):
    return w.scaled(**{"T": 24, "d": 64, "d_ff": 96, "E": 8, "k": 2, **kw})


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 lies halfway between the bf16 numbers 1 and 1 + 2^-7: ties go
    # to the even significand (1); 1 + 3 * 2^-8 goes up to 1 + 2^-6
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5], dtype=np.float32)
    bits = I.f32_to_bf16_bits(vals)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0, -2.5]


def test_same_seed_same_arrays_and_other_seed_differs():
    w = _small(W.GPTOSS_DECODE)
    a, b, c = I.make_inputs(w), I.make_inputs(w), I.make_inputs(w, seed=w.seed + 1)
    assert a.keys() == b.keys()
    for key in a:
        if a[key] is not None:
            assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["x"], c["x"])


def test_dense_layout_and_scales():
    w = _small(W.GPTOSS_DECODE, T=512, d=256, d_ff=128)
    a = I.make_inputs(w)
    assert a["x"].shape == (512, 256) and a["x"].dtype == np.uint16
    assert a["router_w"].shape == (8, 256)
    assert a["w_gate"].shape == (8, 128, 256) and a["w_down"].shape == (8, 256, 128)
    assert a["b_gate"].shape == (8, 128) and a["b_down"].shape == (8, 256)
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    # x ~ N(0, 1), weights ~ N(0, 1/d_in), biases ~ N(0, 0.02^2)
    assert abs(f(a["x"]).std() - 1.0) < 0.02
    assert abs(f(a["w_gate"]).std() * 256 ** 0.5 - 1.0) < 0.02
    assert abs(f(a["w_down"]).std() * 128 ** 0.5 - 1.0) < 0.02
    assert abs(f(a["b_gate"]).std() / 0.02 - 1.0) < 0.1
    # the decode workload's router bias is zero
    assert not f(a["router_b"]).any()


def test_zipf_router_bias():
    w = _small(W.GPTOSS_PREFILL)
    b = I.make_inputs(w)["router_b"]
    got = (b.astype(np.uint32) << 16).view(np.float32)
    want = -w.zipf_s * np.log(np.arange(1, w.E + 1))
    assert np.allclose(got, want, rtol=2 ** -8, atol=0)
    assert got[0] == 0.0 and np.all(np.diff(got) < 0)


def test_mxfp4_codes_and_scales():
    w = _small(W.GPTOSS_MXFP4)
    a = I.make_inputs(w)
    assert a["w_gate_codes"].shape == (8, 96, 32) and a["w_gate_scales"].shape == (8, 96, 2)
    assert a["w_down_codes"].shape == (8, 64, 48) and a["w_down_scales"].shape == (8, 64, 3)
    s = a["w_gate_scales"].astype(int) - 127
    assert s.min() >= w.mx_scale_exp_lo and s.max() <= w.mx_scale_exp_hi
    nib = np.concatenate([a["w_up_codes"] & 15, a["w_up_codes"] >> 4]).ravel()
    assert set(np.unique(nib).tolist()) == set(range(16))


def test_mxfp8_codes_cover_the_finite_e4m3_codes():
    w = _small(W.GPTOSS_MXFP8_MX8, d=256, d_ff=256)
    a = I.make_inputs(w)
    codes = np.concatenate([a[k].ravel() for k in ("w_gate_codes", "w_up_codes", "w_down_codes")])
    mag = codes & 0x7F
    assert not np.any(mag == 0x7F)              # no NaN code
    assert np.any(mag == 0x7E)                  # 448
    assert np.any((mag > 0) & (mag < 8))        # subnormals
    assert np.any(mag == 0) and np.any(codes == 0x80)  # both zeros
    assert len(np.unique(codes)) == 254
    s = a["w_gate_scales"].astype(int) - 127
    assert s.min() >= w.mx_scale_exp_lo and s.max() <= w.mx_scale_exp_hi


def test_nvfp4_scales_and_general_tensor_scales():
    w = _small(W.GPTOSS_NVFP4)
    a = I.make_inputs(w)
    sc = a["w_gate_scales"]
    assert sc.shape == (8, 96, 4)
    assert not np.any(sc & 0x80)                # positive
    expo = sc >> 3
    assert expo.min() >= 4 and expo.max() <= 8  # no subnormal, no NaN
    for name, e in (("w_gate", -9), ("w_up", -9), ("w_down", -8)):
        t = float(a[name + "_tensor_scale"])
        m = np.ldexp(t, -e)
        assert 1.0 <= m < 2.0
    # at least one tensor scale uses more significand bits than bf16 keeps
    ms = [np.ldexp(float(a[n + "_tensor_scale"]), 9 if n != "w_down" else 8) for n in ("w_gate", "w_up", "w_down")]
    assert any((np.float32(m).view(np.uint32) & 0xFFFF) != 0 for m in ms)


@pytest.mark.parametrize("wl, bits, group", [(W.GLM4_MOE_LITE_INT4, 4, 32), (W.GLM4_MOE_LITE_INT8, 8, 64)])
def test_affine_codes_and_groups(wl, bits, group):
    w = _small(wl, d=128, d_ff=64, E=8, k=2, n_group=2, topk_group=1, d_ff_shared=32)
    a = I.make_inputs(w)
    q = a["w_gate_q"]
    assert q.shape == (8, 64, 128 * bits // 8)
    assert a["w_gate_qscales"].shape == (8, 64, 128 // group) == a["w_gate_qbiases"].shape
    if bits == 4:
        vals = np.concatenate([q & 15, q >> 4]).ravel()
        assert vals.max() == 15 and vals.min() == 0
    else:
        assert q.max() == 255 and q.min() == 0
    # the shared expert stays bf16
    assert a["shared_w_gate"].dtype == np.uint16 and a["shared_w_gate"].shape == (32, 128)


def test_block_norm_weight():
    w = _small(W.GLM4_MOE_LITE_BLOCK, d=512)
    g = I.make_inputs(w)["norm_w"]
    v = (g.astype(np.uint32) << 16).view(np.float32)
    assert v.shape == (512,)
    assert abs(v.mean() - 1.0) < 0.02 and abs(v.std() / 0.1 - 1.0) < 0.15
