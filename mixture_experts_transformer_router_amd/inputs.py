"""Seeded synthetic inputs for an MoE-FFN layer.

This module only draws random numbers and encodes them (fp32 -> bf16 bit
patterns by round-to-nearest-even, random MXFP4 codes and block scales).  It
holds none of the layer's arithmetic, so both the GPU path and the CPU oracle
can consume its arrays.

Layout of every array (row-major, contiguous):

  x            [T, d]            activations
  router_w     [E, d]            router weight, [out, in]
  router_b     [E]               router bias (absent when the workload has none)
  w_gate/w_up  [E, d_ff, d]      expert gate / up projections, [out, in]
  b_gate/b_up  [E, d_ff]
  w_down       [E, d, d_ff]      expert down projection, [out, in]
  b_down       [E, d]
  shared_w_gate/shared_w_up [d_ff_shared, d], shared_w_down [d, d_ff_shared]
  norm_w       [d]               RMSNorm scale of a MoE block (block workloads)

bf16 arrays are stored as numpy uint16 bit patterns; f32 arrays as float32.
MXFP4 weights replace w_* by (codes, scales):
  *_codes  uint8 [E, rows, cols/2]: element 2i of a row in the low nibble,
           element 2i+1 in the high nibble; nibble = e2m1 code (bit 3 = sign)
  *_scales uint8 [E, rows, cols/32]: e8m0 exponent byte of each block of 32
           consecutive input-dim elements.
Affine group-quantized weights (weights "affine4" / "affine8") replace w_* by
  *_q        uint8 [E, rows, cols * bits / 8]: unsigned codes (4 bits: element
             2i in the low nibble; 8 bits: one byte per element)
  *_qscales, *_qbiases  bf16 [E, rows, cols / group] (group 32 for 4 bits,
             64 for 8 bits): w = scale * q + bias.

Draw order from numpy.random.default_rng(seed) (PCG64): x, router_w,
router_b, w_gate, b_gate, w_up, b_up, w_down, b_down, shared gate/up/down,
norm_w; weights drawn one expert at a time.  norm_w ~ 1 + N(0, 0.1^2).  Weights ~ N(0, 1/d_in) (std d_in^-1/2),
biases ~ N(0, 0.02^2), x ~ N(0, 1).  The router bias is zero, normal, or
log Zipf(s) over expert rank (b_e = -s*ln(e+1)), per workload.
"""
from __future__ import annotations

import numpy as np

from .workloads import Workload


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal(rng, shape, std, dtype):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def _stacked_normal(rng, E, rows, cols, std, dtype):
    out = np.empty((E, rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for e in range(E):
        out[e] = _normal(rng, (rows, cols), std, dtype)
    return out


def _affine(rng, E, rows, cols, bits, group, std):
    """Affine group-quantized weights: uniform codes over [0, 2^bits), a
    bf16 scale and bias per group of `group` elements of a row, chosen so that
    scale * q + bias has standard deviation ~std and mean ~0."""
    levels = 1 << bits
    q_std = ((levels * levels - 1) / 12.0) ** 0.5
    codes = np.empty((E, rows, cols * bits // 8), dtype=np.uint8)
    scales = np.empty((E, rows, cols // group), dtype=np.uint16)
    biases = np.empty((E, rows, cols // group), dtype=np.uint16)
    for e in range(E):
        q = rng.integers(0, levels, size=(rows, cols), dtype=np.uint8)
        codes[e] = q if bits == 8 else (q[:, 0::2] | (q[:, 1::2] << np.uint8(4)))
        sc = (std / q_std) * (1.0 + 0.1 * rng.standard_normal(size=(rows, cols // group), dtype=np.float32))
        bi = -sc * ((levels - 1) / 2.0) + 0.1 * std * rng.standard_normal(size=sc.shape, dtype=np.float32)
        scales[e] = f32_to_bf16_bits(sc.astype(np.float32))
        biases[e] = f32_to_bf16_bits(bi.astype(np.float32))
    return codes, scales, biases


def _mxfp4(rng, E, rows, cols, lo, hi):
    assert cols % 32 == 0
    codes = np.empty((E, rows, cols // 2), dtype=np.uint8)
    scales = np.empty((E, rows, cols // 32), dtype=np.uint8)
    for e in range(E):
        c = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
        codes[e] = c[:, 0::2] | (c[:, 1::2] << np.uint8(4))
        scales[e] = rng.integers(127 + lo, 127 + hi + 1, size=(rows, cols // 32), dtype=np.uint8)
    return codes, scales


def _mxfp8(rng, E, rows, cols, lo, hi):
    """E4M3 codes uniform over the 254 finite codes (both zeros, the
    subnormals and the largest magnitude 448 included; never a NaN code
    S.1111.111) and e8m0 scale bytes 127 + [lo, hi] per 32 elements."""
    assert cols % 32 == 0
    codes = np.empty((E, rows, cols), dtype=np.uint8)
    scales = np.empty((E, rows, cols // 32), dtype=np.uint8)
    for e in range(E):
        mag = rng.integers(0, 127, size=(rows, cols), dtype=np.uint8)     # 0x00 .. 0x7E
        sign = rng.integers(0, 2, size=(rows, cols), dtype=np.uint8)
        codes[e] = (sign << np.uint8(7)) | mag
        scales[e] = rng.integers(127 + lo, 127 + hi + 1, size=(rows, cols // 32), dtype=np.uint8)
    return codes, scales


def _nvfp4(rng, E, rows, cols, lo, hi):
    """e2m1 codes uniform over the 16 codes, positive E4M3 block scales (one per
    16 elements) with exponent field in [lo, hi] and any mantissa."""
    assert cols % 16 == 0
    codes = np.empty((E, rows, cols // 2), dtype=np.uint8)
    scales = np.empty((E, rows, cols // 16), dtype=np.uint8)
    for e in range(E):
        c = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
        codes[e] = c[:, 0::2] | (c[:, 1::2] << np.uint8(4))
        expo = rng.integers(lo, hi + 1, size=(rows, cols // 16), dtype=np.uint8)
        mant = rng.integers(0, 8, size=(rows, cols // 16), dtype=np.uint8)
        scales[e] = (expo << np.uint8(3)) | mant
    return codes, scales


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw every input array of workload `w` (see module docstring for layout)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    dt = w.dtype
    T, d, F, E = w.T, w.d, w.d_ff, w.E
    out: dict = {}
    out["x"] = _normal(rng, (T, d), 1.0, dt)
    out["router_w"] = _normal(rng, (E, d), d ** -0.5, dt)
    if w.router_bias == "normal":
        out["router_b"] = _normal(rng, (E,), w.bias_std, dt)
    elif w.router_bias == "zero":
        z = np.zeros(E, dtype=np.float32)
        out["router_b"] = f32_to_bf16_bits(z) if dt == "bf16" else z
    elif w.router_bias == "zipf":
        z = (-w.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
        out["router_b"] = f32_to_bf16_bits(z) if dt == "bf16" else z
    else:
        out["router_b"] = None

    def bias(n_rows, n):
        if not w.expert_bias:
            return None
        return _stacked_normal(rng, n_rows, 1, n, w.bias_std, dt).reshape(n_rows, n)

    if w.weights == "dense":
        out["w_gate"] = _stacked_normal(rng, E, F, d, d ** -0.5, dt)
        out["b_gate"] = bias(E, F)
        out["w_up"] = _stacked_normal(rng, E, F, d, d ** -0.5, dt)
        out["b_up"] = bias(E, F)
        out["w_down"] = _stacked_normal(rng, E, d, F, F ** -0.5, dt)
        out["b_down"] = bias(E, d)
    elif w.weights == "mxfp4":
        assert dt == "bf16"
        lo, hi = w.mx_scale_exp_lo, w.mx_scale_exp_hi
        out["w_gate_codes"], out["w_gate_scales"] = _mxfp4(rng, E, F, d, lo, hi)
        out["b_gate"] = bias(E, F)
        out["w_up_codes"], out["w_up_scales"] = _mxfp4(rng, E, F, d, lo, hi)
        out["b_up"] = bias(E, F)
        out["w_down_codes"], out["w_down_scales"] = _mxfp4(rng, E, d, F, lo, hi)
        out["b_down"] = bias(E, d)
    elif w.weights == "mxfp8":
        assert dt == "bf16"
        lo, hi = w.mx_scale_exp_lo, w.mx_scale_exp_hi
        out["w_gate_codes"], out["w_gate_scales"] = _mxfp8(rng, E, F, d, lo, hi)
        out["b_gate"] = bias(E, F)
        out["w_up_codes"], out["w_up_scales"] = _mxfp8(rng, E, F, d, lo, hi)
        out["b_up"] = bias(E, F)
        out["w_down_codes"], out["w_down_scales"] = _mxfp8(rng, E, d, F, lo, hi)
        out["b_down"] = bias(E, d)
    elif w.weights == "nvfp4":
        # fp32 tensor scales with a full 24-bit significand, drawn uniformly in
        # [1, 2) times 2^-9 (2^-8 for down): decoded weights are generally not
        # bf16 numbers
        assert dt == "bf16"
        for name, (r_, c_) in (("w_gate", (F, d)), ("w_up", (F, d)), ("w_down", (d, F))):
            out[name + "_codes"], out[name + "_scales"] = _nvfp4(rng, E, r_, c_, 4, 8)
            m = np.float32(rng.uniform(1.0, 2.0))
            out[name + "_tensor_scale"] = np.float32(np.ldexp(m, -(9 if name != "w_down" else 8)))
            out["b_" + name[2:]] = bias(E, r_)
    elif w.weights in ("affine4", "affine8"):
        assert dt == "bf16"
        bits = 4 if w.weights == "affine4" else 8
        group = 32 if bits == 4 else 64
        out["w_gate_q"], out["w_gate_qscales"], out["w_gate_qbiases"] = _affine(rng, E, F, d, bits, group, d ** -0.5)
        out["b_gate"] = bias(E, F)
        out["w_up_q"], out["w_up_qscales"], out["w_up_qbiases"] = _affine(rng, E, F, d, bits, group, d ** -0.5)
        out["b_up"] = bias(E, F)
        out["w_down_q"], out["w_down_qscales"], out["w_down_qbiases"] = _affine(rng, E, d, F, bits, group, F ** -0.5)
        out["b_down"] = bias(E, d)
    else:
        raise ValueError(w.weights)

    if w.d_ff_shared:
        Fs = w.d_ff_shared
        out["shared_w_gate"] = _normal(rng, (Fs, d), d ** -0.5, dt)
        out["shared_w_up"] = _normal(rng, (Fs, d), d ** -0.5, dt)
        out["shared_w_down"] = _normal(rng, (d, Fs), Fs ** -0.5, dt)
    if w.block:
        # RMSNorm scale, drawn last so that the layer's other arrays are those
        # of the same workload without the block
        g = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(size=d, dtype=np.float32)
        out["norm_w"] = f32_to_bf16_bits(g) if dt == "bf16" else g
    return out

