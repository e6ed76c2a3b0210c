"""Host checks of the benchmark's work accounting (no GPU): the algorithmic
bytes and flops that the roofline fractions divide by."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_transformer_router_amd import workloads as W  # noqa: E402


def test_bf16_expert_bytes():
    # gate, up and down of 2880 x 2880 in bf16 plus three bias vectors
    assert bench.expert_weight_bytes(W.GPTOSS_DECODE) == 3 * 2880 * 2880 * 2 + 3 * 2880 * 2


def test_mxfp4_expert_bytes():
    # half a byte per element and one scale byte per 32 elements, bf16 biases
    n = 2880 * 2880
    assert bench.expert_weight_bytes(W.GPTOSS_MXFP4) == 3 * (n // 2 + n // 32) + 3 * 2880 * 2


def test_prefill_gate_up_flops():
    # 2 flops per multiply-add of gate and up over T k routed rows:
    # 2 * 32768 * 2 * 2880 * 2880 = 1.087 TFLOP
    counts = [1] * W.GPTOSS_PREFILL.E
    _, flops, n_active = bench.algorithmic_gate_up(W.GPTOSS_PREFILL, counts)
    assert flops == 2.0 * 8192 * 4 * 2 * 2880 * 2880
    assert abs(flops - 1.087e12) < 1e9
    assert n_active == 32


def test_decode_gate_up_bytes_count_active_experts_only():
    w = W.GPTOSS_DECODE
    counts = [0] * w.E
    for e in range(25):
        counts[e] = 1
    nbytes, _, n_active = bench.algorithmic_gate_up(w, counts)
    per_expert = 2 * 2880 * 2880 * 2 + 2 * 2880 * 2
    assert n_active == 25
    assert nbytes == 25 * per_expert + w.T * w.d * 2 + w.P * w.d_ff * 2


@pytest.mark.parametrize("w, beside", [
    (W.GLM4_MOE_LITE, True),                        # bf16, T > 16, no norm, E = 64
    (W.GLM4_MOE_LITE_INT4, True),                   # low-bit routed experts, bf16 shared expert
    (W.GLM4_MOE_LITE_BLOCK, False),                 # the router writes the normalised rows
    (W.GLM4_MOE_LITE.scaled(T=12), False),          # few-token path
    (W.GLM4_MOE_LITE.scaled(E=160), False),         # more routed experts than that path takes
    (W.GPTOSS_PREFILL, False),                      # no shared expert
])
def test_shared_expert_schedule(w, beside):
    assert bench.shared_beside_router(w) is beside


def test_gate_up_stage_counts_the_shared_expert_only_where_it_runs():
    counts = [1] * 64
    base = W.GLM4_MOE_LITE
    _, f_beside, _ = bench.algorithmic_gate_up(base, counts)
    _, f_block, _ = bench.algorithmic_gate_up(W.GLM4_MOE_LITE_BLOCK, counts)
    routed = 2.0 * base.P * 2 * base.d_ff * base.d
    shared = 2.0 * base.T * 2 * base.d_ff_shared * base.d
    assert f_beside == routed
    assert f_block == routed + shared


def test_whole_call_counts_every_product():
    # router plus the three products of every routed row and of the shared expert
    w = W.GLM4_MOE_LITE
    _, flops = bench.algorithmic_call(w, 64)
    expect = 2.0 * w.P * 3 * w.d * w.d_ff + 2.0 * w.T * w.d * w.E + 2.0 * w.T * 3 * w.d * w.d_ff_shared
    assert flops == expect
