"""FP8 weight streaming on the GPU against the oracle's FP8 path: the library
quantizes every linear map to E4M3 with per-row scales at mk_create, the
oracle quantizes the same bf16 weights by its own code, and the decode steps
must agree to the same tolerances as the bf16 path (the quantization is the
same on both sides; only the accumulation differs). Vector-ALU (batch 1, 2)
and matrix-core (batch 3-8) consumers, tiny and full-size ~2B models."""
import pytest

import workload
from tests.test_gpu_parity import run_scenario

pytestmark = pytest.mark.gpu


def test_fp8_tiny_b1():
    run_scenario(workload.TINY_FP8, [128], 24, kv_layers=(0, 1))


def test_fp8_tiny_b2_mixed():
    run_scenario(workload.TINY_FP8, [37, 90], 12, temps=[0.0, 0.7], kv_layers=(0, 1))


def test_fp8_tiny_b5_mfma():
    run_scenario(workload.TINY_FP8, [1, 16, 33, 100, 250], 8, temps=[0.0, 0.7, 0.0, 1.3, 0.0],
                 kv_layers=(0, 1))


def test_fp8_dense2b_b1_full_size():
    run_scenario(workload.DENSE2B_FP8, [8192], 2, kv_layers=(0, 24))


def test_fp8_dense2b_b8_full_size():
    wl = workload.WORKLOADS["dense2b_b8_fp8"]
    run_scenario(workload.DENSE2B_FP8, wl.contexts(), 1, temps=wl.temperatures(), kv_layers=(0, 24))
