"""GPU parity of the persistent decode kernel against the fp64 oracle, through the
C ABI, with teacher forcing. Marked gpu: needs an MI355X and the built library."""
import dataclasses
import sys

import numpy as np
import pytest

import workload

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_persistent_step_amd as mk
    mk.lib()  # fails loudly if the library is missing
    yield


def run_scenario(shape, contexts, steps, temps=None, check_every=1, kv_layers=(0,), rows=None, **kw):
    from tests.scenario import Scenario
    _log(f"[parity] {shape.name} B={len(contexts)} ctx={contexts} steps={steps} temps={temps}")
    sc = Scenario(shape, contexts, steps, temps=temps, **kw)
    worst = 0.0
    compared = 0
    for s in range(steps):
        r = sc.step(run_oracle=(s % check_every == 0), rows=rows)
        if r.orc_logits is not None:
            errs = sc.check(r)
            compared += len(errs)
            worst = max([worst] + errs)
            sc.check_kv_append(r, kv_layers)
    sc.check_pool_untouched(kv_layers)
    assert compared > 0
    if shape.moe:
        assert sc.route_compared > 0
        # each layer of each step streamed between top_k and min(E, B top_k) experts
        used = sc.dec.moe_experts_used()
        lo = steps * shape.n_layers * shape.top_k
        hi = steps * shape.n_layers * min(shape.n_experts, len(contexts) * shape.top_k)
        assert lo <= used <= hi, (used, lo, hi)
        assert sc.dec.moe_experts_used() == 0  # the count restarts
    _log(f"[parity] ok, worst logits rel err {worst:.2e}, {compared} rows compared, "
         f"{sc.route_compared} routings compared, {sc.route_ties} decided differently at a near tie")
    return sc


def test_tiny_b1_64_steps():
    # crosses pages 8 -> 12 of the 16-token page size
    run_scenario(workload.TINY, [128], 64, kv_layers=(0, 1))


def test_tiny_b2_valu_batch2():
    run_scenario(workload.TINY, [37, 90], 20, temps=[0.0, 0.7], kv_layers=(0, 1))


def test_tiny_b5_mfma_ragged_mixed():
    run_scenario(workload.TINY, [1, 16, 33, 100, 250], 12, temps=[0.0, 0.7, 0.0, 1.3, 0.0],
                 kv_layers=(0, 1))


def test_tiny_b8_full_batch():
    ctx = [5, 17, 31, 64, 65, 129, 200, 15]
    run_scenario(workload.TINY, ctx, 6, temps=[0.0, 0.7] * 4)


def test_tiny_position_zero_and_single_page():
    run_scenario(workload.TINY, [0], 20, kv_layers=(0, 1))


def test_tiny_sliding_window():
    swa = dataclasses.replace(workload.TINY, name="tiny_swa", window=[32, 0])
    run_scenario(swa, [100, 7], 20, kv_layers=(0, 1))


def test_tiny_contiguous_pages():
    run_scenario(workload.TINY, [128], 8, shuffle=False)


def test_dense2b_b1_8k_full_size():
    # the configuration the bench times: ~2B model, batch 1, 8K context
    run_scenario(workload.DENSE2B, [8192], 2, kv_layers=(0, 24))


def test_dense2b_b8_ragged_full_size():
    wl = workload.WORKLOADS["dense2b_b8"]
    run_scenario(workload.DENSE2B, wl.contexts(), 1, temps=wl.temperatures(), kv_layers=(0, 24))


def test_dense2b_b2_on_batch8_handle_four_wave_fallback():
    # a handle sized for batch 8 with 8K-token requests runs batch 1 on eight compute
    # waves; its batch-2 variant would need 164,864 B of LDS on eight (the page
    # tables of 8 x 8 segments over 8 x 256 waves plus the batch-2 operands and
    # partials), above the 163,840 B limit, and takes the four-wave kernel; the
    # batch 3..8 matrix-core variant runs eight waves with 8-slot rings
    sc = run_scenario(workload.DENSE2B, [8100, 777], 1, temps=[0.0, 0.7], kv_layers=(0, 24), max_batch=8)
    v1, v2, v8 = (sc.dec.variant_info(b) for b in (1, 2, 8))
    _log(f"[parity] variants: b1 {v1}, b2 {v2}, b8 {v8}")
    assert (v1["compute_waves"], v1["path"]) == (8, 0)
    assert (v2["compute_waves"], v2["path"]) == (4, 0)
    assert (v8["compute_waves"], v8["ring_slots"], v8["path"]) == (8, 8, 1)   # matrix cores, 8 x 8 KB rings


def test_tiny_variants_take_eight_waves_where_they_fit():
    sc = run_scenario(workload.TINY, [20, 40], 2, max_batch=8)
    assert sc.dec.variant_info(1)["compute_waves"] == 8
    assert sc.dec.variant_info(2)["compute_waves"] == 8
    assert sc.dec.variant_info(8)["compute_waves"] == 8
    g8 = run_scenario(workload.TINY_G8, [20], 2)
    assert g8.dec.variant_info(1)["compute_waves"] == 4  # group 8: four waves


def test_swa2b_b4_full_size():
    # ~2B model with a 4096 window on even layers, batch 4 at 16K-32K context
    wl = workload.WORKLOADS["swa2b_b4"]
    run_scenario(workload.SWA2B, wl.contexts(), 1, kv_layers=(0, 1))


def test_tiny_g8_b1():
    # group size 8: eight q heads per kv head in one matrix-core column block
    run_scenario(workload.TINY_G8, [300], 12, kv_layers=(0, 1))


def test_tiny_g8_b8_ragged():
    run_scenario(workload.TINY_G8, [0, 15, 16, 17, 100, 255, 256, 40], 6, temps=[0.0, 0.7] * 4,
                 kv_layers=(0, 1))


def test_tiny_moe_b1():
    # batch 1: four of sixteen experts per layer, vector-ALU path
    run_scenario(workload.TINY_MOE, [100], 16, kv_layers=(0, 1))


def test_tiny_moe_b2():
    run_scenario(workload.TINY_MOE, [37, 90], 12, temps=[0.0, 0.7], kv_layers=(0, 1))


def test_tiny_moe_b8_mfma():
    # batch 8: up to all sixteen experts touched, matrix-core path
    ctx = [5, 17, 31, 64, 65, 129, 200, 15]
    run_scenario(workload.TINY_MOE, ctx, 8, temps=[0.0, 0.7] * 4, kv_layers=(0, 1))


def test_moe30b_b8_full_size():
    # the MoE configuration at full size (48 layers, 128 experts, top-8, batch 8 at
    # 2K-8K context): every request, two steps, every layer's routing compared
    wl = workload.WORKLOADS["moe30b_b8"]
    run_scenario(workload.MOE30B, wl.contexts(), 2, temps=wl.temperatures(), kv_layers=(0, 47))
