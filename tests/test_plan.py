"""Host-only bounds check of the decode library's launch planning
(mk_check_plan): for every benchmark workload and test model, every kernel
variant its batch sizes select, and devices of several CU counts, the GEMV
partitions, exchange-buffer layout (per layer copy and split), 32-bit buffer
offsets and LDS regions must hold every index the kernels form. mk_create runs
the same check before allocating; here it runs without a GPU."""
import dataclasses

import pytest

import workload
from decode_persistent_step_amd import check_plan

MI355X_LDS = 160 * 1024


def _pool(wl, steps=300):
    need = [workload.pages_needed(c, steps) for c in wl.contexts(0)]
    return sum(need), max(need)


@pytest.mark.parametrize("key", sorted(workload.WORKLOADS))
@pytest.mark.parametrize("cus", [256, 304, 192, 128])
def test_benchmark_workloads_plan_in_bounds(key, cus):
    wl = workload.WORKLOADS[key]
    n_pages, mpps = _pool(wl)
    rc, why = check_plan(wl.shape, n_pages, mpps, 8, compute_units=cus, lds_bytes=MI355X_LDS)
    if cus >= 256:   # the MI355X's 256 CUs (more are not used)
        assert rc == 0, f"{key} on {cus} CUs: {why}"
    else:            # fewer CUs: more tiles per workgroup, which may not fit the LDS
        assert rc == 0 or "LDS layout needs" in why, f"{key} on {cus} CUs: {why}"


@pytest.mark.parametrize("shape", [workload.TINY, workload.TINY_G8, workload.TINY_MOE, workload.TINY_FP8,
                                   dataclasses.replace(workload.TINY, name="tiny_swa", window=[32, 0])],
                         ids=lambda s: s.name)
@pytest.mark.parametrize("max_batch", [1, 2, 3, 8])
def test_test_models_plan_in_bounds(shape, max_batch):
    for mpps in (1, 16, 300):
        rc, why = check_plan(shape, 8 * mpps, mpps, max_batch, lds_bytes=MI355X_LDS)
        assert rc == 0, f"{shape.name} batch {max_batch}, {mpps} pages per sequence: {why}"


def test_plan_rejections_name_their_reason():
    # a pool whose layer would exceed 2 GiB (32-bit buffer offsets of the K/V streams)
    rc, why = check_plan(workload.DENSE2B, 300000, 64, 8)
    assert rc == 2 and "2 GiB" in why
    # too few workgroups for the attention segments of 8 requests x 8 kv heads
    rc, why = check_plan(workload.DENSE2B, 4096, 600, 8, compute_units=7)
    assert rc == 2 and "segments" in why
    # an LDS too small for any variant
    rc, why = check_plan(workload.DENSE2B, 4096, 600, 8, lds_bytes=64 * 1024)
    assert rc == 2 and "LDS" in why
    # invalid device sizes
    rc, _ = check_plan(workload.TINY, 8, 4, 1, compute_units=0)
    assert rc == 1
