"""Repeatability of the decode step on the GPU: the same step run twice from
identical state must give bit-identical tokens, logits and K/V rows for dense
models (every sum has a fixed order). MoE steps add the expert outputs with
fp32 atomics in arrival order, so their last bits may vary: the test records
how many logits differ and by how many units in the last place, and bounds
them far below the parity tolerance."""
import numpy as np
import pytest

import workload

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"  [determinism] {msg}", flush=True)


def _twice(shape, contexts, temps, warm_steps, layers):
    """Step `warm_steps` times, then run the next step twice with the same inputs.
    The second run rewrites the K/V slots the first wrote; attention takes the
    current token's K/V from the step's own exchange, so the state is identical."""
    import torch
    from decode_persistent_step_amd import session
    from tests.scenario import Scenario
    sc = Scenario(shape, contexts, warm_steps + 1, temps=temps, with_oracle=False)
    for _ in range(warm_steps):
        sc.step(run_oracle=False)
    n = len(contexts)
    seq_t = torch.tensor(sc.seq, dtype=torch.int32, device="cuda")
    tok_t = torch.tensor(sc.tokens, dtype=torch.int32, device="cuda")
    slots = np.asarray(sc.new_kv_slots(sc.seq), dtype=np.int32)
    runs = []
    for _ in range(2):
        logits = torch.empty((n, shape.vocab), dtype=torch.float32, device="cuda")
        out = sc.dec.decode_step(seq_t, sc.pt, tok_t, sc.temp_t, seed=sc.seed, step=sc.step_idx,
                                 logits_out=logits)
        torch.cuda.synchronize()
        kv = [session.read_kv_rows(sc.dec, l, kv, slots) for l in layers for kv in (0, 1)]
        runs.append((out.cpu().numpy().copy(), logits.cpu().numpy().copy(), kv))
    assert sc.dec.last_error()[0] == 0
    return runs


def _ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between fp32 arrays of one sign."""
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


@pytest.mark.parametrize("name,contexts,temps,layers", [
    ("tiny", [128], [0.0], (0, 1)),
    ("tiny", [5, 17, 31, 64, 65, 129, 200, 15], [0.0, 0.7] * 4, (0, 1)),
    ("dense2b", [8192], [0.0], (0, 12, 24)),
])
def test_dense_step_is_bit_reproducible(name, contexts, temps, layers):
    shape = {"tiny": workload.TINY, "dense2b": workload.DENSE2B}[name]
    _log(f"{name} batch {len(contexts)}")
    (t1, l1, kv1), (t2, l2, kv2) = _twice(shape, contexts, temps, 2, layers)
    assert np.array_equal(t1, t2)
    assert np.array_equal(l1.view(np.int32), l2.view(np.int32)), "logits bits differ"
    for a, b in zip(kv1, kv2):
        assert np.array_equal(a, b), "K/V rows differ"


def test_moe_step_variation_is_last_bits_only():
    """Tiny MoE at batch 8 (atomic expert sums): tokens equal, every logit within
    a few fp32 ulps relative to the row's scale; the count of differing logits
    and the largest ulp distance are printed."""
    shape = workload.TINY_MOE
    ctx = [5, 17, 31, 64, 65, 129, 200, 15]
    (t1, l1, kv1), (t2, l2, kv2) = _twice(shape, ctx, [0.0] * 8, 2, (0, 1))
    differ = int(np.sum(l1.view(np.int32) != l2.view(np.int32)))
    rel = float(np.max(np.abs(l1.astype(np.float64) - l2) / np.max(np.abs(l1), axis=1, keepdims=True)))
    same_sign = np.sign(l1) == np.sign(l2)
    ulp = int(np.max(_ulps(l1[same_sign], l2[same_sign]))) if same_sign.any() else 0
    _log(f"tiny MoE batch 8: {differ} of {l1.size} logits differ, largest {ulp} ulp, "
         f"largest difference {rel:.2e} of the row's largest logit")
    assert rel <= 1e-5, rel
    kv_diff = sum(int(np.sum(a != b)) for a, b in zip(kv1, kv2))
    _log(f"tiny MoE batch 8: {kv_diff} K/V values differ (layer 1 follows layer 0's atomic sums)")
    for b in range(len(ctx)):
        if t1[b] != t2[b]:
            srt = np.sort(l1[b])[::-1]
            assert srt[0] - srt[1] < 1e-3, f"request {b}: tokens {t1[b]} / {t2[b]} without a near tie"
