"""Pins of the oracle's FP8 weight path (E4M3 codes, one fp32 scale per output
row; the reading of the pages' 8-bit weights is in oracle.c): the code table
against the format's anchor values, the encoder against torch's own
float8_e4m3fn cast (an independent library routine) including exact ties and
subnormals, saturation, the per-row quantizer's closed forms, the FP8
matrix-vector product against brute force, and a whole-step wiring pin:
with power-of-two row scales the FP8 step equals, bit for bit, the bf16 step
run on the dequantized weights (which are then exact bf16 values)."""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import workload


def test_code_table_anchors_and_order():
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
               0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for q, v in anchors.items():
        assert oracle.fp8_value(q) == v, hex(q)
    assert math.isnan(oracle.fp8_value(0x7F)) and math.isnan(oracle.fp8_value(0xFF))
    vals = [oracle.fp8_value(q) for q in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))          # codes 0..0x7E increase
    assert [oracle.fp8_value(q | 0x80) for q in range(1, 0x7F)] == [-v for v in vals[1:]]


def test_encoder_matches_torch_cast_on_grids_ties_and_subnormals():
    import torch
    rng = np.random.default_rng(3)
    vals = np.array([oracle.fp8_value(q) for q in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2                         # exact ties: nearest even code
    xs = np.concatenate([vals, -vals, mids, -mids, rng.standard_normal(4000) * 50,
                         rng.standard_normal(4000) * 2.0 ** -8, np.linspace(-448, 448, 4001)]).astype(np.float32)
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)  # ties exact in fp32
    mine = np.array([oracle.fp8_encode(float(x)) for x in xs], dtype=np.uint8)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    # ties go to the even mantissa: between 1.0 (0x38) and 1.125 (0x39) -> 0x38;
    # between 1.125 and 1.25 (0x3A) -> 0x3A
    assert oracle.fp8_encode(1.0625) == 0x38 and oracle.fp8_encode(1.1875) == 0x3A


def test_encoder_saturates_and_round_trips():
    for x in (448.0, 449.0, 463.9, 464.0, 500.0, 1e30):
        assert oracle.fp8_encode(x) == 0x7E and oracle.fp8_encode(-x) == 0xFE
    for q in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert oracle.fp8_encode(oracle.fp8_value(q)) == (q if q != 0x80 else 0x80)
    assert oracle.fp8_encode(2.0 ** -11) == 0x00        # a quarter of the smallest subnormal
    assert oracle.fp8_encode(0.75 * 2.0 ** -9) == 0x01   # nearest: 2^-9
    # subnormal ties go to the even code: 0.5, 1.5, 2.5 x 2^-9 -> 0, 2, 2
    assert [oracle.fp8_encode(t * 2.0 ** -9) for t in (0.5, 1.5, 2.5)] == [0x00, 0x02, 0x02]


def test_quantize_rows_closed_forms_and_error_bound():
    from tests.test_oracle_components import bf16_pattern
    rng = np.random.default_rng(5)
    W = ((rng.standard_normal((6, 48)) * 0.02).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    W[1, 7] = bf16_pattern(-448.0 * 2.0 ** -10)   # row 1: amax exactly 448 * 2^-10
    W[2, :] = 0                                   # all-zero row: scale 1, codes 0
    q, sc = oracle.fp8_quantize_rows(W)
    assert sc[1] == np.float32(2.0 ** -10) and q[1, 7] == 0xFE
    assert sc[2] == 1.0 and np.all(q[2] == 0)
    for r in range(6):
        w = (W[r].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        amax = np.max(np.abs(w))
        if amax > 0:
            assert sc[r] == np.float32(np.float32(amax) / np.float32(448.0))
        deq = np.array([oracle.fp8_value(int(c)) for c in q[r]]) * np.float64(sc[r])
        t = np.abs(w) / np.float64(sc[r])
        # half a grid step of the value's binade (2^-9 grid below 2^-6), relative to the scale
        step = np.where(t < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3))
        assert np.all(np.abs(deq - w) <= 0.5 * step * np.float64(sc[r]) * (1 + 1e-6) + 1e-30)


def test_matvec_fp8_matches_brute_force():
    rng = np.random.default_rng(7)
    q = rng.integers(0, 256, size=(9, 40), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x33                   # no NaN codes
    sc = rng.uniform(0.01, 2.0, size=9).astype(np.float32)
    x = rng.standard_normal(40)
    want = np.array([float(sc[r]) * sum(oracle.fp8_value(int(q[r, c])) * x[c] for c in range(40))
                     for r in range(9)])
    assert np.allclose(oracle.matvec_fp8(q, sc, x), want, rtol=1e-14, atol=1e-300)


def _pow2_scaled(shape, seed):
    """Weights whose every linear map has a row maximum of +-448 x 2^-10 (so each
    row's scale is exactly 2^-10) and the dequantized bf16 copy of them."""
    w = workload.gen_weights(shape, seed=seed)
    big = np.uint16(0x3EE0)  # 0.4375 = 448 x 2^-10 in bf16
    names = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]
    for n in names:
        for a in w[n]:
            a[:, 0] = big
    w["lm_head"][:, 0] = big
    deq = dict(w)

    def dq(a):
        q, sc = oracle.fp8_quantize_rows(a)
        assert np.all(sc == np.float32(2.0 ** -10))
        vals = np.vectorize(oracle.fp8_value)(q) * 2.0 ** -10
        out = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32).astype(np.float64), vals)
        return out

    for n in names:
        deq[n] = [dq(a) for a in w[n]]
    deq["lm_head"] = dq(w["lm_head"])
    return w, deq


def test_fp8_step_equals_bf16_step_on_dequantized_weights_bitwise():
    shape = dataclasses.replace(workload.TINY, name="fp8_micro", n_layers=2, d_model=128, n_q_heads=4,
                                n_kv_heads=2, head_dim=32, ffn_dim=256, vocab=512)
    w, deq = _pow2_scaled(shape, seed=4)
    m8 = oracle.OracleModel(shape, w, 8, 4, weight_format="fp8")
    mb = oracle.OracleModel(shape, deq, 8, 4)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((2, 8, 2, 16, 32)).astype(np.float32)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    m8.kpool[...] = kb
    m8.vpool[...] = kb[::-1]
    mb.kpool[...] = m8.kpool
    mb.vpool[...] = m8.vpool
    t8, l8 = m8.decode_step([21, 5], [[0, 1, 2, 3], [4, 5, 6, 7]], [3, 9], [0.0, 0.9], seed=2, step=1)
    tb, lb = mb.decode_step([21, 5], [[0, 1, 2, 3], [4, 5, 6, 7]], [3, 9], [0.0, 0.9], seed=2, step=1)
    assert np.array_equal(l8, lb) and np.array_equal(t8, tb)
    assert np.array_equal(m8.kpool, mb.kpool) and np.array_equal(m8.vpool, mb.vpool)


def test_fp8_step_differs_from_bf16_by_the_quantization_only():
    """On ordinary weights the FP8 step is not the bf16 step (the codes round the
    weights), but close: logits within a few percent of the row's scale."""
    shape = dataclasses.replace(workload.TINY, name="fp8_micro", n_layers=2, d_model=128, n_q_heads=4,
                                n_kv_heads=2, head_dim=32, ffn_dim=256, vocab=512)
    w = workload.gen_weights(shape, seed=8)
    m8 = oracle.OracleModel(shape, w, 8, 4, weight_format="fp8")
    mb = oracle.OracleModel(shape, w, 8, 4)
    _, l8 = m8.decode_step([3], [[0, 1, 2, 3]], [7])
    _, lb = mb.decode_step([3], [[0, 1, 2, 3]], [7])
    rel = np.max(np.abs(l8 - lb)) / np.max(np.abs(lb))
    assert 1e-4 < rel < 0.1, rel
