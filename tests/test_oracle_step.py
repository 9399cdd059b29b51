"""Wiring pins of the oracle's whole decode step: planted weights whose output
has a closed form, and invariances the definition implies (batch independence,
page-permutation invariance, zero layers, window reduction, MoE with one
expert). The pages print no worked example of a decode step, so the whole-step
result is pinned by these plus the component pins."""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import workload
from tests.test_oracle_components import as_bf16, bf16_pattern, bf16_vals, to_bf16_exact

MICRO = workload.ModelShape("micro", n_layers=1, d_model=16, n_q_heads=2, n_kv_heads=1,
                            head_dim=8, ffn_dim=32, vocab=64)
ONE = bf16_pattern(1.0)


def zero_weights(shape):
    w = {"embed": np.zeros((shape.vocab, shape.d_model), np.uint16),
         "final_norm": np.full(shape.d_model, ONE, np.uint16),
         "lm_head": np.zeros((shape.vocab, shape.d_model), np.uint16)}
    for n, s in shape.weight_shapes().items():
        fill = ONE if n in ("attn_norm", "ffn_norm") else 0
        w[n] = [np.full(s, fill, np.uint16) for _ in range(shape.n_layers)]
    return w


def identity_rows(rows, cols, scale=1.0):
    W = np.zeros((rows, cols), np.uint16)
    for i in range(min(rows, cols)):
        W[i, i] = bf16_pattern(scale)
    return W


def model(shape, w, n_pages=8, mpps=4):
    return oracle.OracleModel(shape, w, n_pages, mpps)


def test_residual_passthrough_closed_form():
    """W_o = W_down = 0: x_L = E[tok], logits = W_lm (g_f * rmsnorm(E[tok])). The
    planted lm_head entry W_lm[t, j] is off the diagonal so a transposed head fails."""
    s = MICRO
    w = zero_weights(s)
    c, j, tok, t = 0.5, 5, 9, 40
    w["embed"][tok, j] = bf16_pattern(c)
    w["lm_head"][t, j] = bf16_pattern(1.0)
    w["final_norm"][j] = bf16_pattern(1.5)
    m = model(s, w)
    toks, logits = m.decode_step([3], [[0, 1, 2, 3]], [tok])
    want = np.zeros(s.vocab)
    want[t] = 1.5 * c / math.sqrt(c * c / s.d_model + s.rms_eps)
    assert np.allclose(logits[0], want, rtol=1e-14, atol=0)
    assert toks[0] == t


MICRO_GQA = workload.ModelShape("micro_gqa", n_layers=1, d_model=16, n_q_heads=4,
                                n_kv_heads=2, head_dim=4, ffn_dim=32, vocab=64)


def perm_rows(n, shift):
    """W[(i + shift) % n, i] = 1: input i goes to output (i + shift) % n."""
    W = np.zeros((n, n), np.uint16)
    for i in range(n):
        W[(i + shift) % n, i] = bf16_pattern(1.0)
    return W


def test_uniform_attention_wiring_closed_form():
    """W_q = 0 makes attention uniform over positions 0..p (p+1 keys, the new one
    included). Prefilled V of kv head 0 is e_0 and of kv head 1 is e_1, the new v is
    0 (W_v = 0); q heads 0,1 read kv head 0 and q heads 2,3 read kv head 1
    (consecutive GQA groups). So o = a (e_0 + e_4 + e_9 + e_13), a = p/(p+1).
    W_o shifts every index by 3 (not symmetric), W_down = 0, zero embedding row,
    W_lm = I: logits = rmsnorm(W_o o)."""
    s = MICRO_GQA
    w = zero_weights(s)
    w["wo"][0] = perm_rows(s.d_model, 3)
    w["wk"][0] = identity_rows(s.n_kv_heads * s.head_dim, s.d_model, 0.5)
    w["lm_head"][: s.d_model] = identity_rows(s.d_model, s.d_model)
    m = model(s, w)
    p = 21
    pages = [5, 2, 6, 0]
    for j in range(p):
        m.vpool[0, pages[j // 16], 0, j % 16, 0] = ONE
        m.vpool[0, pages[j // 16], 1, j % 16, 1] = ONE
    toks, logits = m.decode_step([p], [pages], [7])
    a = p / (p + 1)
    o = np.zeros(s.d_model)
    o[[0, 4, 9, 13]] = a
    h = np.zeros(s.d_model)
    h[(np.arange(s.d_model) + 3) % s.d_model] = o
    want = np.zeros(s.vocab)
    want[: s.d_model] = h / math.sqrt(np.mean(h * h) + s.rms_eps)
    assert np.allclose(logits[0], want, rtol=1e-12, atol=0)
    assert toks[0] == 0  # ties among 3, 7, 12, 0 go to the lowest index


def test_key_layout_and_head_selection():
    """A single planted key of kv head 1 at position 9 aligned with q makes that
    position dominate for q heads 2, 3 only; with W_o = I and V = one-hot position
    codes the output shows which position each head attended to."""
    s = MICRO_GQA
    w = zero_weights(s)
    tok, j = 7, 2
    w["embed"][tok, j] = bf16_pattern(1.0)
    w["wq"][0][:, j] = bf16_pattern(1.0)      # every q entry equals n_j
    w["wo"][0] = identity_rows(s.d_model, s.d_model)
    w["lm_head"][: s.d_model] = identity_rows(s.d_model, s.d_model)
    m = model(s, w)
    pages = [3, 1, 0, 2]
    p = 12
    kpos = 9
    for dim in range(s.head_dim):
        m.kpool[0, pages[0], 1, kpos, dim] = bf16_pattern(64.0)
    for jj in range(p):
        for g in range(s.n_kv_heads):
            m.vpool[0, pages[0], g, jj, 3] = bf16_pattern(float(jj + 1))
    _, _, lx = m.decode_step([p], [pages], [tok], want_layers=True)
    x = lx[0, 0]
    # q heads 2, 3 (kv head 1) put ~all weight on position 9 -> dim 3 of their slice ~ 10
    assert abs(x[8 + 3] - 10.0) < 1e-6 and abs(x[12 + 3] - 10.0) < 1e-6
    # q heads 0, 1 (kv head 0) see all-zero keys: uniform over 13 keys, the new v = 0
    mean_code = sum(range(1, p + 1)) / (p + 1)
    assert abs(x[3] - mean_code) < 1e-9 and abs(x[4 + 3] - mean_code) < 1e-9


def test_kv_append_slot_and_values_closed_form():
    """x = c e_j; n = rmsnorm(x) = e_j c / sqrt(c^2/d + eps); W_k, W_v one-hot pick n_j
    into dims (r, r'); k is rotated at position p, v is not; both land in slot
    (page_table[p // 16], p % 16) as bf16 and nothing else in the pool changes."""
    s = MICRO
    w = zero_weights(s)
    c, j, tok, r, rv = 0.75, 4, 11, 2, 6
    w["embed"][tok, j] = bf16_pattern(c)
    w["wk"][0][r, j] = bf16_pattern(1.0)
    w["wv"][0][rv, j] = bf16_pattern(-2.0)
    m = model(s, w)
    rng = np.random.default_rng(0)
    m.kpool[...] = rng.integers(0, 0x7F00, m.kpool.shape, dtype=np.uint16)
    m.vpool[...] = rng.integers(0, 0x7F00, m.vpool.shape, dtype=np.uint16)
    k0, v0 = m.kpool.copy(), m.vpool.copy()
    p, pages = 37, [3, 7, 1, 0]
    m.decode_step([p], [pages], [tok])
    nj = c / math.sqrt(c * c / s.d_model + s.rms_eps)
    half = s.head_dim // 2
    a = p * s.rope_base ** (-2.0 * r / s.head_dim)          # r < half
    kw = np.zeros(s.head_dim)
    kw[r], kw[r + half] = nj * math.cos(a), nj * math.sin(a)
    vw = np.zeros(s.head_dim)
    vw[rv] = -2.0 * nj
    pg, sl = pages[p // 16], p % 16
    got_k = bf16_vals(m.kpool[0, pg, 0, sl])
    got_v = bf16_vals(m.vpool[0, pg, 0, sl])
    assert np.allclose(got_k, kw, rtol=2 ** -8, atol=0)
    assert np.allclose(got_v, vw, rtol=2 ** -8, atol=0)
    mask = np.ones(m.kpool.shape, bool)
    mask[0, pg, 0, sl] = False
    assert np.array_equal(m.kpool[mask], k0[mask]) and np.array_equal(m.vpool[mask], v0[mask])


def _random_model(shape, n_pages, mpps, seed=0):
    w = workload.gen_weights(shape, seed=seed)
    return w, model(shape, w, n_pages, mpps)


def _fill_random_kv(m, rng):
    m.kpool[...] = as_bf16(to_bf16_exact(rng.normal(0, 1, m.kpool.shape)))
    m.vpool[...] = as_bf16(to_bf16_exact(rng.normal(0, 1, m.vpool.shape)))


SMALL = dataclasses.replace(workload.TINY, name="small", n_layers=2, d_model=64, n_q_heads=4,
                            n_kv_heads=2, head_dim=16, ffn_dim=96, vocab=300)


def test_batch_independence_bitwise():
    w, m = _random_model(SMALL, 16, 4)
    rng = np.random.default_rng(1)
    _fill_random_kv(m, rng)
    base_k, base_v = m.kpool.copy(), m.vpool.copy()
    seq = [5, 40, 17]
    pt = [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]]
    toks_in = [3, 100, 299]
    temps = [0.0, 0.7, 0.0]
    tb, lb = m.decode_step(seq, pt, toks_in, temps, seed=9, step=4)
    for b in range(3):
        m.kpool[...], m.vpool[...] = base_k, base_v
        t1, l1 = m.decode_step([seq[b]], [pt[b]], [toks_in[b]], [temps[b]], seed=9, step=4)
        assert np.array_equal(l1[0], lb[b])
        if temps[b] == 0.0:
            assert t1[0] == tb[b]


def test_page_permutation_invariance_bitwise():
    w, m1 = _random_model(SMALL, 12, 4)
    m2 = model(SMALL, w, 12, 4)
    rng = np.random.default_rng(2)
    p = 45
    ids1, ids2 = [0, 1, 2, 3], [9, 4, 11, 6]
    for l in range(SMALL.n_layers):
        k = as_bf16(to_bf16_exact(rng.normal(0, 1, (p, SMALL.n_kv_heads, SMALL.head_dim))))
        v = as_bf16(to_bf16_exact(rng.normal(0, 1, (p, SMALL.n_kv_heads, SMALL.head_dim))))
        m1.prefill_from(ids1, l, k, v)
        m2.prefill_from(ids2, l, k, v)
    t1, l1 = m1.decode_step([p], [ids1], [17])
    t2, l2 = m2.decode_step([p], [ids2], [17])
    assert np.array_equal(l1, l2) and t1[0] == t2[0]
    # the new slot holds identical K/V in both pools
    for l in range(SMALL.n_layers):
        assert np.array_equal(m1.kpool[l, ids1[p // 16], :, p % 16], m2.kpool[l, ids2[p // 16], :, p % 16])


def test_window_at_least_context_equals_full_bitwise():
    w, m1 = _random_model(SMALL, 8, 8)
    swa = dataclasses.replace(SMALL, window=[64, 0])
    m2 = model(swa, w, 8, 8)
    rng = np.random.default_rng(3)
    _fill_random_kv(m1, rng)
    m2.kpool[...], m2.vpool[...] = m1.kpool, m1.vpool
    pt = [list(range(8))]
    t1, l1 = m1.decode_step([60], pt, [5])
    t2, l2 = m2.decode_step([60], pt, [5])
    assert np.array_equal(l1, l2)
    # a window smaller than the context changes the result
    m3 = model(dataclasses.replace(SMALL, window=[8, 0]), w, 8, 8)
    m3.kpool[...], m3.vpool[...] = m2.kpool, m2.vpool
    _, l3 = m3.decode_step([60], pt, [5])
    assert not np.allclose(l3, l1)


def test_zeroed_layer_is_transparent_bitwise():
    """A second layer with W_o = W_down = 0 adds exact zeros to the residual."""
    one = dataclasses.replace(SMALL, n_layers=1)
    w1, m1 = _random_model(one, 8, 4)
    w2 = {k: (list(v) if isinstance(v, list) else v) for k, v in w1.items()}
    for n, shp in SMALL.weight_shapes().items():
        extra = np.zeros(shp, np.uint16) if n in ("wo", "w_down") else \
            workload.gen_tensor(SMALL, n, 1, seed=77)
        w2[n] = w1[n] + [extra]
    m2 = model(SMALL, w2, 8, 4)
    rng = np.random.default_rng(4)
    _fill_random_kv(m1, rng)
    m2.kpool[0], m2.vpool[0] = m1.kpool[0], m1.vpool[0]
    t1, l1 = m1.decode_step([20], [[0, 1, 2, 3]], [42])
    t2, l2 = m2.decode_step([20], [[0, 1, 2, 3]], [42])
    assert np.array_equal(l1, l2)


def test_moe_single_expert_equals_dense_bitwise():
    dense = dataclasses.replace(SMALL, n_layers=1)
    moe = dataclasses.replace(dense, ffn_dim=0, n_experts=1, top_k=1, expert_ffn_dim=96)
    wd, md = _random_model(dense, 8, 4)
    wm = dict(wd)
    wm["w_gate"] = [wd["w_gate"][0][None]]
    wm["w_up"] = [wd["w_up"][0][None]]
    wm["w_down"] = [wd["w_down"][0][None]]
    wm["router"] = [workload.gen_tensor(moe, "router", 0)]
    mm = model(moe, wm, 8, 4)
    rng = np.random.default_rng(5)
    _fill_random_kv(md, rng)
    mm.kpool[...], mm.vpool[...] = md.kpool, md.vpool
    t1, l1 = md.decode_step([30], [[0, 1, 2, 3]], [7])
    t2, l2 = mm.decode_step([30], [[0, 1, 2, 3]], [7])
    assert np.array_equal(l1, l2)


def test_moe_routing_selects_planted_experts():
    """Router rows that copy one input coordinate with distinct positive gains make
    the selection known; experts other than the selected ones have huge weights
    that would show if they were used."""
    d, E, k, fe = 16, 6, 2, 4
    shape = workload.ModelShape("moe_micro", n_layers=1, d_model=d, n_q_heads=2, n_kv_heads=1,
                                head_dim=8, ffn_dim=0, vocab=32, n_experts=E, top_k=k,
                                expert_ffn_dim=fe)
    w = zero_weights(shape)
    tok, j = 3, 2
    w["embed"][tok, j] = bf16_pattern(1.0)
    gains = [0.5, 4.0, 1.0, 3.0, 0.25, 2.0]        # top-2: experts 1 (4.0) and 3 (3.0)
    for e, gval in enumerate(gains):
        w["router"][0][e, j] = bf16_pattern(gval)
        w["w_gate"][0][e, 0, j] = bf16_pattern(1.0)
        w["w_up"][0][e, 0, j] = bf16_pattern(1.0)
        w["w_down"][0][e, e, 0] = bf16_pattern(1.0 if e in (1, 3) else 256.0)
    w["lm_head"][:d] = identity_rows(d, d)
    m = model(shape, w)
    _, logits = m.decode_step([0], [[0, 1, 2, 3]], [tok])
    n = 1.0 / math.sqrt(1.0 / d + shape.rms_eps)         # n2_j (h = x = e_j)
    ffn = n / (1 + math.exp(-n)) * n                     # silu(n) * n per selected expert
    r1, r3 = 4.0 * n, 3.0 * n
    w1 = 1.0 / (1.0 + math.exp(r3 - r1))
    h = np.zeros(d)
    h[j] = 1.0
    h[1] += w1 * ffn
    h[3] += (1 - w1) * ffn
    want = h / math.sqrt(np.mean(h * h) + shape.rms_eps)
    assert np.allclose(logits[0, :d], want, rtol=1e-12)
    assert np.all(logits[0, d:] == 0)
    # the routing margin: 2nd-best taken (3.0 n) against the best left out (2.0 n)
    _, _, gap = m.decode_step([0], [[0, 1, 2, 3]], [tok], want_route_gap=True)
    assert gap[0] == pytest.approx(1.0 * n, rel=1e-12)


def test_route_gap_is_infinite_for_dense_and_all_experts():
    w, m = _random_model(SMALL, 4, 4)
    _, _, gap = m.decode_step([5], [[0, 1, 2, 3]], [1], want_route_gap=True)
    assert np.isinf(gap[0]) and gap[0] > 0
    moe = dataclasses.replace(SMALL, n_layers=1, ffn_dim=0, n_experts=2, top_k=2, expert_ffn_dim=32)
    wm = workload.gen_weights(moe, seed=9)
    mm = model(moe, wm, 8, 4)
    _, _, gap = mm.decode_step([5], [[0, 1, 2, 3]], [1], want_route_gap=True)
    assert np.isinf(gap[0])


def test_step_rejects_uncovered_page_table():
    w, m = _random_model(SMALL, 4, 4)
    with pytest.raises(ValueError):
        m.decode_step([20], [[0, -1, 2, 3]], [1])    # page for position 20 invalid
    with pytest.raises(ValueError):
        m.decode_step([64], [[0, 1, 2, 3]], [1])     # beyond max_pages_per_seq
    with pytest.raises(ValueError):
        m.decode_step([3], [[7, 1, 2, 3]], [1])      # page id beyond the pool


def _planted_router(gains, w_down_sel=(1, 3)):
    d, E, k, fe = 16, len(gains), 2, 4
    shape = workload.ModelShape("moe_micro", n_layers=1, d_model=d, n_q_heads=2, n_kv_heads=1,
                                head_dim=8, ffn_dim=0, vocab=32, n_experts=E, top_k=k,
                                expert_ffn_dim=fe)
    w = zero_weights(shape)
    tok, j = 3, 2
    w["embed"][tok, j] = bf16_pattern(1.0)
    for e, gval in enumerate(gains):
        w["router"][0][e, j] = bf16_pattern(gval)
        w["w_gate"][0][e, 0, j] = bf16_pattern(1.0)
        w["w_up"][0][e, 0, j] = bf16_pattern(1.0)
        w["w_down"][0][e, e, 0] = bf16_pattern(1.0 if e in w_down_sel else 256.0)
    w["lm_head"][:d] = identity_rows(d, d)
    return shape, w, tok, j


def test_forced_routing_closed_form_and_margins():
    """A forced selection {1, 5} (logit gains 4 and 2, while expert 3 at gain 3 is
    left out) is used with the softmax of its own logits; the oracle still reports
    its own top-2 {1, 3}, that choice's margin (3 n - 2 n) and the forced set's
    margin (2 n - 3 n < 0, not a top-2 set). Expert 5's down row is 256, so its
    use shows in the closed form."""
    gains = [0.5, 4.0, 1.0, 3.0, 0.25, 2.0]
    shape, w, tok, j = _planted_router(gains)
    m = model(shape, w)
    n = 1.0 / math.sqrt(1.0 / shape.d_model + shape.rms_eps)
    ffn = n / (1 + math.exp(-n)) * n
    _, logits, rt = m.decode_step([0], [[0, 1, 2, 3]], [tok], route_in=[[[5, 1]]], want_route=True)
    assert rt["sel"][0, 0].tolist() == [1, 3]
    assert rt["gap"][0, 0] == pytest.approx(1.0 * n, rel=1e-12)
    assert rt["margin"][0, 0] == pytest.approx(-1.0 * n, rel=1e-12)
    w1 = 1.0 / (1.0 + math.exp(2.0 * n - 4.0 * n))
    h = np.zeros(shape.d_model)
    h[j] = 1.0
    h[1] += w1 * ffn
    h[5] += (1 - w1) * 256.0 * ffn
    want = h / math.sqrt(np.mean(h * h) + shape.rms_eps)
    assert np.allclose(logits[0, :shape.d_model], want, rtol=1e-12)


def test_forcing_the_own_selection_is_bitwise_neutral():
    """Handing the oracle its own top-k in its own order changes no bit of the step
    (in reverse order only the summation order of the expert outputs changes), and
    its margin is then the own gap; the per-request gap is the minimum of the
    per-layer gaps."""
    moe = dataclasses.replace(SMALL, n_layers=3, ffn_dim=0, n_experts=12, top_k=3, expert_ffn_dim=32)
    wm = workload.gen_weights(moe, seed=13)
    rng = np.random.default_rng(2)
    m1, m2 = model(moe, wm, 8, 4), model(moe, wm, 8, 4)
    _fill_random_kv(m1, rng)
    m2.kpool[...], m2.vpool[...] = m1.kpool, m1.vpool
    t1, l1, gap1, rt = m1.decode_step([20, 5], [[0, 1, 2, 3], [4, 5, 6, 7]], [3, 9],
                                      want_route_gap=True, want_route=True)
    t2, l2, rt2 = m2.decode_step([20, 5], [[0, 1, 2, 3], [4, 5, 6, 7]], [3, 9], route_in=rt["sel"],
                                 want_route=True)
    assert np.array_equal(l1, l2) and np.array_equal(t1, t2)
    m3 = model(moe, wm, 8, 4)
    m3.kpool[...], m3.vpool[...] = m1.kpool, m1.vpool  # (holds the step's own K/V rows: rewritten alike)
    _, l3 = m3.decode_step([20, 5], [[0, 1, 2, 3], [4, 5, 6, 7]], [3, 9],
                           route_in=rt["sel"][:, :, ::-1].copy())
    assert np.max(np.abs(l3 - l1)) <= 1e-13 * np.max(np.abs(l1))
    assert np.array_equal(rt2["sel"], rt["sel"])
    assert np.array_equal(rt2["margin"], rt["gap"])
    assert np.all(rt["gap"] > 0) and np.array_equal(gap1, rt["gap"].min(axis=1))
    # each own selection is the top-k of a full sort of some logits: margin >= 0
    for e in range(2):
        for l in range(3):
            assert len(set(rt["sel"][e, l].tolist())) == 3


def test_forced_routing_rejects_invalid_selections():
    moe = dataclasses.replace(SMALL, n_layers=1, ffn_dim=0, n_experts=6, top_k=2, expert_ffn_dim=32)
    wm = workload.gen_weights(moe, seed=3)
    m = model(moe, wm, 8, 4)
    for bad in ([[[1, 1]]], [[[0, 6]]], [[[-1, 2]]]):
        with pytest.raises(ValueError):
            m.decode_step([4], [[0, 1, 2, 3]], [1], route_in=bad)


def test_moe_weights_and_margin_closed_forms():
    r = np.array([0.0, 2.0, -1.0, 1.0, 2.0])
    # softmax of logits 2 and 1: e / (e + 1) and 1 / (e + 1), in the given order
    assert np.allclose(oracle.moe_weights(r, [3, 1]), [1 / (1 + math.e), math.e / (1 + math.e)], rtol=1e-15)
    # margins: {1, 4} vs the rest (best 1.0) -> 1.0; {1, 3} leaves 4 (2.0) out -> -1.0;
    # an equal logit on both sides -> 0
    assert oracle.moe_margin(r, [1, 4]) == 1.0
    assert oracle.moe_margin(r, [1, 3]) == -1.0
    assert oracle.moe_margin(r, [1]) == 0.0
    assert math.isinf(oracle.moe_margin(r, [0, 1, 2, 3, 4]))
