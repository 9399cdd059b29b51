"""Pins of the oracle's component functions against closed forms, invariants,
exact (rational) brute force and published vectors - never against a retyped
copy of the same formula."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_pattern(x: float) -> int:
    """bf16 bit pattern of a value that is exactly representable in bf16."""
    f = np.array([x], dtype=np.float32).view(np.uint32)[0]
    assert f & 0xFFFF == 0, x
    return int(f >> 16)


def to_bf16_exact(a):
    """Round to bf16-representable float32 by truncation of the low 16 bits of a
    float32 (the result is exactly representable; used only to build inputs)."""
    a = np.asarray(a, dtype=np.float32)
    return (a.view(np.uint32) & 0xFFFF0000).view(np.float32)


def as_bf16(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    assert np.all(a.view(np.uint32) & 0xFFFF == 0)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_vals(h) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ generator


def test_splitmix64_published_vector():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))
    gamma = 0x9E3779B97F4A7C15
    for k, want in enumerate(g["outputs"]):
        state = (g["seed"] + k * gamma) & 0xFFFFFFFFFFFFFFFF
        assert oracle.splitmix64(state) == int(want)
        assert workload.splitmix64(state) == int(want)


def test_generator_moments():
    """Irwin-Hall(4) draws scaled to sigma: mean ~0, std ~sigma (closed form of the
    uniform sum's variance)."""
    x = bf16_vals(workload.fill_normal_bf16((200000,), 0, 77, 0.02))
    assert abs(x.mean()) < 0.02 * 5 / math.sqrt(x.size)
    assert abs(x.std() / 0.02 - 1.0) < 0.01
    g = bf16_vals(workload.fill_normal_bf16((200000,), 0, 78, 0.02, mean=1.0))
    assert abs(g.mean() - 1.0) < 1e-3


# ----------------------------------------------------------------------- bf16


@pytest.mark.parametrize("x,expect", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (3.14159265, 0x4049),
    (1.0 + 2.0 ** -8, 0x3F80),                # halfway, ties to even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),            # halfway, ties to even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),   # just above halfway
    (1.0 + 2.0 ** -8 - 2.0 ** -30, 0x3F80),   # just below halfway
    (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
    (65280.0 + 128.0, 0x4780),                # rounds up across the exponent
])
def test_bf16_round_nearest_even(x, expect):
    assert oracle.f64_to_bf16(x) == expect


def test_bf16_roundtrip_all_finite_patterns():
    for h in list(range(0, 0x7F80, 7)) + list(range(0x8001, 0xFF80, 11)):
        assert oracle.f64_to_bf16(oracle.bf16_to_f64(h)) == h


# --------------------------------------------------------------------- matvec


def test_matvec_orientation_one_hot():
    """W = e_r e_c^T must give y = x_c e_r: catches a transposed operand."""
    rows, cols = 5, 7
    x = np.arange(1, cols + 1, dtype=np.float64) * 0.5
    for r, c in [(0, 0), (4, 6), (2, 5), (3, 1)]:
        W = np.zeros((rows, cols), dtype=np.uint16)
        W[r, c] = bf16_pattern(1.0)
        y = oracle.matvec(W, x)
        want = np.zeros(rows)
        want[r] = x[c]
        assert np.array_equal(y, want)


def test_matvec_against_exact_rational():
    """Exact rational brute force on a tiny random case; the fp64 result must lie
    within Higham's bound gamma_K * sum |w||x|."""
    rng = np.random.default_rng(1)
    rows, cols = 6, 33
    Wf = to_bf16_exact(rng.normal(0, 1, (rows, cols)))
    W = as_bf16(Wf)
    x = rng.normal(0, 1, cols)
    y = oracle.matvec(W, x)
    u = 2.0 ** -53
    gam = cols * u / (1 - cols * u)
    for r in range(rows):
        exact = sum(Fraction(float(Wf[r, c])) * Fraction(float(x[c])) for c in range(cols))
        bound = gam * sum(abs(float(Wf[r, c]) * x[c]) for c in range(cols))
        assert abs(Fraction(y[r]) - exact) <= Fraction(bound) + Fraction(1, 10 ** 30)


# -------------------------------------------------------------------- rmsnorm


@pytest.mark.parametrize("c,eps", [(0.5, 1e-5), (3.0, 1e-5), (1e-3, 1e-5), (2.0, 0.0)])
def test_rmsnorm_constant_vector_closed_form(c, eps):
    d = 64
    g = as_bf16(to_bf16_exact(np.linspace(0.5, 1.5, d)))
    y = oracle.rmsnorm(np.full(d, c), g, eps)
    want = bf16_vals(g) * c / math.sqrt(c * c + eps)
    assert np.allclose(y, want, rtol=1e-14, atol=0)


def test_rmsnorm_norm_identity_and_scale():
    rng = np.random.default_rng(2)
    d, eps = 96, 1e-5
    x = rng.normal(0, 2, d)
    g = as_bf16(to_bf16_exact(rng.uniform(0.5, 1.5, d)))
    y = oracle.rmsnorm(x, g, eps)
    ms = float(np.mean(x * x))
    assert math.isclose(float(np.sum((y / bf16_vals(g)) ** 2)), d * ms / (ms + eps), rel_tol=1e-12)
    # scale invariance when eps is negligible: rmsnorm(a x) == rmsnorm(x) for a > 0
    y0 = oracle.rmsnorm(x, g, 0.0)
    y1 = oracle.rmsnorm(7.0 * x, g, 0.0)
    assert np.allclose(y0, y1, rtol=1e-13)
    # gains enter elementwise
    y2 = oracle.rmsnorm(x, as_bf16(np.ones(d, dtype=np.float32)), eps)
    assert np.allclose(y, y2 * bf16_vals(g), rtol=1e-14)


# ----------------------------------------------------------------------- RoPE


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(3)
    v = rng.normal(0, 1, 3 * 16)
    assert np.array_equal(oracle.rope(v, 3, 16, 0, 10000.0), v)


@pytest.mark.parametrize("dh,i,pos", [(16, 0, 5), (16, 3, 7), (64, 31, 123), (128, 10, 8191)])
def test_rope_unit_vectors_closed_form(dh, i, pos):
    """Rotate-half: e_i -> cos(a) e_i + sin(a) e_{i+dh/2}, e_{i+dh/2} -> -sin(a) e_i +
    cos(a) e_{i+dh/2}, a = pos * base^(-2i/dh)."""
    base, half = 10000.0, dh // 2
    a = pos * base ** (-2.0 * i / dh)
    e = np.zeros(dh)
    e[i] = 1.0
    y = oracle.rope(e, 1, dh, pos, base)
    want = np.zeros(dh)
    want[i], want[i + half] = math.cos(a), math.sin(a)
    assert np.allclose(y, want, atol=1e-12)
    e = np.zeros(dh)
    e[i + half] = 1.0
    y = oracle.rope(e, 1, dh, pos, base)
    want = np.zeros(dh)
    want[i], want[i + half] = -math.sin(a), math.cos(a)
    assert np.allclose(y, want, atol=1e-12)


def test_rope_relative_position_and_norm():
    rng = np.random.default_rng(4)
    dh = 32
    q, k = rng.normal(0, 1, dh), rng.normal(0, 1, dh)

    def dot(a, b):
        return float(np.dot(oracle.rope(q, 1, dh, a, 10000.0), oracle.rope(k, 1, dh, b, 10000.0)))

    assert math.isclose(dot(10, 3), dot(107, 100), rel_tol=1e-9, abs_tol=1e-9)
    assert math.isclose(dot(0, 0), float(np.dot(q, k)), rel_tol=1e-12)
    r = oracle.rope(q, 1, dh, 999, 10000.0)
    h = dh // 2
    assert np.allclose(r[:h] ** 2 + r[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-12)
    twice = oracle.rope(oracle.rope(q, 1, dh, 40, 10000.0), 1, dh, 60, 10000.0)
    assert np.allclose(twice, oracle.rope(q, 1, dh, 100, 10000.0), atol=1e-12)


# -------------------------------------------------------------------- SwiGLU


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(oracle.silu(math.log(3.0)), 0.75 * math.log(3.0), rel_tol=1e-15)
    for z in (0.1, 1.0, 2.5, 7.0, 30.0):
        assert math.isclose(oracle.silu(z) - oracle.silu(-z), z, rel_tol=1e-14)
    assert math.isclose(oracle.silu(50.0), 50.0, rel_tol=1e-15)


def test_swiglu_ffn_one_hot_closed_form():
    """gate/up pick n2[c]; down maps feature f back to row r: y_r = silu(n_c) n_c."""
    d, f = 8, 6
    n2 = np.linspace(-1.5, 2.0, d)
    for (c, feat, r) in [(0, 0, 0), (3, 5, 7), (7, 2, 1)]:
        wg = np.zeros((f, d), dtype=np.uint16)
        wu = np.zeros((f, d), dtype=np.uint16)
        wd = np.zeros((d, f), dtype=np.uint16)
        wg[feat, c] = bf16_pattern(1.0)
        wu[feat, c] = bf16_pattern(2.0)
        wd[r, feat] = bf16_pattern(-1.0)
        y = oracle.swiglu_ffn(wg, wu, wd, n2)
        z = n2[c]
        want = np.zeros(d)
        want[r] = -(z / (1 + math.exp(-z))) * 2.0 * z
        assert np.allclose(y, want, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ attention


def _pool(n_pages, hkv, dh, rng, scale=1.0):
    k = as_bf16(to_bf16_exact(rng.normal(0, scale, (n_pages, hkv, 16, dh))))
    v = as_bf16(to_bf16_exact(rng.normal(0, scale, (n_pages, hkv, 16, dh))))
    return k, v


def test_attention_zero_query_is_mean_of_values():
    rng = np.random.default_rng(5)
    kp, vp = _pool(6, 2, 8, rng)
    pages = [4, 1, 5]
    pos = 40
    o, probs = oracle.attend(kp, vp, pages, 0, pos, 1, np.zeros(8))
    assert np.allclose(probs, 1.0 / (pos + 1), rtol=1e-14)
    vals = np.array([bf16_vals(vp[pages[j // 16], 1, j % 16]) for j in range(pos + 1)])
    assert np.allclose(o, vals.mean(axis=0), rtol=1e-12, atol=1e-15)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(6)
    kp, vp = _pool(3, 1, 16, rng)
    o, probs = oracle.attend(kp, vp, [2], 0, 0, 0, rng.normal(0, 3, 16))
    assert probs[0] == 1.0
    assert np.array_equal(o, bf16_vals(vp[2, 0, 0]))


def test_attention_two_keys_known_softmax():
    """q.K0/sqrt(dh) - q.K1/sqrt(dh) = ln 3 gives probabilities (3/4, 1/4)."""
    dh = 4
    kp = np.zeros((1, 1, 16, dh), dtype=np.uint16)
    vp = np.zeros((1, 1, 16, dh), dtype=np.uint16)
    kp[0, 0, 0, 0] = bf16_pattern(1.0)
    vp[0, 0, 0] = as_bf16(np.array([1.0, 0, 0, 2.0], dtype=np.float32))
    vp[0, 0, 1] = as_bf16(np.array([0, 1.0, 0, -2.0], dtype=np.float32))
    q = np.array([2.0 * math.log(3.0), 0.0, 0.0, 0.0])  # sqrt(dh) = 2
    o, probs = oracle.attend(kp, vp, [0], 0, 1, 0, q)
    assert np.allclose(probs, [0.75, 0.25], rtol=1e-14)
    assert np.allclose(o, [0.75, 0.25, 0.0, 1.0], rtol=1e-14, atol=1e-15)


def test_attention_paged_equals_contiguous_bitwise():
    rng = np.random.default_rng(7)
    hkv, dh, pos = 2, 16, 70
    n_log = pos // 16 + 1
    kc, vc = _pool(n_log, hkv, dh, rng)           # contiguous: page i holds positions 16i..
    perm = [7, 2, 9, 0, 4]
    kp = np.zeros((10, hkv, 16, dh), dtype=np.uint16)
    vp = np.zeros_like(kp)
    kp[perm] = kc
    vp[perm] = vc
    q = rng.normal(0, 1, dh)
    for lo in (0, 13):
        oc, pc = oracle.attend(kc, vc, list(range(n_log)), lo, pos, 1, q)
        op, pp = oracle.attend(kp, vp, perm, lo, pos, 1, q)
        assert np.array_equal(oc, op) and np.array_equal(pc, pp)


def test_attention_probs_sum_to_one_and_window_cases():
    rng = np.random.default_rng(8)
    kp, vp = _pool(8, 1, 32, rng, scale=2.0)
    pages = [3, 6, 0, 7, 1, 2, 5, 4]
    q = rng.normal(0, 2, 32)
    pos = 100
    o_full, p_full = oracle.attend(kp, vp, pages, 0, pos, 0, q)
    assert abs(p_full.sum() - 1.0) < 1e-14 * (pos + 1)
    # window >= pos + 1 reduces to full attention
    assert oracle.window_lo(pos, pos + 1) == 0 and oracle.window_lo(pos, 5000) == 0
    assert oracle.window_lo(pos, 0) == 0
    # window 1 keeps only the current key: o = v_pos
    lo = oracle.window_lo(pos, 1)
    assert lo == pos
    o1, _ = oracle.attend(kp, vp, pages, lo, pos, 0, q)
    assert np.array_equal(o1, bf16_vals(vp[pages[pos // 16], 0, pos % 16]))
    # window W keeps exactly W keys
    assert oracle.window_lo(pos, 16) == pos - 15
    assert oracle.window_lo(3, 16) == 0


# -------------------------------------------------------------------- sampler


def test_greedy_argmax_and_ties():
    l = np.array([0.1, 2.0, -1.0, 2.0, 1.9])
    assert oracle.sample(l, 0.0)[0] == 1           # exact tie -> lowest index
    l2 = l.copy()
    l2[3] = 2.0 + 1e-12
    assert oracle.sample(l2, 0.0)[0] == 3


def test_temperature_to_zero_is_greedy():
    rng = np.random.default_rng(9)
    for s in range(20):
        l = rng.normal(0, 1, 50)
        assert oracle.sample(l, 1e-9, seed=5, step=s)[0] == int(np.argmax(l))


def test_gumbel_noise_mean_and_counter_definition():
    g = np.array([oracle.gumbel(11, 3, 2, i) for i in range(40000)])
    euler_gamma = 0.5772156649015329  # mean of the standard Gumbel distribution
    assert abs(g.mean() - euler_gamma) < 5 * (math.pi / math.sqrt(6)) / math.sqrt(g.size)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    # u = (2 (h >> 41) + 1) / 2^24 with h = SM(SM(SM(SM(seed)+step)+b)+i)
    sm = oracle.splitmix64
    h = sm(sm(sm(sm(11) + 3) + 2) + 5)
    u = (2 * (h >> 41) + 1) / 2.0 ** 24
    assert oracle.gumbel(11, 3, 2, 5) == -math.log(-math.log(u))


def test_temperature_sampler_chi_square():
    """Gumbel-max frequencies over many steps follow softmax(l / T)."""
    l = np.array([0.0, 0.5, -0.3, 1.2, 0.9, -1.0, 0.2, 0.4])
    T = 0.7
    N = 20000
    counts = np.zeros(l.size)
    for s in range(N):
        counts[oracle.sample(l, T, seed=123, step=s, b=1)[0]] += 1
    p = np.exp(l / T - np.max(l / T))
    p /= p.sum()
    chi2 = float(np.sum((counts - N * p) ** 2 / (N * p)))
    from scipy.stats import chi2 as chi2dist
    assert chi2dist.sf(chi2, l.size - 1) > 1e-4, chi2


def test_topk_sampler_reduces_to_greedy_and_to_the_full_sampler():
    """top_k = 1 is greedy whatever the noise; top_k >= V (or 0) is the unlimited
    sampler; greedy ignores top_k."""
    rng = np.random.default_rng(5)
    for s in range(50):
        l = rng.normal(size=40)
        assert oracle.sample_topk(l, 0.8, 1, seed=9, step=s, b=2)[0] == int(np.argmax(l))
        full = oracle.sample(l, 0.8, seed=9, step=s, b=2)[0]
        assert oracle.sample_topk(l, 0.8, 40, seed=9, step=s, b=2)[0] == full
        assert oracle.sample_topk(l, 0.8, 0, seed=9, step=s, b=2)[0] == full
        assert oracle.sample_topk(l, 0.0, 3, seed=9, step=s, b=2)[0] == int(np.argmax(l))


def test_topk_sampler_stays_in_the_top_k_with_index_ties():
    """The token is always one of the k largest logits; among equal logits at
    the boundary the lower indices are the candidates."""
    l = np.array([0.3, 2.0, 1.0, 1.0, 1.0, -0.5, 1.0, 0.9])
    allowed = {1, 2, 3}  # 2.0, then the three lowest-index 1.0s take k = 3: indices 1, 2, 3
    seen = set()
    for s in range(3000):
        t = oracle.sample_topk(l, 5.0, 3, seed=1, step=s, b=0)[0]
        assert t in allowed, (s, t)
        seen.add(t)
    assert seen == allowed


def test_topk_sampler_chi_square():
    """Frequencies follow softmax(l / T) restricted to the k largest logits
    (the Gumbel-max argument applied to the candidate set)."""
    l = np.array([0.0, 0.5, -0.3, 1.2, 0.9, -1.0, 0.2, 0.4])
    T, k, N = 0.7, 3, 20000
    top = [3, 4, 1]
    counts = np.zeros(l.size)
    for s in range(N):
        counts[oracle.sample_topk(l, T, k, seed=77, step=s, b=3)[0]] += 1
    assert counts.sum() == counts[top].sum()
    p = np.exp(l[top] / T - np.max(l[top] / T))
    p /= p.sum()
    chi2 = float(np.sum((counts[top] - N * p) ** 2 / (N * p)))
    from scipy.stats import chi2 as chi2dist
    assert chi2dist.sf(chi2, k - 1) > 1e-4, chi2


# ------------------------------------------------------------------------ MoE


def test_moe_route_matches_full_sort():
    rng = np.random.default_rng(10)
    for _ in range(20):
        r = rng.normal(0, 1, 128)
        r[rng.integers(0, 128, 4)] = r[5]          # plant ties
        idx, w = oracle.moe_route(r, 8)
        order = sorted(range(128), key=lambda e: (-r[e], e))[:8]
        assert list(idx) == order
        assert abs(w.sum() - 1.0) < 1e-15
        sel = r[order]
        p = np.exp(sel - sel.max())
        assert np.allclose(w, p / p.sum(), rtol=1e-14)
        assert np.all(np.diff(w) <= 1e-16)
