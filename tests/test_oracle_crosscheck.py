"""Cross-check of the C oracle's whole decode step against a second, vectorised
numpy fp64 implementation of the same definition, on the tiny 2-layer model
with a mixed greedy/temperature batch. This is a consistency check between two
implementations (written separately, different summation orders), not a pin:
the pins are in test_oracle_components.py and test_oracle_step.py."""
import dataclasses
import math

import numpy as np

import oracle
import workload


def _f(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_rne(x):
    """fp64 -> bf16 bits via exact fp32 intermediate is *not* used: round the fp64
    value to 8 significant bits with numpy's round-half-even on the mantissa."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, |m| in [0.5, 1)
    q = np.round(m * 256.0) / 256.0         # numpy rounds half to even
    return (np.ldexp(q, e).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def numpy_step(shape, w, kpool, vpool, seq_lens, pt, toks_in, temps, seed, step):
    L, d, Hq, Hkv, dh = shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G = Hq // Hkv
    half = dh // 2
    inv = shape.rope_base ** (-2.0 * np.arange(half) / dh)
    out_logits = []
    out_toks = []

    def rms(x, g):
        return x / np.sqrt(np.mean(x * x) + shape.rms_eps) * _f(g)

    def rope(v, p):
        v = v.reshape(-1, dh)
        a = p * inv
        c, s = np.cos(a), np.sin(a)
        x0, x1 = v[:, :half].copy(), v[:, half:].copy()
        return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=1)

    for b, p in enumerate(seq_lens):
        x = _f(w["embed"][toks_in[b]])
        for l in range(L):
            n = rms(x, w["attn_norm"][l])
            q = rope(_f(w["wq"][l]) @ n, p)
            k = rope(_f(w["wk"][l]) @ n, p)
            v = (_f(w["wv"][l]) @ n).reshape(Hkv, dh)
            pg = pt[b][p // 16]
            kpool[l, pg, :, p % 16] = _bf16_rne(k)
            vpool[l, pg, :, p % 16] = _bf16_rne(v)
            win = shape.windows()[l]
            lo = max(0, p - win + 1) if win > 0 else 0
            pos = np.arange(lo, p + 1)
            pages = np.asarray(pt[b])[pos // 16]
            K = _f(kpool[l, pages, :, pos % 16])      # [n][Hkv][dh]
            V = _f(vpool[l, pages, :, pos % 16])
            o = np.empty((Hq, dh))
            for h in range(Hq):
                s = K[:, h // G] @ q[h] / math.sqrt(dh)
                e = np.exp(s - s.max())
                o[h] = (e / e.sum()) @ V[:, h // G]
            hres = x + _f(w["wo"][l]) @ o.reshape(-1)
            n2 = rms(hres, w["ffn_norm"][l])
            g = _f(w["w_gate"][l]) @ n2
            u = _f(w["w_up"][l]) @ n2
            x = hres + _f(w["w_down"][l]) @ (g / (1 + np.exp(-g)) * u)
        logits = _f(w["lm_head"]) @ rms(x, w["final_norm"])
        out_logits.append(logits)
        if temps[b] > 0:
            gum = np.array([oracle.gumbel(seed, step, b, i) for i in range(logits.size)])
            out_toks.append(int(np.argmax(logits / temps[b] + gum)))
        else:
            out_toks.append(int(np.argmax(logits)))
    return np.array(out_toks), np.array(out_logits)


def test_c_oracle_matches_numpy_implementation():
    shape = dataclasses.replace(workload.TINY, window=[32, 0])
    w = workload.gen_weights(shape)
    n_pages, mpps = 40, 12
    m = oracle.OracleModel(shape, w, n_pages, mpps)
    rng = np.random.default_rng(0)
    seq = [128, 77]
    pt = [list(range(0, 12)), list(range(20, 32))]
    for b, p in enumerate(seq):
        for l in range(shape.n_layers):
            m.prefill_from(pt[b], l, workload.gen_kv(shape, b, l, 0, p), workload.gen_kv(shape, b, l, 1, p))
    kp, vp = m.kpool.copy(), m.vpool.copy()
    temps = [0.0, 0.7]
    toks_in = workload.WORKLOADS["tiny"].initial_tokens() + [5]
    t_c, l_c = m.decode_step(seq, pt, toks_in, temps, seed=3, step=2)
    t_n, l_n = numpy_step(shape, w, kp, vp, seq, pt, toks_in, temps, 3, 2)
    assert np.max(np.abs(l_c - l_n)) <= 1e-10 * np.max(np.abs(l_n))
    assert list(t_c) == list(t_n)
    # K/V written by both implementations agree to the bit (or within one bf16 ulp
    # if a value straddles a rounding boundary)
    diff = np.abs(kp.astype(np.int32) - m.kpool.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).sum() <= 2
