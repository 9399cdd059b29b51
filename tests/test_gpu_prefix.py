"""Prefix cache on the GPU: reference counts, copy-on-write of a shared page,
and a batch whose requests share their prefix pages computing bit-identically
to the same batch with private copies of those pages (the decode step reads
pages by id, so only the ids differ between the two runs)."""
import numpy as np
import pytest

import workload

pytestmark = pytest.mark.gpu

SEED = 11


def _log(msg):
    print(f"  [prefix] {msg}", flush=True)


@pytest.fixture(scope="module")
def env():
    from decode_persistent_step_amd import session
    shape = workload.TINY
    w = workload.gen_weights(shape, seed=SEED)
    return shape, session.upload_weights(w)


def _decoder(env, n_pages, mpps):
    from decode_persistent_step_amd import Decoder
    shape, dev_w = env
    return Decoder(shape, dev_w, n_pages, mpps, 2)


def test_refcounts_and_copy_on_write(env):
    from decode_persistent_step_amd import MkError, session
    shape, _ = env
    _log("reference counts")
    dec = _decoder(env, n_pages=8, mpps=4)
    a = dec.kv_alloc(3)
    assert [dec.kv_refcount(p) for p in a] == [1, 1, 1]
    dec.kv_ref(a[:2])
    assert [dec.kv_refcount(p) for p in a] == [2, 2, 1]
    free_id = [p for p in range(8) if p not in a][0]
    with pytest.raises(MkError):
        dec.kv_ref([a[0], a[0]])        # repeated id
    with pytest.raises(MkError):
        dec.kv_ref([a[2], free_id])     # a free page
    with pytest.raises(MkError):
        dec.kv_unref([free_id])
    assert [dec.kv_refcount(p) for p in a] == [2, 2, 1]  # rejected calls changed nothing
    assert dec.kv_refcount(99) == -1 and dec.kv_refcount(free_id) == 0

    _log("copy-on-write")
    n = 16 * 1  # every slot of the page
    k = [workload.gen_kv(shape, 0, l, 0, n, seed=SEED) for l in range(shape.n_layers)]
    v = [workload.gen_kv(shape, 0, l, 1, n, seed=SEED) for l in range(shape.n_layers)]
    for l in range(shape.n_layers):
        session.prefill_kv(dec, l, [a[1]], k[l], v[l])
    assert dec.kv_cow(a[2]) == a[2]     # sole holder: the page itself, no copy
    avail = dec.kv_available()
    c = dec.kv_cow(a[1])                # shared: a private copy
    assert c not in a and dec.kv_available() == avail - 1
    assert dec.kv_refcount(c) == 1 and dec.kv_refcount(a[1]) == 1
    for l in range(shape.n_layers):
        for kv, ref in ((0, k[l]), (1, v[l])):
            got = session.read_kv_rows(dec, l, kv, session.slots_for([c], 0, n))
            assert np.array_equal(got, ref), f"layer {l} kv {kv}: copy differs"

    _log("release")
    dec.kv_unref(a[:2])                 # a[0]: 2 -> 1; a[1]: 1 -> 0, back to the free list
    assert dec.kv_refcount(a[0]) == 1 and dec.kv_refcount(a[1]) == 0
    with pytest.raises(MkError):
        dec.kv_free([a[1]])             # not held any more
    dec.kv_free([a[0], a[2], c])
    assert dec.kv_available() == 8

    _log("copy-on-write without a free page")
    got = dec.kv_alloc(8)
    dec.kv_ref([got[0]])
    with pytest.raises(MkError):
        dec.kv_cow(got[0])
    assert dec.kv_refcount(got[0]) == 2 and dec.kv_available() == 0
    dec.kv_unref([got[0]])
    dec.kv_free(got)
    dec.close()


def test_shared_prefix_matches_private_copies(env):
    """Two requests with the same 87-position prefix (five full pages and a tail
    of 7) and different next tokens, greedy, 20 steps (the tail fills after 9 and
    the requests append into pages of their own). Run once with private copies
    of the prefix and once with the prefix pages shared, the tail made private by
    copy-on-write: every step's tokens and logits must be bit-identical, and the
    shared run must match the oracle stepped on the same shared page table
    (logits, tokens with the tie rule, and the K/V rows each step appends)."""
    import oracle
    import torch
    from decode_persistent_step_amd import session
    from tests.scenario import LOGIT_REL_TOL, TIE_TOL, KV_ABS_TOL, KV_DEEP_TOL, bf16_f64, logits_row_err
    shape, _ = env
    ctx, steps = 87, 20
    need = workload.pages_needed(ctx, steps)
    n_pre = (ctx + 15) // 16
    k = [workload.gen_kv(shape, 0, l, 0, ctx, seed=SEED) for l in range(shape.n_layers)]
    v = [workload.gen_kv(shape, 0, l, 1, ctx, seed=SEED) for l in range(shape.n_layers)]
    host_w = workload.gen_weights(shape, seed=SEED)

    def run(shared: bool):
        n_pages = 2 * need + 2
        dec = _decoder(env, n_pages=n_pages, mpps=need)
        pre = dec.kv_alloc(n_pre)
        for l in range(shape.n_layers):
            session.prefill_kv(dec, l, pre, k[l], v[l])
        if shared:
            dec.kv_ref(pre)                          # request 1 holds the prefix too
            rows1 = pre[:-1] + [dec.kv_cow(pre[-1])]  # and appends to its own tail
            assert all(dec.kv_refcount(p) == 2 for p in pre[:-1]) and dec.kv_refcount(pre[-1]) == 1
        else:
            rows1 = dec.kv_alloc(n_pre)
            for l in range(shape.n_layers):
                session.prefill_kv(dec, l, rows1, k[l], v[l])
        rows0 = list(pre) + dec.kv_alloc(need - n_pre)
        rows1 = list(rows1) + dec.kv_alloc(need - n_pre)
        pt = session.page_table_tensor([rows0, rows1], need)
        orc = None
        if shared:
            # the oracle on the same shared page table, its own pool filled alike
            orc = oracle.OracleModel(shape, host_w, n_pages, need)
            for l in range(shape.n_layers):
                orc.prefill_from(rows0[:n_pre], l, k[l], v[l])
                orc.prefill_from(rows1[:n_pre], l, k[l], v[l])
            pt_np = pt.cpu().numpy()
        seq, toks = [ctx, ctx], [5, 77]
        temps = torch.zeros(2, dtype=torch.float32, device="cuda")
        outs, worst = [], 0.0
        for s in range(steps):
            logits = torch.empty((2, shape.vocab), dtype=torch.float32, device="cuda")
            out = dec.decode_step(torch.tensor(seq, dtype=torch.int32, device="cuda"), pt,
                                  torch.tensor(toks, dtype=torch.int32, device="cuda"), temps,
                                  seed=3, step=s, logits_out=logits)
            torch.cuda.synchronize()
            t = out.cpu().numpy().copy()
            g_log = logits.cpu().numpy().copy()
            outs.append((t, g_log))
            if orc is not None:
                o_tok, o_log = orc.decode_step(seq, pt_np, toks, [0.0, 0.0], seed=3, step=s)
                for b in range(2):
                    e = logits_row_err(g_log[b].astype(np.float64), o_log[b])
                    worst = max(worst, e)
                    assert e <= LOGIT_REL_TOL, f"step {s} request {b}: logits rel err {e:.3e}"
                    if int(t[b]) != int(o_tok[b]):
                        gap = abs(o_log[b][int(t[b])] - o_log[b][int(o_tok[b])])
                        assert gap <= TIE_TOL, f"step {s} request {b}: token {t[b]} vs oracle {o_tok[b]}"
                # the rows this step appended: right slots (each request's own page), oracle's values
                rows = [rows0, rows1]
                slots = np.asarray([int(rows[b][seq[b] // 16]) * 16 + seq[b] % 16 for b in range(2)], np.int32)
                assert slots[0] != slots[1]
                for l in range(shape.n_layers):
                    for kv in (0, 1):
                        g = session.read_kv_rows(dec, l, kv, slots)
                        pool = orc.kpool if kv == 0 else orc.vpool
                        o = np.stack([pool[l, sl // 16, :, sl % 16] for sl in slots])
                        gf, of = bf16_f64(g), bf16_f64(o)
                        rms = np.sqrt(np.mean(of * of, axis=-1, keepdims=True))
                        tol = np.maximum(np.abs(gf), np.abs(of)) * 2.0 ** -7 + \
                            (KV_ABS_TOL if l == 0 else KV_DEEP_TOL) * rms
                        assert not (np.abs(gf - of) > tol).any(), f"step {s} layer {l} kv {kv}: K/V off"
            toks, seq = [int(x) for x in t], [p + 1 for p in seq]  # teacher forcing: the GPU's tokens
        assert dec.last_error()[0] == 0
        dec.close()
        if orc is not None:
            _log(f"shared prefix vs oracle: worst logits rel err {worst:.2e} over {steps} steps")
        return outs

    _log("private copies")
    a = run(False)
    _log("shared prefix (and the oracle on the shared page table)")
    b = run(True)
    for s in range(steps):
        assert np.array_equal(a[s][0], b[s][0]), f"step {s}: tokens {a[s][0]} vs {b[s][0]}"
        assert np.array_equal(a[s][1], b[s][1]), f"step {s}: logits differ"
    # the requests diverge, so a tail page written by both would have shown
    assert any(a[s][0][0] != a[s][0][1] for s in range(steps))
    assert not np.array_equal(a[0][1][0], a[0][1][1])
