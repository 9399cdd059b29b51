"""Sampling limited to the top-k logits on the GPU against the oracle: the
kernel's token must be the oracle's (Gumbel-max over the oracle's k largest
logits, with the same noise) unless the oracle's choice is a near tie (the
k-th and (k+1)-th logits, or the two best candidates' scores, within
TIE_TOL, where the kernel's fp32 logits may decide either way)."""
import numpy as np
import pytest

import oracle
import workload

pytestmark = pytest.mark.gpu

TIE_TOL = 1e-3
LOGIT_REL_TOL = 2e-2


def _log(msg):
    print(f"  [topk] {msg}", flush=True)


def _run(shape, contexts, temps, ks, steps, seed):
    import torch
    from tests.scenario import Scenario, logits_row_err
    sc = Scenario(shape, contexts, steps, temps=temps, seed=seed)
    topk = torch.tensor(ks, dtype=torch.int32, device="cuda")
    n, compared, ties = len(contexts), 0, 0
    seqs, toks = list(contexts), list(sc.tokens)
    for s in range(steps):
        logits = torch.empty((n, shape.vocab), dtype=torch.float32, device="cuda")
        out = sc.dec.decode_step(torch.tensor(seqs, dtype=torch.int32, device="cuda"), sc.pt,
                                 torch.tensor(toks, dtype=torch.int32, device="cuda"), sc.temp_t,
                                 seed=seed, step=s, logits_out=logits, top_k=topk)
        torch.cuda.synchronize()
        g_tok = out.cpu().numpy()
        g_log = logits.cpu().numpy().astype(np.float64)
        _, o_log = sc.orc.decode_step(seqs, sc.pt_list, toks, temps, seed=seed, step=s)
        for b in range(n):
            assert logits_row_err(g_log[b], o_log[b]) <= LOGIT_REL_TOL, (s, b)
            T, k, l = temps[b], ks[b], o_log[b]
            ref = oracle.sample_topk(l, T, k, seed=seed, step=s, b=b)[0]
            srt = np.sort(l)[::-1]
            ambiguous = k < l.size and k > 0 and srt[k - 1] - srt[k] < TIE_TOL
            if T > 0 and 0 < k < l.size:
                cand = np.argsort(-l, kind="stable")[:k]
                sc_c = np.sort([l[i] / T + oracle.gumbel(seed, s, b, int(i)) for i in cand])[::-1]
                ambiguous = ambiguous or (k > 1 and sc_c[0] - sc_c[1] < TIE_TOL)
                assert int(g_tok[b]) in set(int(i) for i in np.argsort(-l, kind="stable")[:k + 4])
            elif T == 0:
                ambiguous = srt[0] - srt[1] < TIE_TOL
            if ambiguous:
                # several tokens are correct: the kernel's must be one of them
                ties += 1
                g = int(g_tok[b])
                if T == 0:
                    assert l[g] >= srt[0] - TIE_TOL, f"step {s} request {b}: greedy token {g} not a near maximum"
                else:
                    # a possible candidate, beating within TIE_TOL every logit that is
                    # a candidate under any reading of the tie
                    assert l[g] >= srt[k - 1] - TIE_TOL, f"step {s} request {b}: token {g} not a candidate"
                    sg = l[g] / T + oracle.gumbel(seed, s, b, g)
                    for i in np.nonzero(l > srt[k] + TIE_TOL)[0]:
                        si = l[i] / T + oracle.gumbel(seed, s, b, int(i))
                        assert sg >= si - TIE_TOL, f"step {s} request {b}: token {g} loses to {i}"
                continue
            assert int(g_tok[b]) == ref, f"step {s} request {b}: token {g_tok[b]} vs oracle {ref}"
            compared += 1
        toks, seqs = [int(t) for t in g_tok], [p + 1 for p in seqs]
    _log(f"{shape.name}: {compared} tokens compared, {ties} near ties")
    assert sc.dec.last_error()[0] == 0
    assert compared >= n * steps // 2


def test_topk_tiny_batch4():
    """k = 1 (greedy whatever the noise), 5, 3 at T = 0 (greedy), 16, at
    temperatures 0.8 .. 1.5, eight steps."""
    _run(workload.TINY, [40, 100, 7, 64], [0.8, 1.5, 0.0, 0.9], [1, 5, 3, 16], steps=8, seed=21)


def test_topk_dense2b_batch2():
    """Full-size vocabulary (32000: eight lm_head tiles per workgroup), k = 16
    and 2, three steps."""
    _run(workload.DENSE2B, [300, 41], [1.0, 0.7], [16, 2], steps=3, seed=5)


def test_topk_above_the_limit_is_clamped():
    """16 < k < vocab samples as k = 16 (the largest limited top-k); k >= vocab
    and k <= 0 as no limit."""
    import torch
    from tests.scenario import Scenario
    shape = workload.TINY
    sc = Scenario(shape, [30, 30, 30], 1, temps=[1.0, 1.0, 1.0], seed=4, with_oracle=False)

    def run(ks):
        out = sc.dec.decode_step(torch.tensor([30, 30, 30], dtype=torch.int32, device="cuda"), sc.pt,
                                 torch.tensor(sc.tokens, dtype=torch.int32, device="cuda"), sc.temp_t,
                                 seed=4, step=0, top_k=torch.tensor(ks, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        return out.cpu().numpy().copy()

    a = run([17, shape.vocab, -3])
    b = run([16, 0, 0])
    c = sc.dec.decode_step(torch.tensor([30, 30, 30], dtype=torch.int32, device="cuda"), sc.pt,
                           torch.tensor(sc.tokens, dtype=torch.int32, device="cuda"), sc.temp_t,
                           seed=4, step=0).cpu().numpy()
    assert np.array_equal(a, b) and a[1] == c[1] and a[2] == c[2]
    assert sc.dec.last_error()[0] == 0


@pytest.mark.parametrize("limit", [False, True])
def test_sampling_on_an_invalid_request(limit):
    """A request made invalid by its token, sampled at T > 0 (with or without a
    top-k limit), still gets token -1 and the error; its valid neighbour samples
    as without it."""
    import torch
    from tests.scenario import Scenario
    shape = workload.TINY
    sc = Scenario(shape, [30, 30], 1, temps=[1.0, 1.0], seed=6, with_oracle=False)
    topk = torch.tensor([4, 4], dtype=torch.int32, device="cuda") if limit else None

    def run(tokens):
        out = sc.dec.decode_step(torch.tensor([30, 30], dtype=torch.int32, device="cuda"), sc.pt,
                                 torch.tensor(tokens, dtype=torch.int32, device="cuda"), sc.temp_t,
                                 seed=6, step=0, top_k=topk)
        torch.cuda.synchronize()
        return out.cpu().numpy().copy()

    good = run(sc.tokens)
    assert sc.dec.last_error()[0] == 0
    t = run([shape.vocab + 5, sc.tokens[1]])
    rc, where = sc.dec.last_error()
    print(f"  [topk] invalid request, limit={limit}: error {rc} at {where}, tokens {t}", flush=True)
    assert rc == 5 and t[0] == -1 and t[1] == good[1]
