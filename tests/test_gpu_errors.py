"""GPU tests of the error conventions of include/mk.h: bad requests are reported
per request without disturbing the others, an expired bounded wait ends the
launch with MK_ERR_DEVICE_TIMEOUT instead of hanging, and the page allocator is
all-or-nothing. Every condition is forced from the host; no kernel faults."""
import sys

import numpy as np
import pytest

import workload

pytestmark = pytest.mark.gpu

MK_ERR_INVALID_ARG, MK_ERR_OOM, MK_ERR_BAD_PAGE, MK_ERR_DEVICE_TIMEOUT = 1, 3, 5, 6


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_persistent_step_amd as mk
    mk.lib()
    return mk


def _scenario(contexts, steps=2, **kw):
    from tests.scenario import Scenario
    return Scenario(workload.TINY, contexts, steps, **kw)


def _step(sc, seq, pt, tok, logits=True):
    import torch
    n = len(seq)
    seq_t = torch.tensor(seq, dtype=torch.int32).cuda()
    tok_t = torch.tensor(tok, dtype=torch.int32).cuda()
    pt_t = torch.from_numpy(np.ascontiguousarray(pt)).cuda()
    lg = torch.empty((n, sc.shape.vocab), dtype=torch.float32).cuda() if logits else None
    out = sc.dec.decode_step(seq_t, pt_t, tok_t, sc.temp_t[:n], seed=sc.seed, step=0, logits_out=lg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lg.cpu().numpy() if logits else None)


def test_bad_page_id_is_reported_per_request(mk):
    _log("[errors] bad page id in request 1")
    sc = _scenario([40, 70])
    good_tok, good_log = _step(sc, sc.seq, sc.pt_list, sc.tokens)
    assert sc.dec.last_error() == (0, -1)
    pt = sc.pt_list.copy()
    pt[1, 2] = sc.n_pages + 7  # a page the request attends over
    tok, log = _step(sc, sc.seq, pt, sc.tokens)
    rc, where = sc.dec.last_error()
    assert rc == MK_ERR_BAD_PAGE
    assert tok[1] == -1
    # the other request is computed exactly as without the bad neighbour
    assert tok[0] == good_tok[0]
    assert np.array_equal(log[0], good_log[0])
    assert sc.dec.last_error() == (0, -1)  # cleared by the read


def test_bad_token_and_length_are_reported(mk):
    _log("[errors] out-of-range token and sequence length")
    sc = _scenario([40, 70, 12])
    tok = list(sc.tokens)
    tok[1] = workload.TINY.vocab + 3
    seq = list(sc.seq)
    seq[2] = -5
    out, _ = _step(sc, seq, sc.pt_list, tok)
    rc, where = sc.dec.last_error()
    assert rc == MK_ERR_BAD_PAGE
    assert where in (1, 2)
    assert out[1] == -1 and out[2] == -1 and out[0] >= 0


def test_bad_temperature_is_reported_per_request(mk):
    """A NaN or negative temperature makes only that request invalid (token -1,
    MK_ERR_BAD_PAGE latched); the others get the same tokens, and logits equal up
    to rounding: an invalid request takes no part in the attention partition, so
    the others' K/V splits, and the order of their sums, change."""
    import torch
    _log("[errors] NaN and negative temperatures")
    sc = _scenario([40, 70, 25], temps=[0.0, 0.9, 0.0])

    def run(temps):
        lg = torch.empty((3, sc.shape.vocab), dtype=torch.float32).cuda()
        out = sc.dec.decode_step(torch.tensor(sc.seq, dtype=torch.int32).cuda(), sc.pt,
                                 torch.tensor(sc.tokens, dtype=torch.int32).cuda(),
                                 torch.tensor(temps, dtype=torch.float32).cuda(), seed=sc.seed,
                                 step=0, logits_out=lg)
        torch.cuda.synchronize()
        return out.cpu().numpy().copy(), lg.cpu().numpy().copy()

    good_tok, good_log = run([0.0, 0.9, 0.0])
    assert sc.dec.last_error() == (0, -1)
    for bad in (float("nan"), -1.0):
        tok, log = run([0.0, 0.9, bad])
        rc, where = sc.dec.last_error()
        assert rc == MK_ERR_BAD_PAGE and where == 2
        assert tok[2] == -1
        assert tok[0] == good_tok[0] and tok[1] == good_tok[1]
        assert np.max(np.abs(log[:2] - good_log[:2])) <= 1e-4 * np.max(np.abs(good_log[:2]))
    assert sc.dec.last_error() == (0, -1)


def test_single_invalid_request(mk):
    """Batch 1 whose only request is invalid: the launch ends normally with
    token -1 and the error; the next valid step matches the oracle."""
    _log("[errors] batch 1, invalid token")
    sc = _scenario([50])
    out, _ = _step(sc, sc.seq, sc.pt_list, [workload.TINY.vocab + 1], logits=False)
    rc, where = sc.dec.last_error()
    assert rc == MK_ERR_BAD_PAGE and where == 0 and out[0] == -1
    r = sc.step(run_oracle=True)
    sc.check(r)
    assert sc.dec.last_error() == (0, -1)


def test_invalid_request_in_a_moe_batch(mk):
    """MoE (routing, expert sums by atomics) with an invalid request in the
    batch: its token is -1, the error is latched, and the other request matches
    the oracle."""
    from tests.scenario import Scenario
    import torch
    _log("[errors] MoE batch 2, invalid token in request 0")
    sc = Scenario(workload.TINY_MOE, [33, 61], 2)
    seq_t = torch.tensor(sc.seq, dtype=torch.int32).cuda()
    tok = [workload.TINY_MOE.vocab + 2, sc.tokens[1]]
    lg = torch.empty((2, workload.TINY_MOE.vocab), dtype=torch.float32).cuda()
    out = sc.dec.decode_step(seq_t, sc.pt, torch.tensor(tok, dtype=torch.int32).cuda(), sc.temp_t,
                             seed=sc.seed, step=0, logits_out=lg)
    torch.cuda.synchronize()
    rc, where = sc.dec.last_error()
    assert rc == MK_ERR_BAD_PAGE and where == 0 and int(out[0]) == -1
    ref = sc.orc.decode_step([sc.seq[1]], sc.pt_list[[1]], [tok[1]], [0.0], seed=sc.seed, step=0)
    from tests.scenario import logits_row_err
    assert logits_row_err(lg.cpu().numpy()[1].astype(np.float64), ref[1][0]) <= 2e-2
    assert sc.dec.last_error() == (0, -1)


def test_expired_wait_ends_the_launch(mk):
    _log("[errors] 1 us wait limit: the launch must end with a timeout, then recover")
    sc = _scenario([100])
    sc.dec.set_wait_limit(1)
    _step(sc, sc.seq, sc.pt_list, sc.tokens, logits=False)
    rc, where = sc.dec.last_error()
    assert rc == MK_ERR_DEVICE_TIMEOUT
    sc.dec.set_wait_limit(2_000_000)
    # the next step runs normally and matches the oracle
    r = sc.step(run_oracle=True)
    sc.check(r)
    assert sc.dec.last_error() == (0, -1)


def test_page_allocator_all_or_nothing(mk):
    _log("[errors] page allocator")
    sc = _scenario([20], spare_pages=4)
    free0 = sc.dec.kv_available()
    assert free0 == 4
    with pytest.raises(mk.MkError) as e:
        sc.dec.kv_alloc(free0 + 1)
    assert e.value.status == MK_ERR_OOM
    assert sc.dec.kv_available() == free0
    got = sc.dec.kv_alloc(2)
    assert len(set(got)) == 2 and sc.dec.kv_available() == free0 - 2
    with pytest.raises(mk.MkError):
        sc.dec.kv_free([got[0], got[0]])          # repeated id
    with pytest.raises(mk.MkError):
        sc.dec.kv_free([sc.n_pages + 1])          # out of range
    assert sc.dec.kv_available() == free0 - 2     # rejected calls changed nothing
    sc.dec.kv_free(got)
    assert sc.dec.kv_available() == free0
    with pytest.raises(mk.MkError):
        sc.dec.kv_free([got[0]])                  # not allocated any more


def test_batch_outside_max_batch_is_rejected(mk):
    _log("[errors] batch larger than max_batch")
    sc = _scenario([20, 30])
    import torch
    seq = torch.tensor([20, 30, 40], dtype=torch.int32).cuda()
    tok = torch.tensor([1, 2, 3], dtype=torch.int32).cuda()
    pt3 = torch.cat([sc.pt, sc.pt[:1]]).contiguous()  # consistent with n = 3: the library decides
    with pytest.raises(mk.MkError) as e:
        sc.dec.decode_step(seq, pt3, tok)
    assert e.value.status == MK_ERR_INVALID_ARG
