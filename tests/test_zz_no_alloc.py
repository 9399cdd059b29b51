"""The allocation-free decode entry point, mk_decode_step_noalloc, through the C
ABI: two calls in a row (batch 4, then a smaller batch 2 at later positions)
must give the same tokens, logits and K/V rows, bit for bit, as mk_decode_step
on an identical handle (both run the same kernel; dense steps are
bit-reproducible). A model whose exchange buffers exceed the static array is
rejected before anything is enqueued."""
import numpy as np
import pytest

import workload

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"  [noalloc] {msg}", flush=True)


def test_noalloc_matches_decode_step_twice_then_smaller():
    import torch
    from decode_persistent_step_amd import session
    from tests.scenario import Scenario
    ctx, temps = [40, 129, 7, 300], [0.0, 0.8, 0.0, 1.1]
    ref = Scenario(workload.TINY, ctx, 3, temps=temps, with_oracle=False)
    got = Scenario(workload.TINY, ctx, 3, temps=temps, with_oracle=False)
    seq, toks = list(ctx), list(ref.tokens)
    for call, n in enumerate((4, 2)):
        _log(f"call {call}: batch {n} at positions {seq[:n]}")
        outs = []
        for sc, fn in ((ref, ref.dec.decode_step), (got, got.dec.decode_step_noalloc)):
            seq_t = torch.tensor(seq[:n], dtype=torch.int32, device="cuda")
            tok_t = torch.tensor(toks[:n], dtype=torch.int32, device="cuda")
            tokens = torch.empty(n, dtype=torch.int32, device="cuda")
            logits = torch.empty((n, workload.TINY.vocab), dtype=torch.float32, device="cuda")
            fn(seq_t, sc.pt[:n], tok_t, sc.temp_t[:n].contiguous(), seed=5, step=call,
               tokens_out=tokens, logits_out=logits)
            torch.cuda.synchronize()
            slots = np.asarray(sc.new_kv_slots(seq)[:n], dtype=np.int32)
            kv = [session.read_kv_rows(sc.dec, l, kv, slots) for l in (0, 1) for kv in (0, 1)]
            outs.append((tokens.cpu().numpy().copy(), logits.cpu().numpy().copy(), kv))
            assert sc.dec.last_error()[0] == 0
        (t1, l1, kv1), (t2, l2, kv2) = outs
        assert np.array_equal(t1, t2), (t1, t2)
        assert np.array_equal(l1.view(np.int32), l2.view(np.int32)), "logits differ"
        for a, b in zip(kv1, kv2):
            assert np.array_equal(a, b), "K/V rows differ"
        toks = [int(t) for t in t1] + toks[n:]
        seq = [p + 1 for p in seq[:n]] + seq[n:]


def test_noalloc_rejects_a_model_beyond_the_static_scratch():
    import torch
    from decode_persistent_step_amd import Decoder, MkError, session
    # 8 kv heads of 8 query heads at dh 128: the attention partials alone need
    # 8 requests x 8 heads x 256 workgroups x (4 + 1024) words x 8 B = 135 MB
    big = workload.ModelShape("wide_g8", n_layers=1, d_model=128, n_q_heads=64, n_kv_heads=8,
                              head_dim=128, ffn_dim=128, vocab=256)
    w = session.upload_weights(workload.gen_weights(big, seed=1))
    dec = Decoder(big, w, n_pages=4, max_pages_per_seq=2, max_batch=1)
    pages = dec.kv_alloc(1)
    pt = session.page_table_tensor([pages + [pages[0]]], 2)
    one = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(MkError) as e:
        dec.decode_step_noalloc(one, pt, one, tokens_out=torch.empty(1, dtype=torch.int32, device="cuda"))
    assert e.value.status == 2  # MK_ERR_UNSUPPORTED
    dec.close()
