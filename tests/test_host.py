"""CPU tests of the host side: the C-ABI library loads and exports every call
include/mk.h declares, host-checkable arguments are rejected before any device
work, and the bench's bandwidth arithmetic reproduces the numbers the pages
print (tests/golden/bench_math.json, each case with its citation)."""
import ctypes
import dataclasses
import json
import os
import re

import pytest

import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mk():
    import decode_persistent_step_amd as mk
    try:
        mk.lib()
    except ImportError as e:
        pytest.fail(f"libmk.so not built: {e}")
    return mk


def test_library_exports_every_declared_call(mk):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(mk.lib(), n), f"libmk.so does not export {n}"
    assert sorted(mk.EXPORTS) == names


def test_status_strings(mk):
    seen = set()
    for code in range(7):
        s = mk.status_str(code)
        assert s and s not in seen
        seen.add(s)


def _cfg(mk, shape, **over):
    L = shape.n_layers
    win = (ctypes.c_int32 * L)(*shape.windows())
    vals = dict(n_layers=L, d_model=shape.d_model, n_q_heads=shape.n_q_heads,
                n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, ffn_dim=shape.ffn_dim,
                vocab=shape.vocab, rms_eps=shape.rms_eps, rope_base=shape.rope_base,
                n_experts=0, top_k=0, expert_ffn_dim=0, window=win, max_batch=1,
                page_size=16, n_pages=8, max_pages_per_seq=8, weight_format=0)
    vals.update(over)
    c = mk.ModelCfg(**{k: v for k, v in vals.items()})
    return c, win


def _weights(mk, L):
    one = (ctypes.c_void_p * L)(*([1] * L))  # never dereferenced: rejected before use
    pp = ctypes.cast(one, mk._PP)
    return mk.Weights(1, 1, 1, pp, pp, pp, pp, pp, pp, pp, pp, pp, None), one


@pytest.mark.parametrize("over,expect", [
    (dict(page_size=32), 1),
    (dict(max_batch=9), 1),
    (dict(max_batch=0), 1),
    (dict(n_kv_heads=3), 1),            # Hq not a multiple of Hkv
    (dict(rope_base=0.0), 1),
    (dict(n_experts=4, top_k=5, expert_ffn_dim=64), 1),
    (dict(n_experts=8, top_k=2, expert_ffn_dim=128), 1),   # MoE without router weights
    (dict(n_experts=8, top_k=9, expert_ffn_dim=128), 1),   # top_k above the experts
    (dict(n_experts=200, top_k=9, expert_ffn_dim=128), 2), # beyond 128 experts / top-8
    (dict(n_experts=8, top_k=2, expert_ffn_dim=96), 2),    # expert width not a multiple of 128
    (dict(head_dim=96, n_q_heads=4, n_kv_heads=2), 2),
    (dict(n_q_heads=8, n_kv_heads=2), 2),                  # group size 4
    (dict(d_model=192), 2),
    (dict(weight_format=7), 1),                            # unknown weight format
    (dict(weight_format=1, n_experts=8, top_k=2, expert_ffn_dim=128), 2),  # FP8 MoE
    (dict(weight_format=1, n_q_heads=16, n_kv_heads=2, head_dim=128), 2),   # FP8 with groups of 8
])
def test_create_rejects_before_device_work(mk, over, expect):
    c, win = _cfg(mk, workload.TINY, **over)
    w, keep = _weights(mk, workload.TINY.n_layers)
    if over.get("n_experts", 0) > 0 and expect == 2:
        w.router = w.wq  # present (never dereferenced): the shape check must reject
    h = ctypes.c_void_p(123)
    rc = mk.lib().mk_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h))
    assert rc == expect
    assert h.value is None


def test_create_rejects_null_arguments(mk):
    c, win = _cfg(mk, workload.TINY)
    h = ctypes.c_void_p()
    assert mk.lib().mk_create(None, None, None, ctypes.byref(h)) == 1
    assert mk.lib().mk_create(ctypes.byref(c), None, None, ctypes.byref(h)) == 1
    w, keep = _weights(mk, workload.TINY.n_layers)
    w.wq = None
    assert mk.lib().mk_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h)) == 1


def test_null_handle_calls_fail_cleanly(mk):
    L = mk.lib()
    out = (ctypes.c_int32 * 4)()
    assert L.mk_kv_alloc(None, 1, out) == 1
    assert L.mk_kv_free(None, 1, out) == 1
    assert L.mk_kv_available(None) == 0
    assert L.mk_decode_step(None, None, None, None) == 1
    assert L.mk_last_error(None, None) == 1
    assert L.mk_set_wait_limit(None, 10) == 1
    assert L.mk_set_trace(None, None) == 1
    assert L.mk_set_cooperative(None, 1) == 1
    assert L.mk_decode_step_noalloc(None, None, None, None) == 1
    assert L.mk_set_route_debug(None, None) == 1
    L.mk_destroy(None)


def test_binding_checks_step_tensors_before_the_library(mk):
    """The binding's decode_step rejects tensors of the wrong dtype or device
    (and missing outputs of the allocation-free call) with ValueError before
    anything reaches the library; no handle is needed to get that far."""
    import torch
    dec = mk.Decoder.__new__(mk.Decoder)  # no handle: every case must fail before the call
    dec._torch, dec.shape, dec.max_pages_per_seq, dec.h = torch, workload.TINY, 4, None
    i32 = torch.zeros(2, dtype=torch.int32)
    pt = torch.zeros((2, 4), dtype=torch.int32)
    cases = [
        dict(seq_lens=i32.to(torch.int64), page_table=pt, tokens_in=i32),          # int64 lengths
        dict(seq_lens=i32, page_table=pt, tokens_in=i32,
             temperature=torch.zeros(2, dtype=torch.float64)),                      # float64 temperatures
        dict(seq_lens=i32, page_table=pt, tokens_in=i32, top_k=i32.to(torch.int64)),
        dict(seq_lens=i32, page_table=pt, tokens_in=i32),                           # CPU tensors
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            dec.decode_step(tokens_out=torch.zeros(2, dtype=torch.int32), **kw)
    with pytest.raises(ValueError):
        dec.decode_step_noalloc(i32, pt, i32)   # tokens_out is required


# ------------------------------------------------------------ bench arithmetic
def _golden():
    with open(os.path.join(ROOT, "tests", "golden", "bench_math.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_bench_math_matches_pages(case):
    import bench
    args = {k: v for k, v in case.items()
            if k not in ("name", "expect", "rel_tol", "abs_tol", "expect_below", "cite")}
    rename = {"bytes": "bytes_"}
    args = {rename.get(k, k): v for k, v in args.items()}
    got = getattr(bench, case["name"])(**args)
    if "expect_below" in case:
        assert got < case["expect_below"]
    elif "rel_tol" in case:
        assert abs(got - case["expect"]) <= case["rel_tol"] * abs(case["expect"])
    else:
        assert abs(got - case["expect"]) <= case["abs_tol"]


def test_weight_bytes_equal_parameter_bytes():
    # every parameter except the embedding table is streamed once per step; the
    # embedding contributes one row per request
    import bench
    for shape in (workload.TINY, workload.DENSE2B):
        for B in (1, 8):
            emb = shape.vocab * shape.d_model
            want = 2 * (shape.n_params() - emb + B * shape.d_model)
            assert bench.weight_bytes_per_step(shape, B) == want


def test_moe_weight_bytes_count_all_experts_when_all_are_used():
    # an MoE step that touches every expert in every layer streams every parameter
    # but the embedding table (plus one row per request)
    import bench
    for shape in (workload.TINY_MOE, workload.MOE30B):
        emb = shape.vocab * shape.d_model
        want = 2 * (shape.n_params() - emb + 8 * shape.d_model)
        got = bench.weight_bytes_per_step(shape, 8) + shape.n_layers * shape.n_experts * bench.expert_bytes(shape)
        assert got == want


def test_kv_bytes_count_each_attended_position_once():
    import bench
    s = workload.DENSE2B
    per_pos = 2 * 2 * s.n_kv_heads * s.head_dim * s.n_layers   # K and V, bf16
    # position p attends over p+1 keys (the cached ones and its own)
    assert bench.kv_bytes_per_step(s, [8192]) == per_pos * 8193
    assert bench.kv_bytes_per_step(s, [0, 10]) == per_pos * (1 + 11)


def test_prefill_flops_closed_forms():
    import bench
    s = workload.DENSE2B
    n = 300
    f = bench.prefill_flops(s, 0, n)
    # the linear maps: 2 flops per weight of every layer per token, i.e. twice
    # the parameter count without the embedding, lm_head and the norm gains
    per_tok = 2 * (s.n_params() - 2 * s.vocab * s.d_model - s.d_model - 2 * s.n_layers * s.d_model)
    assert f["linear"] == per_tok * n
    # causal attention without a window: positions 0..n-1 see 1..n keys
    assert f["attention"] == 4 * s.n_q_heads * s.head_dim * s.n_layers * n * (n + 1) // 2
    assert f["lm_head"] == 2 * s.d_model * s.vocab
    # a window w caps each position's keys at w; from pos0 the spans start at pos0 + 1
    w = dataclasses.replace(s, window=[4] * s.n_layers)
    assert bench.prefill_flops(w, 10, 3)["attention"] == 4 * s.n_q_heads * s.head_dim * s.n_layers * 12
    assert bench.prefill_flops(s, 10, 3)["attention"] == 4 * s.n_q_heads * s.head_dim * s.n_layers * (11 + 12 + 13)
