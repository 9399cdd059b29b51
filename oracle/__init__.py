"""TEST INFRASTRUCTURE ONLY: ctypes binding of the plain fp64 CPU oracle.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU library
(``decode_persistent_step_amd``) and never imports it.

Every function here marshals arguments only; the arithmetic is in
``oracle.c``, whose header lists the readings it takes of the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

PAGE = 16


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
             "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_double),
                ("rope_base", ctypes.c_double), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_ffn_dim", ctypes.c_int32),
                ("window", ctypes.POINTER(ctypes.c_int32)), ("n_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class _Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("attn_norm", _PP), ("wq", _PP), ("wk", _PP),
                ("wv", _PP), ("wo", _PP), ("ffn_norm", _PP), ("w_gate", _PP), ("w_up", _PP),
                ("w_down", _PP), ("router", _PP)]


class _Fp8Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


_P8 = ctypes.POINTER(_Fp8Mat)


class _Fp8Weights(ctypes.Structure):
    _fields_ = [("wq", _P8), ("wk", _P8), ("wv", _P8), ("wo", _P8), ("w_gate", _P8), ("w_up", _P8),
                ("w_down", _P8), ("lm_head", _Fp8Mat)]


class _RouteIO(ctypes.Structure):
    _fields_ = [("sel_in", ctypes.c_void_p), ("sel_out", ctypes.c_void_p),
                ("gap_out", ctypes.c_void_p), ("margin_out", ctypes.c_void_p)]


_lib = None
_vp, _i32, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        sig = {
            "orc_bf16_to_f64": (_f64, [ctypes.c_uint16]),
            "orc_f64_to_bf16": (ctypes.c_uint16, [_f64]),
            "orc_splitmix64": (ctypes.c_uint64, [ctypes.c_uint64]),
            "orc_rmsnorm": (None, [_i32, _vp, _vp, _f64, _vp]),
            "orc_matvec": (None, [_i32, _i32, _vp, _vp, _vp]),
            "orc_rope": (None, [_i32, _i32, _i32, _f64, _vp]),
            "orc_silu": (_f64, [_f64]),
            "orc_swiglu_ffn": (None, [_i32, _i32, _vp, _vp, _vp, _vp, _vp]),
            "orc_window_lo": (_i32, [_i32, _i32]),
            "orc_attend": (None, [_i32, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                                  _vp]),
            "orc_moe_route": (None, [_i32, _i32, _vp, _vp, _vp]),
            "orc_moe_weights": (None, [_i32, _vp, _vp, _vp]),
            "orc_moe_margin": (_f64, [_i32, _i32, _vp, _vp]),
            "orc_gumbel": (_f64, [ctypes.c_uint64, ctypes.c_uint32, _i32, _i32]),
            "orc_sample": (_i32, [_i32, _vp, _f64, ctypes.c_uint64, ctypes.c_uint32, _i32,
                                  _vp]),
            "orc_sample_topk": (_i32, [_i32, _vp, _f64, _i32, ctypes.c_uint64, ctypes.c_uint32, _i32, _vp]),
            "orc_decode_step": (_i32, [ctypes.POINTER(_Cfg), ctypes.POINTER(_Weights), _vp, _vp,
                                       _i32, _vp, _vp, _vp, _vp, ctypes.c_uint64,
                                       ctypes.c_uint32, _vp, _vp, _vp, _vp]),
            "orc_fp8_value": (_f64, [ctypes.c_uint8]),
            "orc_fp8_encode": (ctypes.c_uint8, [_f64]),
            "orc_fp8_quantize_rows": (None, [_i32, _i32, _vp, _vp, _vp]),
            "orc_matvec_fp8": (None, [_i32, _i32, _vp, _vp, _vp, _vp]),
            "orc_decode_step_ex": (_i32, [ctypes.POINTER(_Cfg), ctypes.POINTER(_Weights), ctypes.POINTER(_Fp8Weights),
                                          _vp, _vp, _i32, _vp, _vp, _vp, _vp, ctypes.c_uint64,
                                          ctypes.c_uint32, _vp, _vp, _vp, ctypes.POINTER(_RouteIO)]),
            "orc_decode_step_routed": (_i32, [ctypes.POINTER(_Cfg), ctypes.POINTER(_Weights), _vp, _vp,
                                              _i32, _vp, _vp, _vp, _vp, ctypes.c_uint64,
                                              ctypes.c_uint32, _vp, _vp, _vp,
                                              ctypes.POINTER(_RouteIO)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _f64arr(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ------------------------------------------------------------ component calls


def bf16_to_f64(h: int) -> float:
    return float(lib().orc_bf16_to_f64(h))


def f64_to_bf16(x: float) -> int:
    return int(lib().orc_f64_to_bf16(x))


def splitmix64(z: int) -> int:
    return int(lib().orc_splitmix64(z & 0xFFFFFFFFFFFFFFFF))


def rmsnorm(x, g_bf16: np.ndarray, eps: float) -> np.ndarray:
    x = _f64arr(x)
    g = np.ascontiguousarray(g_bf16, dtype=np.uint16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(x.size, _ptr(x), _ptr(g), eps, _ptr(y))
    return y


def matvec(W_bf16: np.ndarray, x) -> np.ndarray:
    W = np.ascontiguousarray(W_bf16, dtype=np.uint16)
    x = _f64arr(x)
    rows, cols = W.shape
    assert x.size == cols
    y = np.empty(rows, dtype=np.float64)
    lib().orc_matvec(rows, cols, _ptr(W), _ptr(x), _ptr(y))
    return y


def rope(v, n_heads: int, head_dim: int, pos: int, base: float) -> np.ndarray:
    v = _f64arr(v).copy()
    lib().orc_rope(n_heads, head_dim, pos, base, _ptr(v))
    return v


def silu(z: float) -> float:
    return float(lib().orc_silu(z))


def swiglu_ffn(w_gate, w_up, w_down, n2) -> np.ndarray:
    w_gate = np.ascontiguousarray(w_gate, dtype=np.uint16)
    w_up = np.ascontiguousarray(w_up, dtype=np.uint16)
    w_down = np.ascontiguousarray(w_down, dtype=np.uint16)
    f, d = w_gate.shape
    n2 = _f64arr(n2)
    y = np.empty(d, dtype=np.float64)
    lib().orc_swiglu_ffn(d, f, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(n2), _ptr(y))
    return y


def window_lo(pos: int, window: int) -> int:
    return int(lib().orc_window_lo(pos, window))


def attend(kpool_layer: np.ndarray, vpool_layer: np.ndarray, pages: Sequence[int], lo: int,
           pos: int, kv_head: int, q) -> tuple:
    """kpool_layer/vpool_layer: bf16 [n_pages][Hkv][16][dh]. Returns (o, probs)."""
    kp = np.ascontiguousarray(kpool_layer, dtype=np.uint16)
    vp = np.ascontiguousarray(vpool_layer, dtype=np.uint16)
    n_pages, hkv, page, dh = kp.shape
    assert page == PAGE
    pg = np.ascontiguousarray(pages, dtype=np.int32)
    q = _f64arr(q)
    o = np.empty(dh, dtype=np.float64)
    probs = np.empty(pos - lo + 1, dtype=np.float64)
    lib().orc_attend(hkv, dh, n_pages, _ptr(kp), _ptr(vp), _ptr(pg), lo, pos, kv_head, _ptr(q),
                     _ptr(o), _ptr(probs))
    return o, probs


def moe_route(logits, top_k: int):
    r = _f64arr(logits)
    idx = np.empty(top_k, dtype=np.int32)
    w = np.empty(top_k, dtype=np.float64)
    lib().orc_moe_route(r.size, top_k, _ptr(r), _ptr(idx), _ptr(w))
    return idx, w


def moe_weights(logits, idx) -> np.ndarray:
    """Softmax of the selected experts' logits (orc_moe_weights)."""
    r = _f64arr(logits)
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.empty(ix.size, dtype=np.float64)
    lib().orc_moe_weights(ix.size, _ptr(r), _ptr(ix), _ptr(w))
    return w


def moe_margin(logits, idx) -> float:
    """Smallest selected logit minus the largest unselected one (orc_moe_margin)."""
    r = _f64arr(logits)
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    return float(lib().orc_moe_margin(r.size, ix.size, _ptr(r), _ptr(ix)))


def gumbel(seed: int, step: int, b: int, i: int) -> float:
    return float(lib().orc_gumbel(seed, step, b, i))


def sample(logits, temperature: float, seed: int = 0, step: int = 0, b: int = 0):
    l = _f64arr(logits)
    sc = ctypes.c_double()
    tok = lib().orc_sample(l.size, _ptr(l), temperature, seed, step, b, ctypes.byref(sc))
    return int(tok), float(sc.value)


def sample_topk(logits, temperature: float, top_k: int, seed: int = 0, step: int = 0, b: int = 0):
    """Temperature sampling over the top_k largest logits (orc_sample_topk)."""
    l = _f64arr(logits)
    sc = ctypes.c_double()
    tok = lib().orc_sample_topk(l.size, _ptr(l), temperature, top_k, seed, step, b, ctypes.byref(sc))
    return int(tok), float(sc.value)


def fp8_value(q: int) -> float:
    """Value of an E4M3 code (orc_fp8_value)."""
    return float(lib().orc_fp8_value(q))


def fp8_encode(x: float) -> int:
    """E4M3 code of x, nearest even, saturated at 448 (orc_fp8_encode)."""
    return int(lib().orc_fp8_encode(x))


def fp8_quantize_rows(W_bf16: np.ndarray):
    """(codes uint8 [rows][cols], scales float32 [rows]) of a bf16 matrix."""
    W = np.ascontiguousarray(W_bf16, dtype=np.uint16)
    rows, cols = W.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    sc = np.empty(rows, dtype=np.float32)
    lib().orc_fp8_quantize_rows(rows, cols, _ptr(W), _ptr(q), _ptr(sc))
    return q, sc


def matvec_fp8(q: np.ndarray, scale: np.ndarray, x) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    x = _f64arr(x)
    rows, cols = q.shape
    y = np.empty(rows, dtype=np.float64)
    lib().orc_matvec_fp8(rows, cols, _ptr(q), _ptr(sc), _ptr(x), _ptr(y))
    return y


# ----------------------------------------------------------------- the model


class OracleModel:
    """Weights (bf16 bit patterns, numpy) plus the oracle's own paged K/V pool.

    ``weights`` is the dict produced by ``workload.gen_weights`` (or any dict
    with the same keys and shapes). The pool is [L][n_pages][Hkv][16][dh].
    """

    def __init__(self, shape, weights: dict, n_pages: int, max_pages_per_seq: int,
                 weight_format: Optional[str] = None):
        """weight_format "fp8" (default: the shape's): every linear map of a dense
        model is quantized by the oracle itself (fp8_quantize_rows) and the step
        uses those forms."""
        if weight_format is None:
            weight_format = getattr(shape, "weight_format", "bf16")
        self.shape = shape
        self.w = weights
        self.n_pages = n_pages
        self.max_pages_per_seq = max_pages_per_seq
        L, hkv, dh = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.kpool = np.zeros((L, n_pages, hkv, PAGE, dh), dtype=np.uint16)
        self.vpool = np.zeros((L, n_pages, hkv, PAGE, dh), dtype=np.uint16)
        self._win = np.ascontiguousarray(shape.windows(), dtype=np.int32)
        self._cfg = _Cfg(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads,
                         shape.head_dim, shape.ffn_dim, shape.vocab, shape.rms_eps,
                         shape.rope_base, shape.n_experts, shape.top_k, shape.expert_ffn_dim,
                         self._win.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n_pages,
                         max_pages_per_seq)
        self._keep = []

        def arr(name):
            lst = weights.get(name)
            if lst is None:
                return None
            for a in lst:
                assert a.dtype == np.uint16 and a.flags["C_CONTIGUOUS"]
            ptrs = (ctypes.c_void_p * L)(*[a.ctypes.data for a in lst])
            self._keep.append(ptrs)
            return ctypes.cast(ptrs, _PP)

        for k in ("embed", "final_norm", "lm_head"):
            assert weights[k].dtype == np.uint16 and weights[k].flags["C_CONTIGUOUS"]
        self._w = _Weights(weights["embed"].ctypes.data, weights["final_norm"].ctypes.data,
                           weights["lm_head"].ctypes.data, arr("attn_norm"), arr("wq"),
                           arr("wk"), arr("wv"), arr("wo"), arr("ffn_norm"), arr("w_gate"),
                           arr("w_up"), arr("w_down"), arr("router"))
        self.weight_format = weight_format
        self._w8 = None
        if weight_format == "fp8":
            assert not shape.moe, "FP8 weights: dense models"
            self.fp8 = {}

            def mats(name):
                out = (_Fp8Mat * L)()
                forms = []
                for l, a in enumerate(weights[name]):
                    q, sc = fp8_quantize_rows(a)
                    forms.append((q, sc))
                    out[l] = _Fp8Mat(q.ctypes.data, sc.ctypes.data)
                self.fp8[name] = forms
                self._keep.append(out)
                return ctypes.cast(out, _P8)

            args = [mats(nm) for nm in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]
            qlm, slm = fp8_quantize_rows(weights["lm_head"])
            self.fp8["lm_head"] = [(qlm, slm)]
            self._w8 = _Fp8Weights(*args, _Fp8Mat(qlm.ctypes.data, slm.ctypes.data))
        elif weight_format != "bf16":
            raise ValueError(weight_format)

    def write_kv(self, layer: int, page: int, kv_head: int, slot: int, k_bf16, v_bf16):
        self.kpool[layer, page, kv_head, slot] = k_bf16
        self.vpool[layer, page, kv_head, slot] = v_bf16

    def prefill_from(self, b_pages: Sequence[int], layer: int, k_bf16: np.ndarray,
                     v_bf16: np.ndarray):
        """Scatter logical K/V [n_pos][Hkv][dh] (positions 0..n_pos-1) of one request
        into this pool through its page list."""
        n_pos = k_bf16.shape[0]
        pos = np.arange(n_pos)
        pg = np.asarray(b_pages, dtype=np.int64)[pos // PAGE]
        self.kpool[layer, pg, :, pos % PAGE, :] = k_bf16
        self.vpool[layer, pg, :, pos % PAGE, :] = v_bf16

    def decode_step(self, seq_lens, page_table, tokens_in, temperature=None, seed: int = 0,
                    step: int = 0, want_layers: bool = False, want_route_gap: bool = False,
                    route_in=None, want_route: bool = False):
        """Tokens and logits of one step (plus, on request, x after every layer,
        the per-request smallest top-k boundary gap of the MoE routing, and the
        MoE routing per layer).

        route_in: int32 [n][n_layers][top_k] experts to use in place of the
        oracle's own top-k (MoE models). want_route adds a dict with
        ``sel`` [n][L][top_k] (the oracle's own top-k, best first), ``gap``
        [n][L] (its margin: k-th minus (k+1)-th logit) and ``margin`` [n][L]
        (the margin of the selection used, route_in's if given)."""
        n = len(seq_lens)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        assert pt.shape == (n, self.max_pages_per_seq)
        ti = np.ascontiguousarray(tokens_in, dtype=np.int32)
        T = None if temperature is None else _f64arr(temperature)
        toks = np.empty(n, dtype=np.int32)
        logits = np.empty((n, self.shape.vocab), dtype=np.float64)
        L, K = self.shape.n_layers, max(self.shape.top_k, 1)
        lx = np.empty((n, L, self.shape.d_model), dtype=np.float64) if want_layers else None
        rin = None
        if route_in is not None:
            rin = np.ascontiguousarray(route_in, dtype=np.int32)
            assert rin.shape == (n, L, self.shape.top_k)
        sel = np.full((n, L, K), -1, dtype=np.int32)
        gap = np.full((n, L), np.inf, dtype=np.float64)
        margin = np.full((n, L), np.inf, dtype=np.float64)
        io = _RouteIO(_ptr(rin), _ptr(sel), _ptr(gap), _ptr(margin))
        rc = lib().orc_decode_step_ex(ctypes.byref(self._cfg), ctypes.byref(self._w),
                                      ctypes.byref(self._w8) if self._w8 is not None else None,
                                      _ptr(self.kpool), _ptr(self.vpool), n, _ptr(sl), _ptr(pt),
                                      _ptr(ti), _ptr(T), seed, step, _ptr(toks), _ptr(logits),
                                      _ptr(lx), ctypes.byref(io))
        if rc != 0:
            raise ValueError("oracle rejected the step (page table / token / length / routing)")
        out = (toks, logits)
        if want_layers:
            out += (lx,)
        if want_route_gap:
            out += (gap.min(axis=1) if self.shape.moe else np.full(n, np.inf),)
        if want_route:
            out += ({"sel": sel, "gap": gap, "margin": margin},)
        return out
