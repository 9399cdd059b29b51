"""Python binding of the C-ABI decode library ``libmk.so`` (see include/mk.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind ``mk_decode_step``. PyTorch provides device memory and the
stream. Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
STATUS = {0: "MK_OK", 1: "MK_ERR_INVALID_ARG", 2: "MK_ERR_UNSUPPORTED", 3: "MK_ERR_OOM",
          4: "MK_ERR_HIP", 5: "MK_ERR_BAD_PAGE", 6: "MK_ERR_DEVICE_TIMEOUT"}
PAGE = 16
MAX_BATCH = 8

EXPORTS = ["mk_create", "mk_destroy", "mk_kv_alloc", "mk_kv_free", "mk_kv_available",
           "mk_kv_ref", "mk_kv_unref", "mk_kv_refcount", "mk_kv_cow",
           "mk_kv_layout", "mk_kv_write", "mk_kv_read", "mk_decode_step", "mk_last_error",
           "mk_set_wait_limit", "mk_launch_info", "mk_status_str", "mk_set_trace",
           "mk_set_cooperative", "mk_create_error", "mk_moe_experts_used", "mk_variant_info",
           "mk_set_route_debug", "mk_decode_step_noalloc", "mk_prefill", "mk_check_plan"]


class MkError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class ModelCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("expert_ffn_dim", ctypes.c_int32), ("window", ctypes.POINTER(ctypes.c_int32)),
                ("max_batch", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("weight_format", ctypes.c_int32)]


WEIGHTS_BF16, WEIGHTS_FP8 = 0, 1


_PP = ctypes.POINTER(ctypes.c_void_p)


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("attn_norm", _PP), ("wq", _PP), ("wk", _PP),
                ("wv", _PP), ("wo", _PP), ("ffn_norm", _PP), ("w_gate", _PP), ("w_up", _PP),
                ("w_down", _PP), ("router", _PP)]


class PrefillReq(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("pos0", ctypes.c_int32), ("tokens", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("temperature", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("step", ctypes.c_uint32), ("request", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("tokens_in", ctypes.c_void_p),
                ("temperature", ctypes.c_void_p), ("seed", ctypes.c_uint64),
                ("step", ctypes.c_uint32), ("top_k", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmk.so; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run decode_persistent_step_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        sig = {
            "mk_create": (i32, [ctypes.POINTER(ModelCfg), ctypes.POINTER(Weights), vp,
                                ctypes.POINTER(vp)]),
            "mk_destroy": (None, [vp]),
            "mk_kv_alloc": (i32, [vp, i32, vp]),
            "mk_kv_free": (i32, [vp, i32, vp]),
            "mk_kv_available": (i32, [vp]),
            "mk_kv_ref": (i32, [vp, i32, vp]),
            "mk_kv_unref": (i32, [vp, i32, vp]),
            "mk_kv_refcount": (i32, [vp, i32]),
            "mk_kv_cow": (i32, [vp, i32, vp]),
            "mk_kv_layout": (i32, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp]),
            "mk_kv_write": (i32, [vp, i32, i32, i32, vp, vp]),
            "mk_kv_read": (i32, [vp, i32, i32, i32, vp, vp]),
            "mk_decode_step": (i32, [vp, ctypes.POINTER(Batch), vp, vp]),
            "mk_decode_step_noalloc": (i32, [vp, ctypes.POINTER(Batch), vp, vp]),
            "mk_set_route_debug": (i32, [vp, vp]),
            "mk_prefill": (i32, [vp, ctypes.POINTER(PrefillReq), vp, vp]),
            "mk_check_plan": (i32, [ctypes.POINTER(ModelCfg), i32, i32]),
            "mk_last_error": (i32, [vp, ctypes.POINTER(i32)]),
            "mk_set_wait_limit": (i32, [vp, ctypes.c_uint32]),
            "mk_set_trace": (i32, [vp, vp]),
            "mk_set_cooperative": (i32, [vp, i32]),
            "mk_moe_experts_used": (i32, [vp, vp]),
            "mk_launch_info": (i32, [vp, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     ctypes.POINTER(i32), ctypes.POINTER(i32)]),
            "mk_variant_info": (i32, [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                      ctypes.POINTER(i32), ctypes.POINTER(i32)]),
            "mk_status_str": (ctypes.c_char_p, [i32]),
            "mk_create_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != MK_OK:
        raise MkError(rc, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _model_cfg(shape, n_pages: int, max_pages_per_seq: int, max_batch: int):
    """mk_model_cfg of a model shape and pool (and the window array it points to)."""
    win = (ctypes.c_int32 * shape.n_layers)(*shape.windows())
    cfg = ModelCfg(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                   shape.ffn_dim, shape.vocab, shape.rms_eps, shape.rope_base,
                   shape.n_experts, shape.top_k, shape.expert_ffn_dim, win, max_batch,
                   PAGE, n_pages, max_pages_per_seq,
                   WEIGHTS_FP8 if getattr(shape, "weight_format", "bf16") == "fp8" else WEIGHTS_BF16)
    return cfg, win


def check_plan(shape, n_pages: int, max_pages_per_seq: int, max_batch: int, compute_units: int = 256,
               lds_bytes: int = 160 * 1024):
    """mk_check_plan (host only): (status, reason) of mk_create's planning and
    bounds check for this model and pool on a device of compute_units CUs."""
    cfg, _win = _model_cfg(shape, n_pages, max_pages_per_seq, max_batch)
    rc = lib().mk_check_plan(ctypes.byref(cfg), int(compute_units), int(lds_bytes))
    return int(rc), lib().mk_create_error().decode()


class Decoder:
    """One mk handle: packed weights, the paged K/V pool and the decode step.

    ``shape`` is any object with the model-shape attributes (n_layers, d_model,
    n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_base,
    n_experts, top_k, expert_ffn_dim, windows()). ``weights`` maps the names of
    include/mk.h to torch bf16 CUDA tensors (per-layer entries are lists).
    """

    def __init__(self, shape, weights: Dict, n_pages: int, max_pages_per_seq: int,
                 max_batch: int, stream=None):
        import torch
        self.shape = shape
        self._torch = torch
        L = shape.n_layers
        cfg, self._win = _model_cfg(shape, n_pages, max_pages_per_seq, max_batch)
        keep = []

        def arr(name):
            lst = weights.get(name)
            if lst is None:
                return None
            a = (ctypes.c_void_p * L)(*[t.data_ptr() for t in lst])
            keep.append(a)
            return ctypes.cast(a, _PP)

        w = Weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                    weights["lm_head"].data_ptr(), arr("attn_norm"), arr("wq"), arr("wk"),
                    arr("wv"), arr("wo"), arr("ffn_norm"), arr("w_gate"), arr("w_up"),
                    arr("w_down"), arr("router"))
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        h = ctypes.c_void_p()
        rc = lib().mk_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(self.stream.cuda_stream),
                             ctypes.byref(h))
        _check(rc, "mk_create (" + lib().mk_create_error().decode() + ")")
        self.h = h
        self.max_batch = max_batch
        self.n_pages = n_pages
        self.max_pages_per_seq = max_pages_per_seq

    def close(self):
        if getattr(self, "h", None):
            lib().mk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------- pages
    def kv_alloc(self, n: int) -> List[int]:
        out = (ctypes.c_int32 * max(n, 1))()
        _check(lib().mk_kv_alloc(self.h, n, out), "mk_kv_alloc")
        return list(out[:n])

    def kv_free(self, pages: Sequence[int]):
        a = (ctypes.c_int32 * max(len(pages), 1))(*pages)
        _check(lib().mk_kv_free(self.h, len(pages), a), "mk_kv_free")

    def kv_available(self) -> int:
        return int(lib().mk_kv_available(self.h))

    def kv_ref(self, pages: Sequence[int]):
        """One more reference to each page (a request sharing them)."""
        a = (ctypes.c_int32 * max(len(pages), 1))(*pages)
        _check(lib().mk_kv_ref(self.h, len(pages), a), "mk_kv_ref")

    def kv_unref(self, pages: Sequence[int]):
        """Drop one reference to each page; unreferenced pages become free."""
        a = (ctypes.c_int32 * max(len(pages), 1))(*pages)
        _check(lib().mk_kv_unref(self.h, len(pages), a), "mk_kv_unref")

    def kv_refcount(self, page: int) -> int:
        return int(lib().mk_kv_refcount(self.h, page))

    def kv_cow(self, page: int) -> int:
        """The page's id for a request about to append to it: the same id if the
        request holds the only reference, else a private copy (enqueued on the
        decoder's stream)."""
        out = ctypes.c_int32(-1)
        _check(lib().mk_kv_cow(self.h, page, ctypes.byref(out)), "mk_kv_cow")
        return int(out.value)

    def kv_layout(self):
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        strides = (ctypes.c_int64 * 5)()
        _check(lib().mk_kv_layout(self.h, ctypes.byref(k), ctypes.byref(v), strides), "mk_kv_layout")
        return k.value, v.value, list(strides)

    def kv_write(self, layer: int, kv: int, slots, rows):
        """slots: int32 CUDA [n]; rows: bf16 CUDA [n][n_kv_heads][head_dim]."""
        _check(lib().mk_kv_write(self.h, layer, kv, int(slots.numel()), _ptr(slots), _ptr(rows)),
               "mk_kv_write")

    def kv_read(self, layer: int, kv: int, slots, rows):
        _check(lib().mk_kv_read(self.h, layer, kv, int(slots.numel()), _ptr(slots), _ptr(rows)),
               "mk_kv_read")

    # -------------------------------------------------------------- step
    def _batch(self, seq_lens, page_table, tokens_in, temperature, seed, step, tokens_out, logits_out,
               top_k):
        """Check the step's tensors (dtype, device, contiguity, sizes) and marshal
        them; ValueError before anything reaches the library."""
        torch = self._torch
        n = int(seq_lens.numel())

        def need(t, name, dtype, shape):
            if t is None:
                return
            if not isinstance(t, torch.Tensor):
                raise ValueError(f"{name}: a torch tensor is required")
            if t.dtype != dtype:
                raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
            if t.device.type != "cuda":
                raise ValueError(f"{name}: must be a CUDA tensor")
            if not t.is_contiguous():
                raise ValueError(f"{name}: must be contiguous")
            if tuple(t.shape) != shape:
                raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")

        i32, f32 = torch.int32, torch.float32
        need(seq_lens, "seq_lens", i32, (n,))
        need(tokens_in, "tokens_in", i32, (n,))
        need(page_table, "page_table", i32, (n, self.max_pages_per_seq))
        need(temperature, "temperature", f32, (n,))
        need(top_k, "top_k", i32, (n,))
        need(tokens_out, "tokens_out", i32, (n,))
        need(logits_out, "logits_out", f32, (n, self.shape.vocab))
        return Batch(n, _ptr(seq_lens), _ptr(page_table), _ptr(tokens_in), _ptr(temperature),
                     seed, step, _ptr(top_k))

    def decode_step(self, seq_lens, page_table, tokens_in, temperature=None, seed: int = 0,
                    step: int = 0, tokens_out=None, logits_out=None, top_k=None):
        """All tensors are CUDA tensors: int32 seq_lens, tokens_in [n], page_table
        [n][max_pages_per_seq], float32 temperature [n] or None, int32 top_k [n] or
        None; returns tokens_out (int32 [n]; logits_out float32 [n][vocab] if given)."""
        if tokens_out is None:
            tokens_out = self._torch.empty(int(seq_lens.numel()), dtype=self._torch.int32,
                                           device=seq_lens.device)
        b = self._batch(seq_lens, page_table, tokens_in, temperature, seed, step, tokens_out,
                        logits_out, top_k)
        _check(lib().mk_decode_step(self.h, ctypes.byref(b), _ptr(tokens_out), _ptr(logits_out)),
               "mk_decode_step")
        return tokens_out

    def decode_step_noalloc(self, seq_lens, page_table, tokens_in, temperature=None, seed: int = 0,
                            step: int = 0, tokens_out=None, logits_out=None, top_k=None):
        """mk_decode_step_noalloc: the same step on the library's static per-device
        scratch instead of the handle's buffers (allocates nothing); tokens_out
        must be given."""
        if tokens_out is None:
            raise ValueError("tokens_out is required (the call allocates nothing)")
        b = self._batch(seq_lens, page_table, tokens_in, temperature, seed, step, tokens_out,
                        logits_out, top_k)
        _check(lib().mk_decode_step_noalloc(self.h, ctypes.byref(b), _ptr(tokens_out),
                                            _ptr(logits_out)), "mk_decode_step_noalloc")
        return tokens_out

    def prefill(self, tokens, pos0: int, page_table, temperature: float = 0.0, seed: int = 0, step: int = 0,
                request: int = 0, token_out=None, logits_out=None):
        """mk_prefill: tokens int32 CUDA [n], page_table int32 CUDA [max_pages_per_seq];
        returns token_out (int32 [1]); logits_out float32 [vocab] if given."""
        torch = self._torch
        n = int(tokens.numel())
        if token_out is None:
            token_out = torch.empty(1, dtype=torch.int32, device=tokens.device)
        for t, name, dt, shape in ((tokens, "tokens", torch.int32, (n,)),
                                   (page_table, "page_table", torch.int32, (self.max_pages_per_seq,)),
                                   (token_out, "token_out", torch.int32, (1,)),
                                   (logits_out, "logits_out", torch.float32, (self.shape.vocab,))):
            if t is None:
                continue
            if t.dtype != dt or t.device.type != "cuda" or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"{name}: need a contiguous CUDA {dt} tensor of shape {shape}")
        r = PrefillReq(n, int(pos0), _ptr(tokens), _ptr(page_table), float(temperature), seed, step, request)
        _check(lib().mk_prefill(self.h, ctypes.byref(r), _ptr(token_out), _ptr(logits_out)), "mk_prefill")
        return token_out

    def set_route_debug(self, buf):
        """buf: int32 CUDA tensor [n_layers][8][8] receiving each step's MoE
        selection per layer and request (best first), or None to stop."""
        if buf is not None:
            L = self.shape.n_layers
            if buf.dtype != self._torch.int32 or tuple(buf.shape) != (L, MAX_BATCH, 8) or not buf.is_contiguous():
                raise ValueError(f"route debug buffer must be contiguous int32 [{L}][8][8]")
        _check(lib().mk_set_route_debug(self.h, _ptr(buf)), "mk_set_route_debug")

    def last_error(self):
        where = ctypes.c_int32(-1)
        rc = lib().mk_last_error(self.h, ctypes.byref(where))
        return int(rc), int(where.value)

    def set_trace(self, buf):
        """buf: uint64/int64 CUDA tensor [workgroups][S*L+1][8] (S = 5, or 6 for MoE), or None."""
        _check(lib().mk_set_trace(self.h, _ptr(buf)), "mk_set_trace")

    def set_wait_limit(self, usec: int):
        _check(lib().mk_set_wait_limit(self.h, usec), "mk_set_wait_limit")

    def set_cooperative(self, on: bool):
        _check(lib().mk_set_cooperative(self.h, 1 if on else 0), "mk_set_cooperative")

    def moe_experts_used(self) -> int:
        """Sum over the steps since the last call and their layers of the distinct
        experts selected (MoE models; 0 for dense)."""
        v = ctypes.c_int64()
        _check(lib().mk_moe_experts_used(self.h, ctypes.byref(v)), "mk_moe_experts_used")
        return int(v.value)

    def launch_info(self):
        a, b, c, d = (ctypes.c_int32() for _ in range(4))
        _check(lib().mk_launch_info(self.h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                    ctypes.byref(d)), "mk_launch_info")
        return {"workgroups": a.value, "threads": b.value, "lds_bytes": c.value, "path": d.value}

    def variant_info(self, batch: int):
        """Kernel variant of a step of `batch` requests: compute waves, ring slots, LDS bytes, path."""
        a, b, c, d = (ctypes.c_int32() for _ in range(4))
        _check(lib().mk_variant_info(self.h, int(batch), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                     ctypes.byref(d)), "mk_variant_info")
        return {"compute_waves": a.value, "ring_slots": b.value, "lds_bytes": c.value, "path": d.value}


def status_str(s: int) -> str:
    return lib().mk_status_str(s).decode()
