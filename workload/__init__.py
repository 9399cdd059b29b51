"""Seeded synthetic workloads for the small-batch decode step.

This module is shared by the oracle-side tests and the GPU-side tests and
bench, and holds none of the decode arithmetic: only model shapes, the
counter-based generator of ``gen.c`` (SplitMix64 + Irwin-Hall(4), see that
file's header) and the seeded draws built on it (context lengths, page
shuffles, initial tokens).

Model shapes are the workloads the decode step is measured on: a tiny
2-layer decoder, a ~2B dense decoder at batch 1 and 8, the same model with
alternating sliding-window layers at batch 4, and a 128-expert MoE decoder.
The pages (Cohere Megakernel, "Sınırlar açıkça yazılmış") fix only batch 1-8,
BF16, paged KV, ragged lengths, sliding window, greedy and temperature
sampling; everything about the architecture is a stated reading.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libworkload.so")
_SRC = os.path.join(_HERE, "gen.c")

MASTER_SEED = 0
# fixed seed offsets for the non-tensor draws
SEED_CTX = 0xC7C7
SEED_PAGES = 0x9A9A
SEED_TOKENS = 0x7070
KV_TAG = 1 << 40

PAGE = 16


def build(force: bool = True) -> str:
    """Compile gen.c into libworkload.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
             "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.wl_splitmix64.restype = ctypes.c_uint64
        L.wl_splitmix64.argtypes = [ctypes.c_uint64]
        L.wl_sigma_scale.restype = ctypes.c_float
        L.wl_sigma_scale.argtypes = [ctypes.c_double]
        L.wl_draw_ih4.restype = ctypes.c_int32
        L.wl_draw_ih4.argtypes = [ctypes.c_uint64] * 3
        L.wl_fill_normal_bf16.restype = None
        L.wl_fill_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                          ctypes.c_float]
        L.wl_draw_mod.restype = ctypes.c_uint64
        L.wl_draw_mod.argtypes = [ctypes.c_uint64] * 3
        L.wl_shuffle_i32.restype = None
        L.wl_shuffle_i32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64]
        _lib = L
    return _lib


def splitmix64(z: int) -> int:
    return int(lib().wl_splitmix64(ctypes.c_uint64(z & 0xFFFFFFFFFFFFFFFF)))


def fill_normal_bf16(shape, seed: int, tensor_id: int, sigma: float, mean: float = 0.0,
                     index0: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of shape ``shape`` drawn at flat indices index0.."""
    out = np.empty(shape, dtype=np.uint16)
    lib().wl_fill_normal_bf16(out.ctypes.data, out.size, seed, tensor_id, index0,
                              float(sigma), float(mean))
    return out


def draw_mod(seed: int, i: int, m: int) -> int:
    return int(lib().wl_draw_mod(seed, i, m))


def shuffle_i32(a: np.ndarray, seed: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32).copy()
    lib().wl_shuffle_i32(a.ctypes.data, a.size, seed)
    return a


# ---------------------------------------------------------------- model shapes


@dataclasses.dataclass
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    n_experts: int = 0
    top_k: int = 0
    expert_ffn_dim: int = 0
    window: Optional[List[int]] = None  # per layer; 0 = full attention
    weight_format: str = "bf16"          # "fp8": linear maps streamed as E4M3 codes + row scales

    def windows(self) -> List[int]:
        return list(self.window) if self.window is not None else [0] * self.n_layers

    @property
    def moe(self) -> bool:
        return self.n_experts > 0

    def weight_shapes(self) -> Dict[str, tuple]:
        d, hq, hkv, dh = self.d_model, self.n_q_heads, self.n_kv_heads, self.head_dim
        s = {"attn_norm": (d,), "wq": (hq * dh, d), "wk": (hkv * dh, d), "wv": (hkv * dh, d),
             "wo": (d, hq * dh), "ffn_norm": (d,)}
        if self.moe:
            E, fe = self.n_experts, self.expert_ffn_dim
            s.update({"router": (E, d), "w_gate": (E, fe, d), "w_up": (E, fe, d),
                      "w_down": (E, d, fe)})
        else:
            s.update({"w_gate": (self.ffn_dim, d), "w_up": (self.ffn_dim, d),
                      "w_down": (d, self.ffn_dim)})
        return s

    def n_params(self) -> int:
        per_layer = sum(int(np.prod(v)) for v in self.weight_shapes().values())
        return self.n_layers * per_layer + 2 * self.vocab * self.d_model + self.d_model


@dataclasses.dataclass
class Workload:
    """One measured configuration: a model shape plus the batch it decodes."""
    key: str
    shape: ModelShape
    batch: int
    ctx_lo: int
    ctx_hi: int
    steps: int
    sampling: str = "greedy"  # "greedy" | "mixed" (even b greedy, odd b T=0.7)
    shuffle_pages: bool = True

    def contexts(self, seed: int = MASTER_SEED) -> List[int]:
        if self.ctx_lo == self.ctx_hi:
            return [self.ctx_lo] * self.batch
        span = self.ctx_hi - self.ctx_lo + 1
        return [self.ctx_lo + draw_mod(seed ^ SEED_CTX, b, span) for b in range(self.batch)]

    def temperatures(self) -> List[float]:
        if self.sampling == "mixed":
            return [0.0 if b % 2 == 0 else 0.7 for b in range(self.batch)]
        return [0.0] * self.batch

    def initial_tokens(self, seed: int = MASTER_SEED) -> List[int]:
        return [draw_mod(seed ^ SEED_TOKENS, b, self.shape.vocab) for b in range(self.batch)]


def _alternating(n_layers: int, w: int) -> List[int]:
    # layer l is sliding iff l is even (layer 0 sliding)
    return [w if (l % 2 == 0) else 0 for l in range(n_layers)]


TINY = ModelShape("tiny", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  ffn_dim=1024, vocab=4096)
DENSE2B = ModelShape("dense2b", n_layers=25, d_model=2048, n_q_heads=16, n_kv_heads=8,
                     head_dim=128, ffn_dim=8192, vocab=32000)
SWA2B = dataclasses.replace(DENSE2B, name="swa2b", window=_alternating(25, 4096))
# The same models with FP8 weights (quantized from the bf16 ones by the library
# and, independently, by the oracle).
DENSE2B_FP8 = dataclasses.replace(DENSE2B, name="dense2b_fp8", weight_format="fp8")
TINY_FP8 = dataclasses.replace(TINY, name="tiny_fp8", weight_format="fp8")
# Small shapes for parity tests of the code paths the full configurations take:
# a 16-expert top-4 MoE (batch sizes 1-8 select 4-16 experts), and a group-8
# dense model (the attention grouping of the MoE configuration).
TINY_MOE = ModelShape("tiny_moe", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                      ffn_dim=0, vocab=4096, n_experts=16, top_k=4, expert_ffn_dim=128)
TINY_G8 = ModelShape("tiny_g8", n_layers=2, d_model=256, n_q_heads=8, n_kv_heads=1, head_dim=128,
                     ffn_dim=512, vocab=4096)
MOE30B = ModelShape("moe30b", n_layers=48, d_model=2048, n_q_heads=32, n_kv_heads=4,
                    head_dim=128, ffn_dim=0, vocab=32000, n_experts=128, top_k=8,
                    expert_ffn_dim=768)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, batch=1, ctx_lo=128, ctx_hi=128, steps=1),
    "dense2b_b1": Workload("dense2b_b1", DENSE2B, batch=1, ctx_lo=8192, ctx_hi=8192, steps=256),
    "dense2b_b8": Workload("dense2b_b8", DENSE2B, batch=8, ctx_lo=1024, ctx_hi=8192, steps=256,
                           sampling="mixed"),
    "swa2b_b4": Workload("swa2b_b4", SWA2B, batch=4, ctx_lo=16384, ctx_hi=32768, steps=128),
    "moe30b_b8": Workload("moe30b_b8", MOE30B, batch=8, ctx_lo=2048, ctx_hi=8192, steps=128),
    "dense2b_b1_fp8": Workload("dense2b_b1_fp8", DENSE2B_FP8, batch=1, ctx_lo=8192, ctx_hi=8192, steps=256),
    "dense2b_b8_fp8": Workload("dense2b_b8_fp8", DENSE2B_FP8, batch=8, ctx_lo=1024, ctx_hi=8192, steps=256,
                               sampling="mixed"),
}


# ------------------------------------------------------------ tensor identities


def tensor_id(name: str, layer: int = -1) -> int:
    top = {"embed": 1, "final_norm": 2, "lm_head": 3}
    if name in top:
        return top[name]
    kinds = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
             "router"]
    return 16 * (layer + 1) + kinds.index(name)


def kv_tensor_id(shape: ModelShape, b: int, layer: int, kv: int) -> int:
    return KV_TAG + ((b * shape.n_layers + layer) * 2 + kv)


def gen_tensor(shape: ModelShape, name: str, layer: int = -1, seed: int = MASTER_SEED,
               index0: int = 0, count: Optional[int] = None, literal_gains: bool = False):
    """Generate one weight tensor (or a flat slice of it) as bf16 bit patterns.

    Matrices are ~N(0, 0.02). Norm gains are 1 + N(0, 0.02) (``literal_gains``
    gives the literal ~N(0, 0.02) instead).
    """
    if name in ("embed", "lm_head"):
        full = (shape.vocab, shape.d_model)
    elif name == "final_norm":
        full = (shape.d_model,)
    else:
        full = shape.weight_shapes()[name]
    is_gain = name in ("attn_norm", "ffn_norm", "final_norm")
    mean = 0.0 if (literal_gains or not is_gain) else 1.0
    tid = tensor_id(name, layer)
    if count is None:
        return fill_normal_bf16(full, seed, tid, 0.02, mean, index0)
    return fill_normal_bf16((count,), seed, tid, 0.02, mean, index0)


def gen_weights(shape: ModelShape, seed: int = MASTER_SEED, literal_gains: bool = False):
    """All weights as a dict: top-level arrays plus per-layer lists."""
    w = {n: gen_tensor(shape, n, seed=seed, literal_gains=literal_gains)
         for n in ("embed", "final_norm", "lm_head")}
    for n in shape.weight_shapes():
        w[n] = [gen_tensor(shape, n, l, seed=seed, literal_gains=literal_gains)
                for l in range(shape.n_layers)]
    return w


def gen_kv(shape: ModelShape, b: int, layer: int, kv: int, n_pos: int, pos0: int = 0,
           seed: int = MASTER_SEED) -> np.ndarray:
    """Prefilled K (kv=0) or V (kv=1) of request b, layer ``layer``: bf16 [n_pos][Hkv][dh] ~N(0,1)."""
    hd = shape.n_kv_heads * shape.head_dim
    return fill_normal_bf16((n_pos, shape.n_kv_heads, shape.head_dim), seed,
                            kv_tensor_id(shape, b, layer, kv), 1.0, 0.0, pos0 * hd)


def page_assignment(pages: List[int], need: List[int], seed: int = MASTER_SEED,
                    shuffle: bool = True) -> List[List[int]]:
    """Shuffle the allocated page ids (Fisher-Yates, seeded) and hand each request a
    consecutive run of ``need[b]`` of them."""
    ids = np.asarray(pages, dtype=np.int32)
    if shuffle:
        ids = shuffle_i32(ids, seed ^ SEED_PAGES)
    out, o = [], 0
    for n in need:
        out.append([int(x) for x in ids[o:o + n]])
        o += n
    return out


def pages_needed(ctx: int, steps: int) -> int:
    """Pages covering positions 0 .. ctx + steps - 1 (the step at position p writes slot p)."""
    return (ctx + steps + PAGE - 1) // PAGE
