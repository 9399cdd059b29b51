"""Host-side conveniences around :class:`Decoder`: upload bf16 weights held as
numpy uint16 bit patterns, build page tables, prefill K/V rows through
``mk_kv_write``. Marshalling only; nothing here computes any part of the step.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from . import PAGE, Decoder

PER_LAYER = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down", "router")


def to_device_bf16(a: np.ndarray, device="cuda"):
    import torch
    assert a.dtype == np.uint16
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def upload_weights(weights: Dict, device="cuda") -> Dict:
    out = {}
    for k, v in weights.items():
        if isinstance(v, list):
            out[k] = [to_device_bf16(x, device) for x in v]
        else:
            out[k] = to_device_bf16(v, device)
    return out


def page_table_tensor(rows: Sequence[Sequence[int]], max_pages_per_seq: int, device="cuda"):
    import torch
    pt = np.full((len(rows), max_pages_per_seq), -1, dtype=np.int32)
    for b, r in enumerate(rows):
        pt[b, :len(r)] = r
    return torch.from_numpy(pt).to(device)


def slots_for(pages: Sequence[int], pos0: int, n: int) -> np.ndarray:
    pos = np.arange(pos0, pos0 + n)
    return (np.asarray(pages, dtype=np.int64)[pos // PAGE] * PAGE + pos % PAGE).astype(np.int32)


def prefill_kv(dec: Decoder, layer: int, pages: Sequence[int], k_rows: np.ndarray,
               v_rows: np.ndarray, pos0: int = 0, device="cuda"):
    """Write K and V rows [n][Hkv][dh] (bf16 bit patterns) of positions pos0.. of one
    request into the pool through its page list."""
    import torch
    n = k_rows.shape[0]
    slots = torch.from_numpy(slots_for(pages, pos0, n)).to(device)
    dec.kv_write(layer, 0, slots, to_device_bf16(k_rows, device))
    dec.kv_write(layer, 1, slots, to_device_bf16(v_rows, device))


def read_kv_rows(dec: Decoder, layer: int, kv: int, slots: np.ndarray, device="cuda") -> np.ndarray:
    import torch
    s = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(device)
    rows = torch.empty((len(slots), dec.shape.n_kv_heads, dec.shape.head_dim), dtype=torch.bfloat16,
                       device=device)
    dec.kv_read(layer, kv, s, rows)
    torch.cuda.current_stream().synchronize()
    return rows.view(torch.int16).cpu().numpy().view(np.uint16)
