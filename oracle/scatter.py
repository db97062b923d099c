"""Write-side oracle: the K/V scatter into the page pool -- TEST
INFRASTRUCTURE ONLY (imported by tests, never by the product path).

"Reading vLLM's PagedAttention Kernel", section 3.2: the write path gives every
new token a flat physical slot, physical page * page_size + offset in the
page, and copies the token's key and value rows there; the read path gathers
them back through the block table.  The slots come from the runtime's page
ledger (``ledger.RequestPages.slot_mapping``: anllm "Tutorial 13" section 4, the
request cache's append; tiny-llm "Week 3 Day 4", "Decode Metadata").

This is the definition written out, one token at a time: no batching, no
reordering.  A negative slot (padding) or one past the pool skips the token,
the rule the library documents for pa_append.
"""
from __future__ import annotations

import numpy as np


def scatter_tokens(key_pages: np.ndarray, value_pages: np.ndarray, key: np.ndarray,
                   value: np.ndarray, slot_mapping) -> tuple:
    """Return copies of the pools [P, H_kv, page_size, D] with token t's rows
    key[t], value[t] ([T, H_kv, D]) written at slot slot_mapping[t]."""
    P, Hkv, ps, D = key_pages.shape
    if value_pages.shape != key_pages.shape:
        raise ValueError("key and value pools differ in shape")
    T = len(slot_mapping)
    if key.shape != (T, Hkv, D) or value.shape != (T, Hkv, D):
        raise ValueError("token rows must be [num_tokens, H_kv, D]")
    kp = key_pages.copy()
    vp = value_pages.copy()
    for t in range(T):
        s = int(slot_mapping[t])
        if s < 0 or s >= P * ps:
            continue
        page, off = s // ps, s % ps
        for h in range(Hkv):
            kp[page, h, off, :] = key[t, h, :]
            vp[page, h, off, :] = value[t, h, :]
    return kp, vp


def scatter_tokens_fp8(key_pages: np.ndarray, value_pages: np.ndarray, key_bf16: np.ndarray,
                       value_bf16: np.ndarray, slot_mapping, k_scale: float,
                       v_scale: float) -> tuple:
    """The scatter into an fp8 pool: uint8 pools [P, H_kv, page_size, D];
    token t's bf16 rows (uint16 bit patterns [T, H_kv, D]) are widened to
    fp32 exactly and stored as the codes of row / scale (fp8.quantize_rows:
    the write rule of the kv-cache dtype with per-tensor scales), at slot
    slot_mapping[t] as for scatter_tokens."""
    from . import fp8
    k32 = (np.asarray(key_bf16, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    v32 = (np.asarray(value_bf16, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    kq = fp8.quantize_rows(k32, k_scale)
    vq = fp8.quantize_rows(v32, v_scale)
    return scatter_tokens(key_pages, value_pages, kq, vq, slot_mapping)
