"""Seeded synthetic inputs for the paged-attention read path.

This module only *builds inputs*: page pools, block tables, context lengths,
query tensors and the garbage planted in slots that must never be read.  It
holds none of the attention arithmetic, and it is the one module that both the
CPU oracle tests and the GPU path consume.

Layouts follow the paged_attention contract of tiny-llm "Week 3 Day 4: Direct
Paged Attention" (section "The Paged Attention API", and "How This Maps to
tiny-llm" for the contiguous pool):

  query        [B, H_q, L, D]
  key_pages    [num_pages, H_kv, page_size, D]   (value_pages: same shape)
  block_table  [B, max_pages]  int32, unused entries padded with -1
  context_lens [B]             int32, visible tokens including the L new rows
  query_lens   [B] or None     int32, valid query rows per request (<= L)

Floating-point data is stored as float32 arrays for dtype "f32" and as uint16
bfloat16 bit patterns (round-to-nearest-even from a float32 draw) for "bf16".

Draw order is fixed per workload and stated in each builder; every draw comes
from one ``numpy.random.default_rng(seed)`` stream, so equal seeds give equal
bytes on every machine.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Union

import numpy as np

GARBAGE_DEFAULT = 1.0e4

# Standard seeds, one per named workload.
SEEDS = {"C1": 1, "C2": 2, "C3": 3, "C4": 4, "C5": 5}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for test helpers)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class PagedInputs:
    """One call's worth of paged-attention inputs (host arrays)."""

    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    B: int
    H_q: int
    H_kv: int
    L: int
    D: int
    page_size: int
    num_pages: int
    max_pages: int
    scale: float
    causal: bool
    query: np.ndarray               # [B, H_q, L, D] float32 or uint16 (bf16 bits)
    key_pages: np.ndarray           # [num_pages, H_kv, page_size, D]
    value_pages: np.ndarray         # same shape
    block_table: np.ndarray         # [B, max_pages] int32
    context_lens: np.ndarray        # [B] int32
    query_lens: Optional[np.ndarray] = None   # [B] int32 or None
    meta: Dict[str, object] = field(default_factory=dict)
    kv_dtype: Optional[str] = None  # None: pages share `dtype`; "fp8_e4m3": uint8 codes
    k_scale: float = 1.0            # fp8 pages: value = code value * scale
    v_scale: float = 1.0

    @property
    def group(self) -> int:
        return self.H_q // self.H_kv

    def rows_valid(self) -> np.ndarray:
        """Valid query rows per request (L where query_lens is absent)."""
        if self.query_lens is None:
            return np.full(self.B, self.L, dtype=np.int64)
        return self.query_lens.astype(np.int64)

    def kv_elem_bytes(self) -> int:
        """Bytes of one stored K or V element."""
        if self.kv_dtype == "fp8_e4m3":
            return 1
        return 4 if self.dtype == "f32" else 2

    def kv_token_bytes(self) -> int:
        """Bytes of one token's K plus V across all kv heads."""
        return self.H_kv * self.D * 2 * self.kv_elem_bytes()


@dataclass
class MixedInputs:
    """A ragged batch served as one decode call plus one prefill call that
    read the same page pool (the two share key_pages/value_pages arrays)."""

    name: str
    seed: int
    decode: PagedInputs
    prefill: PagedInputs
    meta: Dict[str, object] = field(default_factory=dict)


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

# fp8 pages hold 8-bit codes (sign, 4 exponent bits, 3 mantissa bits) drawn
# directly: sign uniform, exponent field uniform in [4, 8], mantissa uniform,
# i.e. magnitudes from 2^-3 to 1.875 * 2 before the pool's scale.  Garbage is
# a fixed code: 0x7E (the largest magnitude) for the default, 0xFE for its
# negative, 0x00 for zero, 0x7F (NaN) for "nan".
FP8_GARBAGE_CODES = {GARBAGE_DEFAULT: 0x7E, -GARBAGE_DEFAULT: 0xFE, 0.0: 0x00}


def _draw_fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    u = rng.integers(0, 1 << 8, size=shape, dtype=np.uint16)   # sign and mantissa bits
    e = rng.integers(4, 9, size=shape, dtype=np.uint16)        # exponent field
    return ((u & 0x80) | (e << 3) | (u & 0x07)).astype(np.uint8)


def _draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    if dtype == "fp8_e4m3":
        return _draw_fp8_codes(rng, shape)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _garbage_value(dtype: str, garbage: float) -> Union[np.float32, np.uint16, np.uint8]:
    if dtype == "fp8_e4m3":
        if garbage != garbage:  # NaN
            return np.uint8(0x7F)
        return np.uint8(FP8_GARBAGE_CODES[float(garbage)])
    g = np.array([garbage], dtype=np.float32)
    return f32_to_bf16_bits(g)[0] if dtype == "bf16" else g[0]


def _fill_pool(rng, dtype, num_pages, H_kv, ps, D, page_order: Sequence[int],
               valid_slots: Sequence[int], garbage) -> np.ndarray:
    """Pool whose pages in ``page_order`` get N(0,1) values in their first
    ``valid_slots[i]`` slots; every other slot and page holds ``garbage``.

    ``garbage`` is a float, or the string "random" (fresh N(0,1)*1e3 draws) or
    "nan".  Values are drawn page by page in ``page_order``.
    """
    np_dtype = {"bf16": np.uint16, "f32": np.float32, "fp8_e4m3": np.uint8}[dtype]
    pool = np.empty((num_pages, H_kv, ps, D), dtype=np_dtype)
    if isinstance(garbage, str) and garbage == "random":
        fill = None
    elif isinstance(garbage, str) and garbage == "nan":
        fill = _garbage_value(dtype, float("nan"))
    else:
        fill = _garbage_value(dtype, float(garbage))
    if fill is not None:
        pool[...] = fill
    else:
        # stale data of arbitrary magnitude from a child stream, so the live
        # values are the same bytes as with a constant garbage fill
        grng = rng.spawn(1)[0]
        chunk = max(1, (1 << 22) // (H_kv * ps * D))
        for s in range(0, num_pages, chunk):
            e = min(num_pages, s + chunk)
            if dtype == "fp8_e4m3":   # any byte, NaN codes included
                pool[s:e] = grng.integers(0, 256, size=(e - s, H_kv, ps, D), dtype=np.uint16)
                continue
            g = grng.standard_normal(size=(e - s, H_kv, ps, D), dtype=np.float32) * np.float32(1e3)
            pool[s:e] = f32_to_bf16_bits(g) if dtype == "bf16" else g
    order = np.asarray(page_order, dtype=np.int64)
    vs = np.asarray(valid_slots, dtype=np.int64)
    slot_idx = np.arange(ps)
    chunk = max(1, (1 << 22) // (H_kv * ps * D))      # ~4M elements per draw
    for s in range(0, len(order), chunk):
        e = min(len(order), s + chunk)
        vals = _draw_values(rng, (e - s, H_kv, ps, D), dtype)
        dead = slot_idx[None, :] >= vs[s:e, None]          # [pages, ps] unused slots
        if dead.any():
            pg, sl = np.nonzero(dead)
            if fill is not None:
                vals[pg, :, sl, :] = fill
            else:
                vals[pg, :, sl, :] = pool[order[s:e][pg], :, sl, :]
        pool[order[s:e]] = vals
    return pool


def _pages_needed(ctx: int, ps: int) -> int:
    return (ctx + ps - 1) // ps


def _tables_from_ids(ctx: Sequence[int], ps: int, max_pages: int,
                     page_ids: Sequence[Sequence[int]]) -> np.ndarray:
    bt = np.full((len(ctx), max_pages), -1, dtype=np.int32)
    for b, ids in enumerate(page_ids):
        bt[b, :len(ids)] = ids
    return bt


def _valid_slots_per_page(ctx: int, ps: int) -> List[int]:
    n = _pages_needed(ctx, ps)
    return [min(ps, ctx - i * ps) for i in range(n)]


def _queries(rng, dtype, B, H_q, L, D, query_lens, garbage):
    q = _draw_values(rng, (B, H_q, L, D), dtype)
    if query_lens is not None:
        fill = _garbage_value(dtype, GARBAGE_DEFAULT if isinstance(garbage, str) else float(garbage))
        for b in range(B):
            q[b, :, int(query_lens[b]):, :] = fill
    return q


# ----------------------------------------------------------------------------
# generic builder (tests)
# ----------------------------------------------------------------------------

def make_random(seed: int, *, B: int, H_q: int, H_kv: int, L: int, D: int,
                page_size: int, ctx: Union[Sequence[int], tuple], dtype: str = "bf16",
                causal: bool = True, query_lens: Optional[Sequence[int]] = None,
                extra_free_pages: int = 3, max_pages: Optional[int] = None,
                garbage=GARBAGE_DEFAULT, scale: Optional[float] = None,
                name: str = "random", kv_dtype: Optional[str] = None,
                kv_scales=(0.5, 0.5)) -> PagedInputs:
    """Random paged inputs.

    Draw order: context lengths (when ``ctx`` is a (lo, hi) range) ->
    physical-id permutation -> (random garbage) -> K -> V -> Q.
    Physical ids are a seeded permutation of the whole pool, so logical pages
    land at arbitrary physical pages; ``extra_free_pages`` pages stay free and
    hold garbage, as do unused tail slots of each request's last page.
    ``kv_dtype="fp8_e4m3"``: the pages hold random fp8 codes (see
    _draw_fp8_codes) with k_scale, v_scale = ``kv_scales``; the query and
    output keep ``dtype``.
    """
    rng = np.random.default_rng(seed)
    if isinstance(ctx, tuple):
        lo, hi = ctx
        ctx_l = [int(v) for v in rng.integers(lo, hi + 1, size=B)]
    else:
        ctx_l = [int(v) for v in ctx]
        assert len(ctx_l) == B
    if query_lens is not None:
        query_lens = np.asarray(query_lens, dtype=np.int32)
    npg = [_pages_needed(c, page_size) for c in ctx_l]
    if max_pages is None:
        max_pages = max(1, max(npg) if npg else 1)
    live = sum(npg)
    num_pages = max(1, live + extra_free_pages)
    perm = rng.permutation(num_pages)
    ids, cur = [], 0
    for n in npg:
        ids.append([int(p) for p in perm[cur:cur + n]])
        cur += n
    order = [p for row in ids for p in row]
    slots = [s for c in ctx_l for s in _valid_slots_per_page(c, page_size)]
    pdt = kv_dtype or dtype
    kp = _fill_pool(rng, pdt, num_pages, H_kv, page_size, D, order, slots, garbage)
    vp = _fill_pool(rng, pdt, num_pages, H_kv, page_size, D, order, slots, garbage)
    q = _queries(rng, dtype, B, H_q, L, D, query_lens, garbage)
    bt = _tables_from_ids(ctx_l, page_size, max_pages, ids)
    fp8 = kv_dtype == "fp8_e4m3"
    return PagedInputs(
        name=name, seed=seed, dtype=dtype, B=B, H_q=H_q, H_kv=H_kv, L=L, D=D,
        page_size=page_size, num_pages=num_pages, max_pages=max_pages,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)), causal=causal,
        query=q, key_pages=kp, value_pages=vp, block_table=bt,
        context_lens=np.asarray(ctx_l, dtype=np.int32), query_lens=query_lens,
        meta={"live_pages": live, "garbage": garbage}, kv_dtype=kv_dtype,
        k_scale=float(kv_scales[0]) if fp8 else 1.0, v_scale=float(kv_scales[1]) if fp8 else 1.0)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def make_c1(seed: int = SEEDS["C1"]) -> PagedInputs:
    """Tiny fp32 decode: B=2, H_q=H_kv=4, D=64, L=1, page_size=4,
    context_lens [10, 7], a pool of 16 pages.  Request 0 uses pages [12, 5, 3]
    (the worked address example of "Why block_table Matters"); request 1 takes
    two pages from a seeded permutation of the other 13.  Draw order:
    permutation -> K -> V -> Q."""
    rng = np.random.default_rng(seed)
    B, H, D, L, ps, P = 2, 4, 64, 1, 4, 16
    ctx = [10, 7]
    others = [p for p in range(P) if p not in (12, 5, 3)]
    perm = rng.permutation(len(others))
    ids = [[12, 5, 3], [others[perm[0]], others[perm[1]]]]
    order = [p for row in ids for p in row]
    slots = [s for c in ctx for s in _valid_slots_per_page(c, ps)]
    kp = _fill_pool(rng, "f32", P, H, ps, D, order, slots, GARBAGE_DEFAULT)
    vp = _fill_pool(rng, "f32", P, H, ps, D, order, slots, GARBAGE_DEFAULT)
    q = _queries(rng, "f32", B, H, L, D, None, GARBAGE_DEFAULT)
    bt = _tables_from_ids(ctx, ps, 3, ids)
    return PagedInputs(
        name="C1", seed=seed, dtype="f32", B=B, H_q=H, H_kv=H, L=L, D=D,
        page_size=ps, num_pages=P, max_pages=3, scale=1.0 / math.sqrt(D), causal=True,
        query=q, key_pages=kp, value_pages=vp, block_table=bt,
        context_lens=np.asarray(ctx, dtype=np.int32),
        meta={"workload": "tiny fp32 decode", "live_pages": 5})


def _uniform_pool_config(name, seed, *, B, H_q, H_kv, D, L, ps, ctx_lo, ctx_hi,
                         pool_pages=None, free_frac=None, prefix_lo=None,
                         prefix_hi=None, causal=True, kv_dtype=None,
                         kv_scales=(0.5, 0.5)) -> PagedInputs:
    """Shared builder for C2-C4.  Draw order: contexts (or prefixes) ->
    physical-id permutation -> K -> V -> Q."""
    rng = np.random.default_rng(seed)
    if prefix_lo is not None:
        prefix = rng.integers(prefix_lo, prefix_hi + 1, size=B)
        ctx = [int(p) + L for p in prefix]
        max_ctx = prefix_hi + L
    else:
        ctx = [int(c) for c in rng.integers(ctx_lo, ctx_hi + 1, size=B)]
        max_ctx = ctx_hi
    max_pages = _pages_needed(max_ctx, ps)
    npg = [_pages_needed(c, ps) for c in ctx]
    live = sum(npg)
    num_pages = pool_pages if pool_pages is not None else int(math.ceil(live * (1.0 + free_frac)))
    assert num_pages >= live
    perm = rng.permutation(num_pages)
    ids, cur = [], 0
    for n in npg:
        ids.append([int(p) for p in perm[cur:cur + n]])
        cur += n
    order = [p for row in ids for p in row]
    slots = [s for c in ctx for s in _valid_slots_per_page(c, ps)]
    pdt = kv_dtype or "bf16"
    kp = _fill_pool(rng, pdt, num_pages, H_kv, ps, D, order, slots, GARBAGE_DEFAULT)
    vp = _fill_pool(rng, pdt, num_pages, H_kv, ps, D, order, slots, GARBAGE_DEFAULT)
    q = _queries(rng, "bf16", B, H_q, L, D, None, GARBAGE_DEFAULT)
    bt = _tables_from_ids(ctx, ps, max_pages, ids)
    fp8 = kv_dtype == "fp8_e4m3"
    return PagedInputs(
        name=name, seed=seed, dtype="bf16", B=B, H_q=H_q, H_kv=H_kv, L=L, D=D,
        page_size=ps, num_pages=num_pages, max_pages=max_pages,
        scale=1.0 / math.sqrt(D), causal=causal, query=q, key_pages=kp,
        value_pages=vp, block_table=bt, context_lens=np.asarray(ctx, dtype=np.int32),
        meta={"live_pages": live}, kv_dtype=kv_dtype,
        k_scale=float(kv_scales[0]) if fp8 else 1.0, v_scale=float(kv_scales[1]) if fp8 else 1.0)


def make_c2(seed: int = SEEDS["C2"]) -> PagedInputs:
    """GQA decode, bf16, Llama-3-8B head shape: B=64, H_q=32, H_kv=8, D=128,
    L=1, page_size=16, context_lens ~ U{128..4096}, a pool of 20000 pages
    with shuffled physical ids."""
    x = _uniform_pool_config("C2", seed, B=64, H_q=32, H_kv=8, D=128, L=1, ps=16,
                             ctx_lo=128, ctx_hi=4096, pool_pages=20000)
    x.meta["workload"] = "GQA decode bf16 B64 Hq32 Hkv8 D128 ps16 ctx U[128,4096]"
    return x


def make_c2_fp8(seed: int = SEEDS["C2"]) -> PagedInputs:
    """The GQA decode workload with fp8 (E4M3) K/V pages: the shape, contexts
    and pool of C2 (same seed, same draw order), page elements drawn as fp8
    codes (_draw_fp8_codes), k_scale = v_scale = 0.5; query and output bf16."""
    x = _uniform_pool_config("C2-fp8", seed, B=64, H_q=32, H_kv=8, D=128, L=1, ps=16,
                             ctx_lo=128, ctx_hi=4096, pool_pages=20000, kv_dtype="fp8_e4m3")
    x.meta["workload"] = "GQA decode bf16 query, fp8 e4m3 pages, B64 Hq32 Hkv8 D128 ps16 ctx U[128,4096]"
    return x


def make_c3(seed: int = SEEDS["C3"]) -> PagedInputs:
    """Chunked causal prefill, bf16, Qwen2.5-7B-like heads: B=4, H_q=28,
    H_kv=4, D=128, a 512-row query chunk appended after a prefix
    ~ U{0..2048}; page_size=16; pool = live pages + 10% free pages."""
    x = _uniform_pool_config("C3", seed, B=4, H_q=28, H_kv=4, D=128, L=512, ps=16,
                             ctx_lo=None, ctx_hi=None, free_frac=0.10,
                             prefix_lo=0, prefix_hi=2048)
    x.meta["workload"] = "chunked causal prefill bf16 B4 Hq28 Hkv4 D128 L512 prefix U[0,2048] ps16"
    return x


def make_c3_fp8(seed: int = SEEDS["C3"]) -> PagedInputs:
    """The chunked prefill workload with fp8 (E4M3) K/V pages: the shape,
    prefixes and pool of C3 (same seed, same draw order), page elements
    drawn as fp8 codes (_draw_fp8_codes), k_scale = v_scale = 0.5; query and
    output bf16."""
    x = _uniform_pool_config("C3-fp8", seed, B=4, H_q=28, H_kv=4, D=128, L=512, ps=16,
                             ctx_lo=None, ctx_hi=None, free_frac=0.10,
                             prefix_lo=0, prefix_hi=2048, kv_dtype="fp8_e4m3")
    x.meta["workload"] = ("chunked causal prefill bf16 query, fp8 e4m3 pages, B4 Hq28 Hkv4 D128 "
                          "L512 prefix U[0,2048] ps16")
    return x


def make_c4(seed: int = SEEDS["C4"]) -> PagedInputs:
    """Long-context split-KV decode, bf16: B=8, H_q=32, H_kv=8, D=128, L=1,
    context_lens ~ U{32768..131072}, page_size=16, pool = live + 10% free."""
    x = _uniform_pool_config("C4", seed, B=8, H_q=32, H_kv=8, D=128, L=1, ps=16,
                             ctx_lo=32768, ctx_hi=131072, free_frac=0.10)
    x.meta["workload"] = "long-context decode bf16 B8 Hq32 Hkv8 D128 ps16 ctx U[32768,131072]"
    return x


def make_c5(seed: int = SEEDS["C5"]) -> MixedInputs:
    """Mixed ragged batch, bf16: 48 decode requests (L=1) and 8 prefill
    requests (L ~ U{64..256}); H_q=32, H_kv=8, D=128, page_size=128, contexts
    ~ U{256..16384}.  14 requests (25%) share one 2048-token prefix: their
    first 16 block-table entries name the same 16 physical pages (complete and
    read-only).  Pool = ceil(used / 0.9) pages, ids shuffled.

    Draw order: prefill query lengths -> sharer choice -> contexts ->
    physical-id permutation -> K -> V -> Q(decode) -> Q(prefill).
    """
    rng = np.random.default_rng(seed)
    H_q, H_kv, D, ps = 32, 8, 128, 128
    n_dec, n_pre, shared_tokens = 48, 8, 2048
    n_req = n_dec + n_pre
    max_ctx = 16384
    max_pages = max_ctx // ps
    qlen_pre = [int(v) for v in rng.integers(64, 256 + 1, size=n_pre)]
    qlen = [1] * n_dec + qlen_pre
    sharers = sorted(int(v) for v in rng.choice(n_req, size=n_req // 4, replace=False))
    ctx = []
    for r in range(n_req):
        lo = shared_tokens + qlen[r] if r in sharers else max(256, qlen[r])
        ctx.append(int(rng.integers(lo, max_ctx + 1)))
    n_shared_pages = shared_tokens // ps
    own_pages = []
    for r in range(n_req):
        n = _pages_needed(ctx[r], ps)
        own_pages.append(n - n_shared_pages if r in sharers else n)
    used = n_shared_pages + sum(own_pages)
    num_pages = int(math.ceil(used / 0.9))
    perm = rng.permutation(num_pages)
    shared_ids = [int(p) for p in perm[:n_shared_pages]]
    cur = n_shared_pages
    ids, order, slots = [], list(shared_ids), [ps] * n_shared_pages
    for r in range(n_req):
        mine = [int(p) for p in perm[cur:cur + own_pages[r]]]
        cur += own_pages[r]
        row = (shared_ids + mine) if r in sharers else mine
        ids.append(row)
        vs = _valid_slots_per_page(ctx[r], ps)
        order.extend(mine)
        slots.extend(vs[len(vs) - len(mine):])
    kp = _fill_pool(rng, "bf16", num_pages, H_kv, ps, D, order, slots, GARBAGE_DEFAULT)
    vp = _fill_pool(rng, "bf16", num_pages, H_kv, ps, D, order, slots, GARBAGE_DEFAULT)
    q_dec = _queries(rng, "bf16", n_dec, H_q, 1, D, None, GARBAGE_DEFAULT)
    L_pre = max(qlen_pre)
    ql_pre = np.asarray(qlen_pre, dtype=np.int32)
    q_pre = _queries(rng, "bf16", n_pre, H_q, L_pre, D, ql_pre, GARBAGE_DEFAULT)
    bt = _tables_from_ids(ctx, ps, max_pages, ids)
    cl = np.asarray(ctx, dtype=np.int32)
    common = dict(seed=seed, dtype="bf16", H_q=H_q, H_kv=H_kv, D=D, page_size=ps,
                  num_pages=num_pages, max_pages=max_pages, scale=1.0 / math.sqrt(D),
                  causal=True, key_pages=kp, value_pages=vp)
    dec = PagedInputs(name="C5-decode", B=n_dec, L=1, query=q_dec,
                      block_table=np.ascontiguousarray(bt[:n_dec]),
                      context_lens=np.ascontiguousarray(cl[:n_dec]), **common)
    pre = PagedInputs(name="C5-prefill", B=n_pre, L=L_pre, query=q_pre,
                      block_table=np.ascontiguousarray(bt[n_dec:]),
                      context_lens=np.ascontiguousarray(cl[n_dec:]),
                      query_lens=ql_pre, **common)
    meta = {"workload": "mixed ragged batch bf16 48 decode + 8 prefill, Hq32 Hkv8 D128 ps128, "
                        "25% share a 2048-token prefix",
            "sharers": sharers, "shared_page_ids": shared_ids, "used_pages": used}
    dec.meta.update(meta)
    pre.meta.update(meta)
    return MixedInputs(name="C5", seed=seed, decode=dec, prefill=pre, meta=meta)


@dataclass
class RaggedInputs:
    """A ragged batch as ONE call over packed query rows: request b owns rows
    query_start_loc[b] .. query_start_loc[b + 1] - 1 of query [T, H_q, D]
    (token-major).  ``parts`` holds the same requests as padded inputs (the
    decode requests first, then the prefill ones, in the order of the packed
    batch), which is how the oracle sees them."""

    name: str
    seed: int
    B: int
    H_q: int
    H_kv: int
    D: int
    page_size: int
    num_pages: int
    max_pages: int
    scale: float
    causal: bool
    max_query_len: int
    query: np.ndarray               # [T, H_q, D] uint16 (bf16 bits)
    query_start_loc: np.ndarray     # [B + 1] int32
    key_pages: np.ndarray
    value_pages: np.ndarray
    block_table: np.ndarray         # [B, max_pages]
    context_lens: np.ndarray        # [B]
    parts: MixedInputs

    def unpack(self, packed: np.ndarray):
        """Split packed output rows [T, H_q, D] into the padded layouts of the
        decode part [B_dec, H_q, 1, D] and the prefill part [B_pre, H_q, L, D]
        (rows past a request's own left at zero)."""
        dec, pre = self.parts.decode, self.parts.prefill
        out_d = np.zeros((dec.B, self.H_q, dec.L, self.D), dtype=packed.dtype)
        out_p = np.zeros((pre.B, self.H_q, pre.L, self.D), dtype=packed.dtype)
        qsl = self.query_start_loc
        for b in range(self.B):
            rows = packed[qsl[b]:qsl[b + 1]].transpose(1, 0, 2)   # [H_q, Lb, D]
            if b < dec.B:
                out_d[b, :, :rows.shape[1]] = rows
            else:
                out_p[b - dec.B, :, :rows.shape[1]] = rows
        return out_d, out_p


def pack_ragged(m: MixedInputs) -> RaggedInputs:
    """The requests of a mixed workload (decode part, then prefill part) as
    one batch of packed query rows over the same pool."""
    dec, pre = m.decode, m.prefill
    rows, lens = [], []
    for b in range(dec.B):
        n = int(dec.rows_valid()[b])
        rows.append(dec.query[b, :, :n].transpose(1, 0, 2))
        lens.append(n)
    for b in range(pre.B):
        n = int(pre.rows_valid()[b])
        rows.append(pre.query[b, :, :n].transpose(1, 0, 2))
        lens.append(n)
    qsl = np.zeros(len(lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    assert dec.max_pages == pre.max_pages
    return RaggedInputs(
        name=m.name + "-ragged", seed=m.seed, B=dec.B + pre.B, H_q=dec.H_q, H_kv=dec.H_kv,
        D=dec.D, page_size=dec.page_size, num_pages=dec.num_pages, max_pages=dec.max_pages,
        scale=dec.scale, causal=dec.causal, max_query_len=max(lens),
        query=np.ascontiguousarray(np.concatenate(rows, axis=0)), query_start_loc=qsl,
        key_pages=dec.key_pages, value_pages=dec.value_pages,
        block_table=np.ascontiguousarray(np.concatenate([dec.block_table, pre.block_table])),
        context_lens=np.ascontiguousarray(np.concatenate([dec.context_lens, pre.context_lens])),
        parts=m)


# ----------------------------------------------------------------------------
# shared prefixes: groups of consecutive requests whose tables name the same
# first pages (block sharing, as prefix caching produces it)
# ----------------------------------------------------------------------------

@dataclass
class SharedGroups:
    """Group k holds requests group_start[k] .. group_start[k + 1] - 1 and
    shares its first prefix_lens[k] keys (whole pages); the groups are
    consecutive ranges from request 0, and requests past the last group share
    nothing."""

    group_start: np.ndarray   # [G + 1] int32
    prefix_lens: np.ndarray   # [G] int32

    @property
    def num_groups(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def max_group_size(self) -> int:
        return int(np.diff(self.group_start).max()) if self.num_groups else 1


def make_shared(seed: int, *, H_q: int, H_kv: int, L: int, D: int, page_size: int,
                group_sizes: Sequence[int], prefix_pages: Sequence[int],
                suffix: tuple, dtype: str = "bf16", causal: bool = True,
                query_lens: Optional[Sequence[int]] = None, extra_free_pages: int = 3,
                garbage=GARBAGE_DEFAULT, name: str = "shared", kv_dtype: Optional[str] = None,
                kv_scales=(0.5, 0.5)):
    """Requests in groups of consecutive requests: group k has
    ``group_sizes[k]`` members whose first ``prefix_pages[k]`` block-table
    entries name the same physical pages (complete pages), followed by pages
    of their own; member context = prefix keys + a suffix of U{suffix[0]..
    suffix[1]} keys (suffix[0] >= L, so every query row sees the whole
    prefix).  ``kv_dtype="fp8_e4m3"``: the pages hold fp8 codes (as in
    make_random) with k_scale, v_scale = ``kv_scales``.  Returns
    (PagedInputs, SharedGroups).

    Draw order: suffix lengths -> physical-id permutation -> K -> V -> Q.
    """
    rng = np.random.default_rng(seed)
    assert len(group_sizes) == len(prefix_pages) and suffix[0] >= L
    B = int(sum(group_sizes))
    suf = [int(v) for v in rng.integers(suffix[0], suffix[1] + 1, size=B)]
    ctx, member_of = [], []
    for k, n in enumerate(group_sizes):
        for _ in range(n):
            member_of.append(k)
    for b in range(B):
        ctx.append(prefix_pages[member_of[b]] * page_size + suf[b])
    own = [_pages_needed(ctx[b], page_size) - prefix_pages[member_of[b]] for b in range(B)]
    live = sum(prefix_pages) + sum(own)
    num_pages = max(1, live + extra_free_pages)
    perm = rng.permutation(num_pages)
    cur = 0
    shared_ids = []
    for k in range(len(group_sizes)):
        shared_ids.append([int(p) for p in perm[cur:cur + prefix_pages[k]]])
        cur += prefix_pages[k]
    order = [p for ids in shared_ids for p in ids]
    slots = [page_size] * len(order)
    ids = []
    for b in range(B):
        mine = [int(p) for p in perm[cur:cur + own[b]]]
        cur += own[b]
        ids.append(shared_ids[member_of[b]] + mine)
        order.extend(mine)
        vs = _valid_slots_per_page(ctx[b], page_size)
        slots.extend(vs[len(vs) - len(mine):])
    max_pages = max(_pages_needed(c, page_size) for c in ctx)
    if query_lens is not None:
        query_lens = np.asarray(query_lens, dtype=np.int32)
    pdt = kv_dtype or dtype
    kp = _fill_pool(rng, pdt, num_pages, H_kv, page_size, D, order, slots, garbage)
    vp = _fill_pool(rng, pdt, num_pages, H_kv, page_size, D, order, slots, garbage)
    q = _queries(rng, dtype, B, H_q, L, D, query_lens, garbage)
    bt = _tables_from_ids(ctx, page_size, max_pages, ids)
    fp8 = kv_dtype == "fp8_e4m3"
    gs = np.zeros(len(group_sizes) + 1, dtype=np.int32)
    gs[1:] = np.cumsum(group_sizes)
    x = PagedInputs(
        name=name, seed=seed, dtype=dtype, B=B, H_q=H_q, H_kv=H_kv, L=L, D=D,
        page_size=page_size, num_pages=num_pages, max_pages=max_pages,
        scale=1.0 / math.sqrt(D), causal=causal, query=q, key_pages=kp, value_pages=vp,
        block_table=bt, context_lens=np.asarray(ctx, dtype=np.int32), query_lens=query_lens,
        meta={"live_pages": live, "garbage": garbage}, kv_dtype=kv_dtype,
        k_scale=float(kv_scales[0]) if fp8 else 1.0, v_scale=float(kv_scales[1]) if fp8 else 1.0)
    return x, SharedGroups(gs, np.asarray([p * page_size for p in prefix_pages], dtype=np.int32))


def c5_decode_grouped(m: MixedInputs):
    """The decode part of a mixed workload with its prefix sharers moved to
    the front as one group (the shared pages' keys as its prefix), the other
    requests after it in no group.  Returns (PagedInputs, SharedGroups,
    order): request i of the result is request order[i] of the decode part."""
    dec = m.decode
    sharers = [b for b in m.meta["sharers"] if b < dec.B]
    rest = [b for b in range(dec.B) if b not in sharers]
    order = np.asarray(sharers + rest, dtype=np.int64)
    x = PagedInputs(
        name=dec.name + "-grouped", seed=dec.seed, dtype=dec.dtype, B=dec.B, H_q=dec.H_q,
        H_kv=dec.H_kv, L=dec.L, D=dec.D, page_size=dec.page_size, num_pages=dec.num_pages,
        max_pages=dec.max_pages, scale=dec.scale, causal=dec.causal,
        query=np.ascontiguousarray(dec.query[order]), key_pages=dec.key_pages,
        value_pages=dec.value_pages, block_table=np.ascontiguousarray(dec.block_table[order]),
        context_lens=np.ascontiguousarray(dec.context_lens[order]),
        query_lens=None if dec.query_lens is None else
        np.ascontiguousarray(dec.query_lens[order]), meta=dict(dec.meta))
    n_shared = len(m.meta["shared_page_ids"])
    gs = np.asarray([0, len(sharers)] if sharers else [0], dtype=np.int32)
    pre = [n_shared * dec.page_size] if sharers else []
    return x, SharedGroups(gs, np.asarray(pre, dtype=np.int32)), order


BUILDERS = {"C1": make_c1, "C2": make_c2, "C3": make_c3, "C4": make_c4, "C5": make_c5}


def make_config(name: str, seed: Optional[int] = None):
    """Build one of the five named workloads (C5 returns a MixedInputs)."""
    fn = BUILDERS[name]
    return fn() if seed is None else fn(seed)


# ----------------------------------------------------------------------------
# write path: new tokens appended after each request's cached context
# ----------------------------------------------------------------------------

@dataclass
class AppendInputs:
    """One step's K/V write: ``n_new[b]`` tokens of request b land at
    positions ctx_old[b] .. ctx_old[b] + n_new[b] - 1 of its block table
    (``paged`` covers the grown contexts; its pool holds the old tokens and
    garbage elsewhere).  Token rows are request-major; ``pad_tokens`` extra
    rows with slot -1 are spread among them (padding the runtime may send)."""

    name: str
    seed: int
    paged: PagedInputs
    ctx_old: np.ndarray             # [B] int32
    n_new: np.ndarray               # [B] int32
    key: np.ndarray                 # [T, H_kv, D] float32 or uint16 (bf16 bits)
    value: np.ndarray               # [T, H_kv, D]
    slot_mapping: np.ndarray        # [T] int32: page * page_size + offset, or -1

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    def moved_bytes(self) -> int:
        """Bytes an append reads plus writes for the tokens with a slot (K and
        V rows read in `dtype`, written in the pool's element type)."""
        p = self.paged
        live = int((self.slot_mapping >= 0).sum())
        src = 4 if p.dtype == "f32" else 2
        return live * p.H_kv * p.D * (src + p.kv_elem_bytes()) * 2


def make_append(seed: int, *, B: int, H_kv: int, D: int, page_size: int,
                ctx_old: Union[Sequence[int], tuple], n_new: Union[Sequence[int], tuple],
                dtype: str = "bf16", pad_tokens: int = 0, extra_free_pages: int = 3,
                garbage=GARBAGE_DEFAULT, name: str = "append",
                kv_dtype: Optional[str] = None, kv_scales=(0.5, 0.5)) -> AppendInputs:
    """Random write-path inputs.  Draw order: the paged pool of the grown
    contexts (make_random with this seed) -> old context lengths (when a
    range) -> new-token counts (when a range) -> pad positions -> K rows ->
    V rows, from a child stream of the seed.  kv_dtype "fp8_e4m3": the pool
    holds fp8 codes with scales kv_scales; the new rows stay in `dtype`."""
    rng = np.random.default_rng([seed, 1])
    old = ([int(v) for v in rng.integers(ctx_old[0], ctx_old[1] + 1, size=B)]
           if isinstance(ctx_old, tuple) else [int(v) for v in ctx_old])
    new = ([int(v) for v in rng.integers(n_new[0], n_new[1] + 1, size=B)]
           if isinstance(n_new, tuple) else [int(v) for v in n_new])
    assert len(old) == B and len(new) == B
    grown = [o + n for o, n in zip(old, new)]
    paged = make_random(seed, B=B, H_q=H_kv, H_kv=H_kv, L=1, D=D, page_size=page_size,
                        ctx=grown, dtype=dtype, causal=False,
                        extra_free_pages=extra_free_pages, garbage=garbage, name=name,
                        kv_dtype=kv_dtype, kv_scales=kv_scales)
    slots = []
    bt = paged.block_table
    for b in range(B):
        for pos in range(old[b], grown[b]):
            slots.append(int(bt[b, pos // page_size]) * page_size + pos % page_size)
    T = len(slots) + pad_tokens
    pad_at = set(int(i) for i in rng.choice(T, size=pad_tokens, replace=False)) if pad_tokens else set()
    it = iter(slots)
    slot_mapping = np.array([-1 if t in pad_at else next(it) for t in range(T)], dtype=np.int32)
    key = _draw_values(rng, (T, H_kv, D), dtype)
    value = _draw_values(rng, (T, H_kv, D), dtype)
    return AppendInputs(name=name, seed=seed, paged=paged,
                        ctx_old=np.asarray(old, dtype=np.int32),
                        n_new=np.asarray(new, dtype=np.int32), key=key, value=value,
                        slot_mapping=slot_mapping)
