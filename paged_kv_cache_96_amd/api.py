"""Thin Python binding of libpa.so for torch device tensors.

Each function marshals tensors into the C structs of include/pa.h and calls
the C entry point of the same name on torch's current HIP stream; the
computation itself happens only in the HIP kernels.  torch provides device
memory and streams, nothing else.
"""
from __future__ import annotations

import ctypes
import math
from typing import NamedTuple, Optional

import torch

from . import _lib
from ._lib import (PaArgs, PaWorkspace, SCHEDULE_BALANCED, SCHEDULE_KEY_SPLIT,  # noqa: F401
                   SCHEDULE_PARTITIONS)

_DTYPES = {torch.float32: _lib.PA_DTYPE_F32, torch.bfloat16: _lib.PA_DTYPE_BF16}
_MASKS = {"none": _lib.PA_MASK_NONE, None: _lib.PA_MASK_NONE, "causal": _lib.PA_MASK_CAUSAL}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpa must be contiguous")
    return t.data_ptr()


def _int32(t: Optional[torch.Tensor], name: str) -> Optional[torch.Tensor]:
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _same_gpu(ref: torch.Tensor, **tensors) -> None:
    """The kernels dereference every pointer on the GPU: each tensor must live
    on the device of `ref`, and that device must be a GPU."""
    if ref.device.type != "cuda":
        raise ValueError("tensors passed to libpa must be on the GPU")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, not on {ref.device}")


def _shape(t: Optional[torch.Tensor], want: tuple, name: str) -> None:
    if t is not None and tuple(t.shape) != want:
        raise ValueError(f"{name} must have shape {list(want)}, not {list(t.shape)}")


def make_args(query: torch.Tensor, key_pages: torch.Tensor, value_pages: torch.Tensor,
              block_table: torch.Tensor, context_lens: torch.Tensor, out: torch.Tensor, *,
              scale: Optional[float] = None, mask: Optional[str] = "causal",
              query_lens: Optional[torch.Tensor] = None,
              debug_trace: Optional[torch.Tensor] = None,
              debug_visits: Optional[torch.Tensor] = None,
              k_scale: Optional[float] = None, v_scale: Optional[float] = None,
              query_start_loc: Optional[torch.Tensor] = None,
              max_query_len: Optional[int] = None,
              debug_errors: Optional[torch.Tensor] = None) -> PaArgs:
    """Fill a pa_args from tensors (shapes as in include/pa.h).  uint8 pages
    are fp8 E4M3 codes (PA_KV_FP8_E4M3) and need k_scale and v_scale.  With
    query_start_loc ([B + 1] int32) the query and out are packed rows
    [T, H_q, D] and max_query_len bounds every request's rows.
    debug_errors ([2] int32, zeroed by the caller) turns on the contract
    check of the calls made with these arguments."""
    if query_start_loc is not None:
        if query.dim() != 3 or max_query_len is None or query_lens is not None:
            raise ValueError("packed rows: query [T, H_q, D], max_query_len, no query_lens")
        T, Hq, D = query.shape
        B, L = block_table.shape[0], int(max_query_len)
        _int32(query_start_loc, "query_start_loc")
        _shape(query_start_loc, (B + 1,), "query_start_loc")
    else:
        B, Hq, L, D = query.shape
    P, Hkv, ps, D2 = key_pages.shape
    if D2 != D or tuple(value_pages.shape) != tuple(key_pages.shape):
        raise ValueError("query / key_pages / value_pages head sizes disagree")
    if tuple(out.shape) != tuple(query.shape) or out.dtype != query.dtype:
        raise ValueError("out must match query in shape and dtype")
    fp8 = key_pages.dtype == torch.uint8
    if value_pages.dtype != key_pages.dtype:
        raise ValueError("key_pages and value_pages must share one dtype")
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("fp8 (uint8) pages need k_scale and v_scale")
    if not fp8 and key_pages.dtype != query.dtype:
        raise ValueError("query and pages must share one dtype (or the pages be fp8 codes)")
    _int32(block_table, "block_table")
    _int32(context_lens, "context_lens")
    _int32(query_lens, "query_lens")
    _int32(debug_trace, "debug_trace")
    _int32(debug_visits, "debug_visits")
    _int32(debug_errors, "debug_errors")
    _same_gpu(query, key_pages=key_pages, value_pages=value_pages, block_table=block_table,
              context_lens=context_lens, out=out, query_lens=query_lens,
              debug_trace=debug_trace, debug_visits=debug_visits,
              query_start_loc=query_start_loc, debug_errors=debug_errors)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch, max_pages]")
    cap = block_table.shape[1] * ps
    _shape(context_lens, (B,), "context_lens")
    _shape(query_lens, (B,), "query_lens")
    _shape(debug_trace, (B, cap, 2), "debug_trace")
    _shape(debug_visits, (B, Hkv, cap), "debug_visits")
    _shape(debug_errors, (2,), "debug_errors")
    a = PaArgs()
    a.query = _ptr(query)
    a.key_pages = _ptr(key_pages)
    a.value_pages = _ptr(value_pages)
    a.block_table = _ptr(block_table)
    a.context_lens = _ptr(context_lens)
    a.query_lens = _ptr(query_lens)
    a.out = _ptr(out)
    a.batch, a.num_q_heads, a.num_kv_heads, a.q_len, a.head_dim = B, Hq, Hkv, L, D
    a.num_pages, a.page_size, a.max_pages = P, ps, block_table.shape[1]
    a.dtype = _DTYPES.get(query.dtype, 99)  # 99: the library rejects it as unsupported
    a.mask = _MASKS[mask]
    a.scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
    a.debug_trace = _ptr(debug_trace)
    a.debug_visits = _ptr(debug_visits)
    a.kv_dtype = _lib.PA_KV_FP8_E4M3 if fp8 else _lib.PA_KV_SAME
    a.k_scale = float(k_scale) if fp8 else 1.0
    a.v_scale = float(v_scale) if fp8 else 1.0
    a.query_start_loc = _ptr(query_start_loc)
    a.num_tokens = int(query.shape[0]) if query_start_loc is not None else 0
    a.debug_errors = _ptr(debug_errors)
    # the struct holds raw device addresses: keep the tensors alive with it
    a._tensors = (query, key_pages, value_pages, block_table, context_lens, out, query_lens,
                  debug_trace, debug_visits, query_start_loc, debug_errors)
    return a


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class DecodePlan(NamedTuple):
    """What pa_decode_plan chose: the schedule (SCHEDULE_PARTITIONS or
    SCHEDULE_BALANCED), partitions or piece slots, the partition size
    (partition schedule only), the size of the partial states in bytes and
    the number of arrival counters of a fused merge (balanced only)."""
    num_splits: int
    partition_tokens: int
    workspace_bytes: int
    schedule: int
    num_counters: int


def pa_decode_plan(args: PaArgs, *, num_cus: int = 0, partition_tokens: int = 0) -> DecodePlan:
    """The library's plan for `args`; partition_tokens > 0 asks for the
    partition schedule with that partition size."""
    ws = PaWorkspace()
    ws.partition_tokens = int(partition_tokens)
    nbytes = ctypes.c_size_t(0)
    _lib.check("pa_decode_plan", _lib.lib().pa_decode_plan(ctypes.byref(args), int(num_cus),
                                                            ctypes.byref(ws), ctypes.byref(nbytes)))
    return DecodePlan(ws.num_splits, ws.partition_tokens, nbytes.value, ws.schedule,
                      ws.num_counters)


class Workspace:
    """Device buffers of a decode plan (torch owns the memory).  Partition
    schedule: states [B, H_q, L, num_splits(, D)]; balanced schedule:
    `block_rows` states per piece slot, [num_splits, block_rows(, D)].  The
    buffers are allocated and the counters zeroed on torch's current stream:
    a call on another stream must first wait for it."""

    def __init__(self, B: int, Hq: int, L: int, D: int, num_splits: int, partition_tokens: int,
                 device, schedule: int = SCHEDULE_PARTITIONS, block_rows: int = 0,
                 num_counters: int = 0):
        self.num_splits = int(num_splits)
        self.schedule = int(schedule)
        self.partition_tokens = int(partition_tokens)
        # arrival counters of the fused merge: zeroed once, left zero by every call
        self.counters = (torch.zeros(int(num_counters), dtype=torch.int32, device=device)
                         if num_counters > 0 else None)
        if self.num_splits > 1:
            if self.schedule == SCHEDULE_BALANCED:
                if block_rows < 1:
                    raise ValueError("the balanced schedule needs block_rows")
                lead = (self.num_splits, int(block_rows))
            else:
                lead = (B, Hq, L, self.num_splits)
            self.partial_out = torch.empty(lead + (D,), dtype=torch.float32, device=device)
            self.partial_lse = torch.empty(lead, dtype=torch.float32, device=device)
        else:
            self.partial_out = self.partial_lse = None
        self.c = PaWorkspace()
        self.c.partial_out = _ptr(self.partial_out)
        self.c.partial_lse = _ptr(self.partial_lse)
        self.c.num_splits = self.num_splits
        self.c.partition_tokens = self.partition_tokens
        self.c.schedule = self.schedule
        self.c.num_counters = int(num_counters)
        self.c.counters = _ptr(self.counters)

    def tensors(self):
        """The device tensors of the workspace."""
        return [t for t in (self.partial_out, self.partial_lse, self.counters) if t is not None]

    @classmethod
    def for_plan(cls, plan: DecodePlan, query: torch.Tensor, fused: bool = True) -> "Workspace":
        """Buffers for `plan`; `fused` (balanced schedule) adds the arrival
        counters, so that pa_decode merges the pieces itself."""
        B, Hq, L, D = query.shape
        rows = 0
        if plan.schedule == SCHEDULE_BALANCED and plan.num_splits > 1:
            rows = plan.workspace_bytes // (plan.num_splits * (D + 1) * 4)
        return cls(B, Hq, L, D, plan.num_splits, plan.partition_tokens, query.device,
                   schedule=plan.schedule, block_rows=rows,
                   num_counters=plan.num_counters if fused else 0)


def pa_decode(args: PaArgs, workspace: Optional[Workspace] = None, stream=None) -> None:
    ws = ctypes.byref(workspace.c) if workspace is not None else None
    _lib.check("pa_decode", _lib.lib().pa_decode(ctypes.byref(args), ws, _stream(stream)))


def pa_decode_noalloc(args: PaArgs, stream=None) -> None:
    """pa_decode (balanced schedule, fused merge) with the library's own
    scratch in place of a workspace: allocates nothing."""
    _lib.check("pa_decode_noalloc", _lib.lib().pa_decode_noalloc(ctypes.byref(args),
                                                                  _stream(stream)))


def pa_split_reduce(args: PaArgs, workspace: Workspace, stream=None) -> None:
    _lib.check("pa_split_reduce", _lib.lib().pa_split_reduce(ctypes.byref(args),
                                                              ctypes.byref(workspace.c),
                                                              _stream(stream)))


class PrefillPlan(NamedTuple):
    """What pa_prefill_plan chose: the slots of the key split (0: the call
    runs unsplit and needs no workspace), the size of the piece states in
    bytes and the number of arrival counters."""
    num_splits: int
    workspace_bytes: int
    num_counters: int


def pa_prefill_plan(args: PaArgs, *, num_cus: int = 0) -> PrefillPlan:
    ws = PaWorkspace()
    nbytes = ctypes.c_size_t(0)
    _lib.check("pa_prefill_plan", _lib.lib().pa_prefill_plan(ctypes.byref(args), int(num_cus),
                                                              ctypes.byref(ws), ctypes.byref(nbytes)))
    return PrefillPlan(ws.num_splits, nbytes.value, ws.num_counters)


class PrefillWorkspace:
    """Device buffers of a prefill plan (torch owns the memory): piece states
    partial_out [num_splits, D / 8, 256, 4] and partial_lse [num_splits, 2,
    256] fp32, and the arrival counters (zeroed once, left zero by every
    call).  Allocated and zeroed on torch's current stream: a call on
    another stream must first wait for it."""

    def __init__(self, plan: PrefillPlan, D: int, device):
        self.num_splits = int(plan.num_splits)
        self.c = PaWorkspace()
        self.c.schedule = SCHEDULE_KEY_SPLIT
        self.c.num_splits = self.num_splits
        self.c.num_counters = int(plan.num_counters)
        if self.num_splits > 0:
            self.partial_out = torch.empty((self.num_splits, D // 8, 256, 4),
                                           dtype=torch.float32, device=device)
            self.partial_lse = torch.empty((self.num_splits, 2, 256), dtype=torch.float32,
                                           device=device)
            self.counters = torch.zeros(int(plan.num_counters), dtype=torch.int32, device=device)
        else:
            self.partial_out = self.partial_lse = self.counters = None
        self.c.partial_out = _ptr(self.partial_out)
        self.c.partial_lse = _ptr(self.partial_lse)
        self.c.counters = _ptr(self.counters)

    def tensors(self):
        """The device tensors of the workspace."""
        return [t for t in (self.partial_out, self.partial_lse, self.counters) if t is not None]

    @classmethod
    def for_args(cls, args: PaArgs, device, num_cus: int = 0) -> "PrefillWorkspace":
        return cls(pa_prefill_plan(args, num_cus=num_cus), args.head_dim, device)


def pa_prefill(args: PaArgs, workspace: Optional[PrefillWorkspace] = None, stream=None) -> None:
    """Prefill; with a workspace the bf16 kernel may split long key ranges
    (see pa_prefill_plan)."""
    ws = ctypes.byref(workspace.c) if workspace is not None else None
    _lib.check("pa_prefill", _lib.lib().pa_prefill(ctypes.byref(args), ws, _stream(stream)))


class AttentionPlan(NamedTuple):
    """pa_attention_plan's choice: the route (ROUTE_DECODE, ROUTE_PREFILL or
    ROUTE_RAGGED) and the plan of that route's path."""
    route: int
    plan: object  # DecodePlan, PrefillPlan or RaggedPlan


class RaggedPlan(NamedTuple):
    """Both parts of a ragged call: the decode part's piece slots and
    counters, the prefill part's key-split slots, and the bytes of
    partial_out plus partial_lse (see include/pa.h, PA_ROUTE_RAGGED)."""
    num_splits: int
    num_counters: int
    prefill_splits: int
    workspace_bytes: int


class RaggedWorkspace:
    """Device buffers of a ragged plan, laid out as include/pa.h describes
    for PA_ROUTE_RAGGED (torch owns the memory; counters zeroed once on
    torch's current stream)."""

    def __init__(self, plan: RaggedPlan, rows_per_block: int, D: int, device):
        S, Sp = int(plan.num_splits), int(plan.prefill_splits)
        lse_dec = -(-S * rows_per_block // 16) * 16
        self.partial_out = torch.empty(S * rows_per_block * D + Sp * D * 128, dtype=torch.float32,
                                       device=device)
        self.partial_lse = torch.empty(lse_dec + Sp * 512, dtype=torch.float32, device=device)
        self.counters = torch.zeros(int(plan.num_counters), dtype=torch.int32, device=device)
        self.c = PaWorkspace()
        self.c.partial_out = _ptr(self.partial_out)
        self.c.partial_lse = _ptr(self.partial_lse)
        self.c.counters = _ptr(self.counters)
        self.c.num_splits = S
        self.c.schedule = SCHEDULE_BALANCED
        self.c.num_counters = int(plan.num_counters)
        self.c.prefill_splits = Sp

    def tensors(self):
        return [self.partial_out, self.partial_lse, self.counters]


class PrefixGroups:
    """A pa_prefix_groups over device tensors group_start [G + 1] and
    prefix_lens [G] int32 (consecutive request ranges from request 0); it
    holds the tensors, so they live as long as the struct that points at
    them.  max_group_size defaults to the largest group, read from
    group_start (a device-to-host copy)."""

    def __init__(self, group_start: torch.Tensor, prefix_lens: torch.Tensor,
                 max_group_size: Optional[int] = None):
        _int32(group_start, "group_start")
        _int32(prefix_lens, "prefix_lens")
        _same_gpu(group_start, prefix_lens=prefix_lens)
        ng = prefix_lens.shape[0]
        _shape(group_start, (ng + 1,), "group_start")
        if max_group_size is None:
            max_group_size = (int((group_start[1:] - group_start[:-1]).max().item())
                              if ng else 1)
        self.group_start, self.prefix_lens = group_start, prefix_lens
        self.c = _lib.PaPrefixGroups()
        self.c.group_start = _ptr(group_start)
        self.c.prefix_lens = _ptr(prefix_lens) if ng else None
        self.c.num_groups = int(ng)
        self.c.max_group_size = int(max_group_size)


PREFIX_PIECES = 16  # prefix states per row of a shared-prefix call (include/pa.h)


class SharedPlan(NamedTuple):
    """pa_decode_shared_plan's choice: the decode part's piece slots, all
    arrival counters, the prefix launch's key-split slots and the bytes of
    partial_out plus partial_lse (layout in include/pa.h)."""
    num_splits: int
    num_counters: int
    prefill_splits: int
    workspace_bytes: int


def pa_decode_shared_plan(args: PaArgs, groups: PrefixGroups, *,
                          num_cus: int = 0) -> SharedPlan:
    ws = PaWorkspace()
    nbytes = ctypes.c_size_t(0)
    _lib.check("pa_decode_shared_plan", _lib.lib().pa_decode_shared_plan(
        ctypes.byref(args), ctypes.byref(groups.c), int(num_cus), ctypes.byref(ws),
        ctypes.byref(nbytes)))
    return SharedPlan(ws.num_splits, ws.num_counters, ws.prefill_splits, nbytes.value)


class SharedWorkspace:
    """Device buffers of a shared-prefix plan in the layout of include/pa.h
    (torch owns the memory; counters zeroed once on torch's current
    stream)."""

    def __init__(self, plan: SharedPlan, args: PaArgs, device):
        S, Sp, D = int(plan.num_splits), int(plan.prefill_splits), int(args.head_dim)
        R = _rows_per_block(min(8, (args.num_q_heads // args.num_kv_heads) * args.q_len))
        rows = args.batch * args.num_q_heads * args.q_len
        r16 = lambda x: -(-x // 16) * 16  # noqa: E731
        n = PREFIX_PIECES
        self.partial_out = torch.empty(S * R * D + rows * n * D, dtype=torch.float32,
                                       device=device)
        self.partial_lse = torch.empty(r16(S * R) + r16(rows * n) + r16(rows),
                                       dtype=torch.float32, device=device)
        if (self.partial_out.numel() + self.partial_lse.numel()) * 4 != plan.workspace_bytes:
            raise ValueError("workspace size disagrees with the library's plan")
        self.counters = torch.zeros(int(plan.num_counters), dtype=torch.int32, device=device)
        self.c = PaWorkspace()
        self.c.partial_out = _ptr(self.partial_out)
        self.c.partial_lse = _ptr(self.partial_lse)
        self.c.counters = _ptr(self.counters)
        self.c.num_splits = S
        self.c.schedule = SCHEDULE_BALANCED
        self.c.num_counters = int(plan.num_counters)
        self.c.prefill_splits = Sp

    def tensors(self):
        return [self.partial_out, self.partial_lse, self.counters]


def pa_decode_shared(args: PaArgs, groups: PrefixGroups, workspace: SharedWorkspace,
                     stream=None) -> None:
    """Decode with each group's shared prefix pages read once per group."""
    _lib.check("pa_decode_shared", _lib.lib().pa_decode_shared(
        ctypes.byref(args), ctypes.byref(groups.c), ctypes.byref(workspace.c),
        _stream(stream)))


def pa_attention_plan(args: PaArgs, *, num_cus: int = 0,
                      partition_tokens: int = 0) -> AttentionPlan:
    ws = PaWorkspace()
    ws.partition_tokens = int(partition_tokens)
    nbytes = ctypes.c_size_t(0)
    route = ctypes.c_int32(-1)
    _lib.check("pa_attention_plan", _lib.lib().pa_attention_plan(
        ctypes.byref(args), int(num_cus), ctypes.byref(ws), ctypes.byref(nbytes),
        ctypes.byref(route)))
    if route.value == _lib.ROUTE_DECODE:
        plan = DecodePlan(ws.num_splits, ws.partition_tokens, nbytes.value, ws.schedule,
                          ws.num_counters)
    elif route.value == _lib.ROUTE_RAGGED:
        plan = RaggedPlan(ws.num_splits, ws.num_counters, ws.prefill_splits, nbytes.value)
    else:
        plan = PrefillPlan(ws.num_splits, nbytes.value, ws.num_counters)
    return AttentionPlan(route.value, plan)


def _rows_per_block(G: int) -> int:
    for r in (1, 2, 4, 8):
        if G <= r:
            return r
    return 8


def attention_workspace(ap: AttentionPlan, args: PaArgs, query: torch.Tensor):
    """Device buffers for an AttentionPlan (decode: with arrival counters, so
    the merge runs inside pa_decode)."""
    if ap.route == _lib.ROUTE_DECODE:
        if query.dim() == 3:  # packed rows: states per row block, not per row
            return Workspace(args.batch, args.num_q_heads, 1, args.head_dim, ap.plan.num_splits,
                             ap.plan.partition_tokens, query.device, schedule=ap.plan.schedule,
                             block_rows=(ap.plan.workspace_bytes //
                                         max(1, ap.plan.num_splits * (args.head_dim + 1) * 4)),
                             num_counters=ap.plan.num_counters)
        return Workspace.for_plan(ap.plan, query, fused=True)
    if ap.route == _lib.ROUTE_RAGGED:
        G = args.num_q_heads // args.num_kv_heads
        return RaggedWorkspace(ap.plan, _rows_per_block(G), args.head_dim, query.device)
    return PrefillWorkspace(ap.plan, args.head_dim, query.device)


def pa_attention(args: PaArgs, workspace=None, stream=None) -> None:
    ws = ctypes.byref(workspace.c) if workspace is not None else None
    _lib.check("pa_attention", _lib.lib().pa_attention(ctypes.byref(args), ws, _stream(stream)))


def paged_attention(query: torch.Tensor, key_pages: torch.Tensor, value_pages: torch.Tensor,
                    block_table: torch.Tensor, context_lens: torch.Tensor, *,
                    scale: Optional[float] = None, mask: Optional[str] = "causal",
                    query_lens: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                    out: Optional[torch.Tensor] = None, stream=None,
                    k_scale: Optional[float] = None,
                    v_scale: Optional[float] = None,
                    query_start_loc: Optional[torch.Tensor] = None,
                    max_query_len: Optional[int] = None) -> torch.Tensor:
    """Convenience call through the library's router (pa_attention): the
    decode path when the query rows of one kv head fit a decode row block,
    the prefill path otherwise.  The workspace is allocated (and its
    counters zeroed) on torch's current stream; when `stream` is another
    stream it first waits for the current one, and the allocator keeps the
    workspace until the work queued on `stream` is done."""
    if out is None:
        out = torch.empty_like(query)
    args = make_args(query, key_pages, value_pages, block_table, context_lens, out, scale=scale,
                     mask=mask, query_lens=query_lens, k_scale=k_scale, v_scale=v_scale,
                     query_start_loc=query_start_loc, max_query_len=max_query_len)
    ap = pa_attention_plan(args, partition_tokens=partition_tokens)
    ws = attention_workspace(ap, args, query)
    if stream is not None:
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream))
        current = torch.cuda.current_stream()
        if stream != current:
            stream.wait_stream(current)
            for t in ws.tensors():
                t.record_stream(stream)
    pa_attention(args, ws, stream)
    return out


def pa_append(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
              key_pages: torch.Tensor, value_pages: torch.Tensor, stream=None,
              k_scale: Optional[float] = None, v_scale: Optional[float] = None) -> None:
    """K/V write path: the rows key[t], value[t] ([T, H_kv, D]) go to slot
    slot_mapping[t] (int32: page * page_size + offset; negative or past the
    pool: skipped) of key_pages / value_pages ([P, H_kv, page_size, D]).
    uint8 pages are an fp8 E4M3 pool: bf16 rows are quantised with k_scale /
    v_scale."""
    T, Hkv, D = key.shape
    P, Hkv2, ps, D2 = key_pages.shape
    if tuple(value.shape) != tuple(key.shape) or tuple(value_pages.shape) != tuple(key_pages.shape):
        raise ValueError("key / value or key_pages / value_pages shapes disagree")
    if Hkv2 != Hkv or D2 != D:
        raise ValueError("token rows and pages disagree in kv heads or head size")
    fp8 = key_pages.dtype == torch.uint8
    if key.dtype != value.dtype or key_pages.dtype != value_pages.dtype:
        raise ValueError("key / value or key_pages / value_pages dtypes disagree")
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("an fp8 (uint8) pool needs k_scale and v_scale")
    if not fp8 and key.dtype != key_pages.dtype:
        raise ValueError("tokens and pages must share one dtype (or the pages be fp8 codes)")
    _int32(slot_mapping, "slot_mapping")
    if tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    _same_gpu(key_pages, value_pages=value_pages, key=key, value=value, slot_mapping=slot_mapping)
    a = _lib.PaAppendArgs()
    a.key, a.value, a.slot_mapping = _ptr(key), _ptr(value), _ptr(slot_mapping)
    a.key_pages, a.value_pages = _ptr(key_pages), _ptr(value_pages)
    a.num_tokens, a.num_kv_heads, a.head_dim, a.num_pages, a.page_size = T, Hkv, D, P, ps
    a.dtype = _DTYPES.get(key.dtype, 99)
    a.cache_dtype = _lib.PA_KV_FP8_E4M3 if fp8 else _lib.PA_KV_SAME
    a.k_scale = float(k_scale) if fp8 else 1.0
    a.v_scale = float(v_scale) if fp8 else 1.0
    _lib.check("pa_append", _lib.lib().pa_append(ctypes.byref(a), _stream(stream)))
