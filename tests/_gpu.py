"""Helpers for GPU parity tests: move generated inputs to the device, run the
C-ABI entry points, compare with the oracle at the stated tolerances."""
import numpy as np
import torch

from workloads import bf16_bits_to_f32

# Parity bars (fp32 outputs: max-abs; bf16 outputs: max-abs and relative L2).
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def dev(a: np.ndarray, dtype: str = None, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


class DeviceInputs:
    """Device copies of a PagedInputs (torch owns the memory)."""

    def __init__(self, x, device="cuda", pages=None):
        self.x = x
        self.q = dev(x.query, device=device)
        if pages is None:
            self.kp = dev(x.key_pages, device=device)
            self.vp = dev(x.value_pages, device=device)
        else:
            self.kp, self.vp = pages
        self.bt = dev(x.block_table, device=device)
        self.cl = dev(x.context_lens, device=device)
        self.ql = None if x.query_lens is None else dev(x.query_lens, device=device)
        self.mask = "causal" if x.causal else "none"

    def out(self):
        return torch.full_like(self.q, float("nan"))


def kv_scales(x) -> dict:
    """make_args keywords for fp8 pages (empty otherwise)."""
    if getattr(x, "kv_dtype", None) == "fp8_e4m3":
        return dict(k_scale=x.k_scale, v_scale=x.v_scale)
    return {}


def run_decode(api, d: DeviceInputs, *, partition_tokens=0, trace=False, keep_ws=False,
               num_cus=0, fused=True):
    """pa_decode (+ pa_split_reduce) through the C ABI with the library's
    plan (partition_tokens > 0: the partition schedule with that size; else
    the balanced schedule, sized for `num_cus`).  Returns (out, extras)."""
    out = d.out()
    x = d.x
    extras = {}
    dbg_t = dbg_v = None
    if trace:
        cap = x.max_pages * x.page_size
        dbg_t = torch.full((x.B, cap, 2), -1, dtype=torch.int32, device=d.q.device)
        dbg_v = torch.zeros((x.B, x.H_kv, cap), dtype=torch.int32, device=d.q.device)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                         query_lens=d.ql, debug_trace=dbg_t, debug_visits=dbg_v,
                         **kv_scales(x))
    plan = api.pa_decode_plan(args, partition_tokens=partition_tokens, num_cus=num_cus)
    S, P, nbytes = plan.num_splits, plan.partition_tokens, plan.workspace_bytes
    ws = api.Workspace.for_plan(plan, d.q, fused=fused)
    api.pa_decode(args, ws)
    if keep_ws and S > 1:
        torch.cuda.synchronize()
        extras["partial_out"] = ws.partial_out.clone()
        extras["partial_lse"] = ws.partial_lse.clone()
    if S > 1:
        api.pa_split_reduce(args, ws)
    torch.cuda.synchronize()
    extras.update(S=S, P=P, ws_bytes=nbytes, ws=ws, args=args, schedule=plan.schedule)
    if trace:
        extras["trace"] = dbg_t.cpu().numpy()
        extras["visits"] = dbg_v.cpu().numpy()
    return out, extras


def run_prefill(api, d: DeviceInputs, *, trace=False, split=True, num_cus=0):
    """pa_prefill on device inputs; `split` passes the key-split workspace
    of pa_prefill_plan (for `num_cus` compute units), whose counters must be
    zero again afterwards (returned in extras["counters"])."""
    out = d.out()
    x = d.x
    extras = {}
    dbg_t = dbg_v = None
    if trace:
        cap = x.max_pages * x.page_size
        dbg_t = torch.full((x.B, cap, 2), -1, dtype=torch.int32, device=d.q.device)
        dbg_v = torch.zeros((x.B, x.H_kv, cap), dtype=torch.int32, device=d.q.device)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                         query_lens=d.ql, debug_trace=dbg_t, debug_visits=dbg_v,
                         **kv_scales(x))
    ws = api.PrefillWorkspace.for_args(args, d.q.device, num_cus=num_cus) if split else None
    api.pa_prefill(args, ws)
    torch.cuda.synchronize()
    if ws is not None and ws.counters is not None:
        extras["counters"] = ws.counters.cpu().numpy()
    if trace:
        extras["trace"] = dbg_t.cpu().numpy()
        extras["visits"] = dbg_v.cpu().numpy()
    return out, extras


def assert_parity(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str = ""):
    g = host_f64(got)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: fp32 max abs {err.max():.3e}"
    else:
        rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err.max() <= BF16_MAX_ABS, f"{what}: bf16 max abs {err.max():.3e}"
        assert rel <= BF16_REL_L2, f"{what}: bf16 rel L2 {rel:.3e}"
    return float(err.max())


def expected_visits(x):
    cap = x.max_pages * x.page_size
    v = np.zeros((x.B, x.H_kv, cap), dtype=np.int32)
    for b in range(x.B):
        v[b, :, :int(x.context_lens[b])] = 1
    return v
