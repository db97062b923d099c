"""The decode (with its fused merge) and the key-split prefill captured in a
HIP graph: the library issues kernel launches only (no memsets, no
allocation, no synchronisation), and every kernel leaves its arrival
counters at zero, so a captured call replays correctly.  Each replay, with
eager work and synchronisations between replays, must equal the eager
result bit for bit."""
import numpy as np
import pytest

import oracle
from tests._gpu import DeviceInputs, assert_parity
from workloads import make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_decode_and_prefill_replay_in_a_graph(api):
    import torch
    xd = make_random(501, B=16, H_q=32, H_kv=8, L=1, D=128, page_size=16, ctx=(64, 3000),
                     dtype="bf16", causal=True, name="graph_decode")
    xp = make_random(502, B=3, H_q=28, H_kv=4, L=300, D=128, page_size=16, ctx=[3000, 300, 1200],
                     dtype="bf16", causal=True, name="graph_prefill")
    dd, dp = DeviceInputs(xd), DeviceInputs(xp)
    out_d, out_p = torch.empty_like(dd.q), torch.empty_like(dp.q)
    args_d = api.make_args(dd.q, dd.kp, dd.vp, dd.bt, dd.cl, out_d, scale=xd.scale, mask=dd.mask)
    args_p = api.make_args(dp.q, dp.kp, dp.vp, dp.bt, dp.cl, out_p, scale=xp.scale, mask=dp.mask)
    # plans and workspaces outside the capture (allocation and zeroing stay eager)
    ws_d = api.Workspace.for_plan(api.pa_decode_plan(args_d), dd.q, fused=True)
    ws_p = api.PrefillWorkspace.for_args(args_p, dp.q.device, num_cus=512)
    assert ws_d.counters is not None and ws_p.counters is not None

    def calls():
        api.pa_decode(args_d, ws_d)
        api.pa_split_reduce(args_d, ws_d)  # returns at once: the merge ran inside pa_decode
        api.pa_prefill(args_p, ws_p)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # eager reference, on the stream the capture will also use
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_d, ref_p = out_d.clone(), out_p.clone()
    assert_parity(ref_d, oracle.attention_of(xd), "bf16", "graph decode (eager)")
    assert_parity(ref_p, oracle.attention_of(xp), "bf16", "graph prefill (eager)")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        out_d.fill_(float("nan"))  # eager work between replays
        out_p.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        assert torch.equal(_bits(out_d), _bits(ref_d)), f"decode replay {rep}"
        assert torch.equal(_bits(out_p), _bits(ref_p)), f"prefill replay {rep}"
        assert not ws_d.counters.any().item() and not ws_p.counters.any().item()
    del g


def test_ragged_shared_and_checked_calls_replay_in_a_graph(api):
    """The ragged one call (two kernels), the shared-prefix decode (two
    kernels) and a decode call with the contract check (a check kernel before
    the decode) captured together; every replay equals the eager result."""
    import torch
    from tests._gpu import dev
    from workloads import make_shared
    xr = make_random(503, B=6, H_q=8, H_kv=2, L=24, D=128, page_size=16,
                     ctx=[500, 64, 210, 30, 1200, 90], dtype="bf16", causal=True,
                     query_lens=[1, 24, 1, 7, 1, 3], extra_free_pages=4)
    lens = [int(v) for v in xr.rows_valid()]
    rows = [xr.query[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)]
    qsl = np.zeros(xr.B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    qr = dev(np.ascontiguousarray(np.concatenate(rows, axis=0)))
    out_r = torch.empty_like(qr)
    args_r = api.make_args(qr, dev(xr.key_pages), dev(xr.value_pages), dev(xr.block_table),
                           dev(xr.context_lens), out_r, scale=xr.scale, mask="causal",
                           query_start_loc=dev(qsl), max_query_len=xr.L)
    ws_r = api.attention_workspace(api.pa_attention_plan(args_r), args_r, qr)

    xs, gs = make_shared(504, H_q=8, H_kv=2, L=1, D=128, page_size=16, group_sizes=[4, 2, 1],
                         prefix_pages=[6, 3, 0], suffix=(1, 120))
    ds = DeviceInputs(xs)
    out_s = torch.empty_like(ds.q)
    args_s = api.make_args(ds.q, ds.kp, ds.vp, ds.bt, ds.cl, out_s, scale=xs.scale, mask=ds.mask)
    groups = api.PrefixGroups(dev(gs.group_start), dev(gs.prefix_lens), gs.max_group_size)
    ws_s = api.SharedWorkspace(api.pa_decode_shared_plan(args_s, groups), args_s, ds.q.device)

    xc = make_random(505, B=8, H_q=32, H_kv=8, L=1, D=128, page_size=16, ctx=(16, 2000),
                     dtype="bf16", causal=True)
    dc = DeviceInputs(xc)
    out_c = torch.empty_like(dc.q)
    err = torch.zeros(2, dtype=torch.int32, device=dc.q.device)
    args_c = api.make_args(dc.q, dc.kp, dc.vp, dc.bt, dc.cl, out_c, scale=xc.scale, mask=dc.mask,
                           debug_errors=err)
    ws_c = api.Workspace.for_plan(api.pa_decode_plan(args_c), dc.q, fused=True)

    def calls():
        api.pa_attention(args_r, ws_r)
        api.pa_decode_shared(args_s, groups, ws_s)
        api.pa_decode(args_c, ws_c)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    refs = [out_r.clone(), out_s.clone(), out_c.clone()]
    assert_parity(refs[1], oracle.attention_of(xs), "bf16", "graph shared (eager)")
    assert_parity(refs[2], oracle.attention_of(xc), "bf16", "graph checked decode (eager)")
    assert err.tolist() == [0, 0]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in (out_r, out_s, out_c):
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] ragged/shared/checked replay {rep}", flush=True)
        for name, o, r in zip(("ragged", "shared", "checked"), (out_r, out_s, out_c), refs):
            assert torch.equal(_bits(o), _bits(r)), f"{name} replay {rep}"
        for w in (ws_r, ws_s, ws_c):
            assert not w.counters.any().item()
        assert err.tolist() == [0, 0]
    del g


def test_fp8_calls_replay_in_a_graph(api):
    """fp8 pages: the key-split prefill (LDS-load staging, 16- and 8-key
    pages), the ragged one call and the shared-prefix decode captured
    together; every replay equals the eager result bit for bit."""
    import torch
    from tests._gpu import dev, kv_scales
    from workloads import make_shared
    F = dict(dtype="bf16", kv_dtype="fp8_e4m3", kv_scales=(0.45, 1.3))
    xs16 = make_random(511, B=3, H_q=28, H_kv=4, L=200, D=128, page_size=16,
                       ctx=[2000, 200, 900], causal=True, **F)
    xs8 = make_random(512, B=3, H_q=28, H_kv=4, L=200, D=128, page_size=8,
                      ctx=[1500, 300, 700], causal=True, **F)
    pre = []
    for x in (xs16, xs8):
        d = DeviceInputs(x)
        out = torch.empty_like(d.q)
        args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                             **kv_scales(x))
        pre.append((x, out, args, api.PrefillWorkspace.for_args(args, d.q.device, num_cus=512), d))

    xr = make_random(513, B=5, H_q=8, H_kv=2, L=24, D=128, page_size=16,
                     ctx=[500, 64, 210, 30, 1200], causal=True, query_lens=[1, 24, 1, 7, 2], **F)
    lens = [int(v) for v in xr.rows_valid()]
    rows = [xr.query[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)]
    qsl = np.zeros(xr.B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    qr = dev(np.ascontiguousarray(np.concatenate(rows, axis=0)))
    out_r = torch.empty_like(qr)
    args_r = api.make_args(qr, dev(xr.key_pages), dev(xr.value_pages), dev(xr.block_table),
                           dev(xr.context_lens), out_r, scale=xr.scale, mask="causal",
                           query_start_loc=dev(qsl), max_query_len=xr.L, **kv_scales(xr))
    ws_r = api.attention_workspace(api.pa_attention_plan(args_r), args_r, qr)

    xs, gs = make_shared(514, H_q=8, H_kv=2, L=1, D=128, page_size=16, group_sizes=[4, 2, 1],
                         prefix_pages=[6, 3, 0], suffix=(1, 120), kv_dtype="fp8_e4m3",
                         kv_scales=(0.45, 1.3))
    ds = DeviceInputs(xs)
    out_s = torch.empty_like(ds.q)
    args_s = api.make_args(ds.q, ds.kp, ds.vp, ds.bt, ds.cl, out_s, scale=xs.scale, mask=ds.mask,
                           **kv_scales(xs))
    groups = api.PrefixGroups(dev(gs.group_start), dev(gs.prefix_lens), gs.max_group_size)
    ws_s = api.SharedWorkspace(api.pa_decode_shared_plan(args_s, groups), args_s, ds.q.device)

    outs = [p[1] for p in pre] + [out_r, out_s]

    def calls():
        for _, _, args, ws, _ in pre:
            api.pa_prefill(args, ws)
        api.pa_attention(args_r, ws_r)
        api.pa_decode_shared(args_s, groups, ws_s)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    for (x, out, _, _, _), ref in zip(pre, refs):
        assert_parity(ref, oracle.attention_of(x), "bf16", f"graph fp8 prefill ps {x.page_size}")
    assert_parity(refs[3], oracle.attention_of(xs), "bf16", "graph fp8 shared (eager)")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph fp8] replay {rep}", flush=True)
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(_bits(o), _bits(ref)), f"fp8 output {i}, replay {rep}"
        for ws in [p[3] for p in pre] + [ws_r, ws_s]:
            if getattr(ws, "counters", None) is not None:
                assert not ws.counters.any().item()
    del g
