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
