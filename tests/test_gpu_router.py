"""GPU checks of the router (pa_attention): each route gives exactly what
its path gives when called directly, and matches the oracle.  Marked gpu:
needs an MI355X and libpa.so."""
import numpy as np
import pytest

import oracle
from tests._gpu import DeviceInputs, assert_parity, run_decode, run_prefill
from workloads import make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()  # fail loudly if the library is missing
    return a


def _routed(api, d, partition_tokens=0):
    import torch
    x = d.x
    print(f"[router] {x.name} B {x.B} H {x.H_q}/{x.H_kv} L {x.L} D {x.D} {x.dtype} "
          f"P_tok {partition_tokens}", flush=True)
    out = api.paged_attention(d.q, d.kp, d.vp, d.bt, d.cl, scale=x.scale, mask=d.mask,
                              query_lens=d.ql, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out


CASES = [
    # (H_q, H_kv, L, dtype, expected route)
    (32, 8, 1, "bf16", 0), (32, 8, 2, "bf16", 0), (32, 8, 4, "bf16", 1), (8, 8, 8, "f32", 0),
    (16, 4, 5, "f32", 1), (28, 4, 96, "bf16", 1),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_route_equals_direct_path_and_oracle(api, case):
    import torch
    Hq, Hkv, Lq, dtype, route = CASES[case]
    x = make_random(300 + case, B=5, H_q=Hq, H_kv=Hkv, L=Lq, D=128 if dtype == "bf16" else 64,
                    page_size=16, ctx=(Lq, 700), dtype=dtype, causal=True, name=f"router{case}")
    d = DeviceInputs(x)
    out = torch.empty_like(d.q)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask)
    assert api.pa_attention_plan(args).route == route
    got = _routed(api, d)
    direct = run_decode(api, d)[0] if route == 0 else run_prefill(api, d)[0]
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                       direct.view(torch.int16) if direct.dtype == torch.bfloat16 else direct)
    assert_parity(got, oracle.attention_of(x), dtype, f"router case {case}")


def test_decode_route_with_partitions_runs_the_merge(api):
    # an explicit partition size: no arrival counters, so pa_attention must
    # follow pa_decode with pa_split_reduce
    x = make_random(77, B=4, H_q=32, H_kv=8, L=1, D=128, page_size=16, ctx=(1500, 3000),
                    dtype="bf16", causal=True, name="router_partitions")
    d = DeviceInputs(x)
    got = _routed(api, d, partition_tokens=256)
    assert_parity(got, oracle.attention_of(x), "bf16", "router partitions")


@pytest.mark.parametrize("Lq", [1, 300])
def test_routed_call_on_a_side_stream(api, Lq):
    """paged_attention on a stream other than the current one: the call waits
    for the workspace set-up (zeroed arrival counters) made on the current
    stream and gives the current-stream result bit for bit, call after call."""
    import torch
    x = make_random(410 + Lq, B=4, H_q=32, H_kv=8, L=Lq, D=128, page_size=16, ctx=(Lq, 2500),
                    dtype="bf16", causal=True, name=f"side_stream{Lq}")
    d = DeviceInputs(x)
    base = api.paged_attention(d.q, d.kp, d.vp, d.bt, d.cl, scale=x.scale, mask=d.mask)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        got = api.paged_attention(d.q, d.kp, d.vp, d.bt, d.cl, scale=x.scale, mask=d.mask,
                                  stream=side)
        side.synchronize()
        assert torch.equal(got.view(torch.int16), base.view(torch.int16)), f"rep {rep}"
    assert_parity(base, oracle.attention_of(x), "bf16", f"side stream L={Lq}")
