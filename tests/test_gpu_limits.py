"""GPU parity at the size limits of the schedules: the balanced decode
schedule's batch limit (2048 requests, per-request tables in LDS) and the
prefill key split's (request, tile) pair limit (2048 pairs, planner tables
in LDS), each at the limit and one past it (where the plan falls back to
partitions, or the prefill runs unsplit).  Marked gpu: needs an MI355X."""
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


@pytest.mark.parametrize("B", [2048, 2049])
def test_decode_at_the_balanced_batch_limit(api, B):
    import torch
    x = make_random(900 + B, B=B, H_q=8, H_kv=2, L=1, D=128, page_size=16, ctx=(1, 70),
                    dtype="bf16", causal=True, extra_free_pages=8, name=f"decode_B{B}")
    d = DeviceInputs(x)
    out = torch.empty_like(d.q)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask)
    plan = api.pa_decode_plan(args)
    want = api.SCHEDULE_BALANCED if B <= 2048 else api.SCHEDULE_PARTITIONS
    print(f"[limits] decode B={B} schedule {plan.schedule} S={plan.num_splits}", flush=True)
    assert plan.schedule == want
    got, _ = run_decode(api, d)
    assert_parity(got, oracle.attention_of(x), "bf16", f"decode B={B}")


@pytest.mark.parametrize("B", [2048, 2049])
def test_prefill_at_the_split_pair_limit(api, B):
    import torch
    # G * L = 64 rows: one row tile per request, so B (request, tile) pairs
    x = make_random(950 + B, B=B, H_q=8, H_kv=2, L=16, D=128, page_size=16, ctx=(16, 200),
                    dtype="bf16", causal=True, extra_free_pages=8, name=f"prefill_B{B}")
    d = DeviceInputs(x)
    out = torch.empty_like(d.q)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask)
    plan = api.pa_prefill_plan(args)
    print(f"[limits] prefill B={B} split slots {plan.num_splits}", flush=True)
    assert (plan.num_splits > 0) == (B <= 2048)
    got, ex = run_prefill(api, d)
    assert_parity(got, oracle.attention_of(x), "bf16", f"prefill B={B}")
    if "counters" in ex:
        assert not ex["counters"].any()
