"""GPU tests of the contract check (pa_args.debug_errors): the kernels take
block tables, context lengths and query rows on trust (tiny-llm "Week 3 Day
4: Direct Paged Attention", "What Must Hold, and What Breaks If It Doesn't":
a page id outside the pool reads memory that is not the request's).  With
the check on, a call first checks its metadata on the device; a violation
sets flags in the error word and every kernel of the call returns before
reading K/V, so these tests hand broken metadata only to checked calls.
Marked gpu."""
import dataclasses

import numpy as np
import pytest

import oracle
from tests._gpu import assert_parity, dev, host_f64
from workloads import make_random, make_shared

pytestmark = pytest.mark.gpu

BAD_PAGE, BAD_CONTEXT, BAD_ROWS, BAD_GROUPS = 1, 2, 4, 8


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def _pack(x):
    lens = [int(v) for v in x.rows_valid()]
    rows = [x.query[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)]
    qsl = np.zeros(x.B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    return np.ascontiguousarray(np.concatenate(rows, axis=0)), qsl


def _call(api, x, entry, checked=True, groups=None, calls=1):
    """One call of `entry` on inputs x; returns (out, errors or None,
    counters or None).  entry: decode (balanced, fused merge), partitions
    (pa_decode + pa_split_reduce), noalloc, prefill (key split), ragged
    (pa_attention over packed rows), shared (pa_decode_shared)."""
    import torch
    err = torch.zeros(2, dtype=torch.int32, device="cuda") if checked else None
    kp, vp, bt, cl = dev(x.key_pages), dev(x.value_pages), dev(x.block_table), dev(x.context_lens)
    mask = "causal" if x.causal else "none"
    counters = None
    if entry == "ragged":
        q, qsl = _pack(x)
        qd = dev(q)
        out = torch.full_like(qd, float("nan"))
        args = api.make_args(qd, kp, vp, bt, cl, out, scale=x.scale, mask=mask,
                             query_start_loc=dev(qsl), max_query_len=x.L, debug_errors=err)
        ap = api.pa_attention_plan(args)
        ws = api.attention_workspace(ap, args, qd)
        for _ in range(calls):
            api.pa_attention(args, ws)
        counters = ws.counters
    else:
        qd = dev(x.query)
        out = torch.full_like(qd, float("nan"))
        ql = None if x.query_lens is None else dev(x.query_lens)
        args = api.make_args(qd, kp, vp, bt, cl, out, scale=x.scale, mask=mask, query_lens=ql,
                             debug_errors=err)
        if entry in ("decode", "partitions"):
            plan = api.pa_decode_plan(args, partition_tokens=32 if entry == "partitions" else 0)
            ws = api.Workspace.for_plan(plan, qd, fused=entry == "decode")
            for _ in range(calls):
                api.pa_decode(args, ws)
                if plan.num_splits > 1 and entry == "partitions":
                    api.pa_split_reduce(args, ws)
            counters = ws.counters
        elif entry == "noalloc":
            for _ in range(calls):
                api.pa_decode_noalloc(args)
        elif entry == "prefill":
            ws = api.PrefillWorkspace.for_args(args, qd.device)
            for _ in range(calls):
                api.pa_prefill(args, ws)
            counters = ws.counters
        elif entry == "shared":
            g = api.PrefixGroups(dev(groups.group_start), dev(groups.prefix_lens),
                                 groups.max_group_size)
            plan = api.pa_decode_shared_plan(args, g)
            ws = api.SharedWorkspace(plan, args, qd.device)
            for _ in range(calls):
                api.pa_decode_shared(args, g, ws)
            counters = ws.counters
        else:
            raise ValueError(entry)
    torch.cuda.synchronize()
    return (out, None if err is None else err.cpu().numpy(),
            None if counters is None else counters.cpu().numpy())


def _decode_inputs(seed=5):
    return make_random(seed, B=6, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                       ctx=[700, 33, 1, 260, 1500, 96], dtype="bf16", causal=True,
                       extra_free_pages=4)


def _prefill_inputs(seed=6):
    return make_random(seed, B=3, H_q=8, H_kv=2, L=40, D=128, page_size=16,
                       ctx=[300, 41, 900], dtype="bf16", causal=True, extra_free_pages=4)


def _ragged_inputs(seed=7):
    return make_random(seed, B=5, H_q=8, H_kv=2, L=24, D=128, page_size=16,
                       ctx=[500, 64, 210, 30, 1200], dtype="bf16", causal=True,
                       query_lens=[1, 24, 1, 7, 1], extra_free_pages=4)


def _shared_inputs(seed=8):
    return make_shared(seed, H_q=8, H_kv=2, L=1, D=128, page_size=16, group_sizes=[3, 2, 1],
                       prefix_pages=[6, 2, 0], suffix=(1, 90))


def _inputs(entry):
    if entry == "prefill":
        return _prefill_inputs(), None
    if entry == "ragged":
        return _ragged_inputs(), None
    if entry == "shared":
        return _shared_inputs()
    return _decode_inputs(), None


ENTRIES = ["decode", "partitions", "noalloc", "prefill", "ragged", "shared"]


@pytest.mark.parametrize("entry", ENTRIES)
def test_checked_call_of_valid_inputs_changes_nothing(api, entry):
    """Valid metadata: the error word stays zero and the output is bit for
    bit that of the unchecked call."""
    import torch
    x, groups = _inputs(entry)
    print(f"contract check, valid inputs: {entry}", flush=True)
    a, err, _ = _call(api, x, entry, checked=True, groups=groups)
    b, _, _ = _call(api, x, entry, checked=False, groups=groups)
    assert err.tolist() == [0, 0]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _out_of_pool(x):
    """Two entries the kernels would read point outside the pool; one
    padding entry past a context (never read) holds a huge id too."""
    bt = x.block_table.copy()
    ps = x.page_size
    b_long = int(np.argmax(x.context_lens))
    n = (int(x.context_lens[b_long]) + ps - 1) // ps
    bt[b_long, n - 1] = x.num_pages          # one past the pool
    bt[b_long, 0] = -3
    b_short = int(np.argmin(x.context_lens))
    m = (int(x.context_lens[b_short]) + ps - 1) // ps
    if m < x.max_pages:
        bt[b_short, m] = 1 << 30             # past the context: not read, not flagged
    return dataclasses.replace(x, block_table=bt)


@pytest.mark.parametrize("entry", ENTRIES)
def test_out_of_pool_pages_are_flagged_and_nothing_runs(api, entry):
    """Out-of-pool block-table entries: flag PA_DEBUG_BAD_PAGE and their
    count (two calls: twice the entries), the output untouched and the
    arrival counters still zero; then the valid inputs give the oracle's
    result."""
    x, groups = _inputs(entry)
    if entry == "shared":
        # break the pages of a request in no shared range (group 2, no prefix)
        bt = x.block_table.copy()
        b = int(groups.group_start[2])
        bt[b, 0] = x.num_pages
        bt[b, (int(x.context_lens[b]) - 1) // x.page_size] = -3
        bad = dataclasses.replace(x, block_table=bt)
    else:
        bad = _out_of_pool(x)
    n_bad = 0
    for b in range(x.B):
        n = (int(x.context_lens[b]) + x.page_size - 1) // x.page_size
        e = bad.block_table[b, :n]
        n_bad += int(((e < 0) | (e >= x.num_pages)).sum())
    assert n_bad in (1, 2)
    print(f"contract check, out-of-pool pages: {entry}", flush=True)
    out, err, counters = _call(api, bad, entry, groups=groups, calls=2)
    assert err[0] == BAD_PAGE and err[1] == 2 * n_bad, err
    assert np.isnan(host_f64(out)).all()
    if counters is not None:
        assert not counters.any()
    good, err2, counters2 = _call(api, x, entry, groups=groups)
    assert err2.tolist() == [0, 0]
    if entry != "ragged":
        assert_parity(good, oracle.attention_of(x), "bf16", f"{entry} after a refused call")
    if counters2 is not None:
        assert not counters2.any()


def test_context_and_row_violations_are_flagged(api):
    import torch
    x = _decode_inputs()
    cap = x.max_pages * x.page_size
    cl = x.context_lens.copy()
    cl[1] = cap + 5                    # its padding entries (-1) now count as read too
    out, err, _ = _call(api, dataclasses.replace(x, context_lens=cl), "decode")
    assert err[0] & BAD_CONTEXT and np.isnan(host_f64(out)).all()
    cl[1] = -2
    out, err, _ = _call(api, dataclasses.replace(x, context_lens=cl), "decode")
    assert err.tolist() == [BAD_CONTEXT, 0] and np.isnan(host_f64(out)).all()
    p = _prefill_inputs()
    ql = np.full(p.B, p.L, dtype=np.int32)
    ql[2] = p.L + 1
    out, err, _ = _call(api, dataclasses.replace(p, query_lens=ql), "prefill")
    assert err.tolist() == [BAD_ROWS, 0] and np.isnan(host_f64(out)).all()
    cl = p.context_lens.copy()
    cl[1] = p.L - 3                    # causal: fewer keys than rows
    out, err, _ = _call(api, dataclasses.replace(p, context_lens=cl), "prefill")
    assert err.tolist() == [BAD_ROWS, 0] and np.isnan(host_f64(out)).all()
    cl[1] = 0                          # an empty context is the zero-output case
    out, err, _ = _call(api, dataclasses.replace(p, context_lens=cl), "prefill")
    assert err.tolist() == [0, 0] and torch.isfinite(out).all()


def test_group_violations_are_flagged(api):
    x, groups = _shared_inputs()
    s1 = int(groups.group_start[1])
    bt = x.block_table.copy()
    bt[s1 + 1, 1] = bt[s1 + 1, 0]      # a member's shared page differs from the first member's
    out, err, _ = _call(api, dataclasses.replace(x, block_table=bt), "shared", groups=groups)
    assert err.tolist() == [BAD_GROUPS, 0] and np.isnan(host_f64(out)).all()
    pl = groups.prefix_lens.copy()
    pl[0] = int(x.context_lens[groups.group_start[0]:groups.group_start[1]].min()) // 16 * 16 + 16
    from workloads import SharedGroups
    g2 = SharedGroups(groups.group_start.copy(), pl)
    out, err, _ = _call(api, x, "shared", groups=g2)
    assert err[0] & BAD_GROUPS and np.isnan(host_f64(out)).all()
    gs = groups.group_start.copy()
    gs[1], gs[2] = gs[2], gs[1]        # decreasing starts
    g3 = SharedGroups(gs, groups.prefix_lens.copy())
    out, err, _ = _call(api, x, "shared", groups=g3)
    assert err[0] & BAD_GROUPS and np.isnan(host_f64(out)).all()
