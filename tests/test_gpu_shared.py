"""GPU parity of the shared-prefix decode (pa_decode_shared) against the
oracle, through the C ABI.  Requests of a group name the same physical pages
for their first keys ("Reading vLLM's PagedAttention Kernel", sections 1-2:
block sharing is what prefix caching builds on); the library reads those
pages once per group and merges each row's prefix state with the rest of its
keys.  Sharing never changes what is computed, so the oracle is the plain
paged attention of the same inputs.  Marked gpu."""
import numpy as np
import pytest

import oracle
from tests._gpu import DeviceInputs, assert_parity, dev, host_f64, kv_scales, run_decode
from workloads import c5_decode_grouped, make_c5, make_shared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def _run_shared(api, x, groups, *, q=None, qsl=None, calls=1, prefix_lens=None, num_cus=0):
    """pa_decode_shared on x (padded rows, or packed rows q / qsl); returns
    (output on the host as float64, counters after the calls)."""
    import torch
    d = DeviceInputs(x)
    qd = d.q if q is None else dev(q)
    out = torch.full_like(qd, float("nan"))
    kw = {}
    if qsl is not None:
        kw = dict(query_start_loc=dev(qsl), max_query_len=x.L)
    args = api.make_args(qd, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                         query_lens=d.ql if qsl is None else None, **kw, **kv_scales(x))
    pl = groups.prefix_lens if prefix_lens is None else prefix_lens
    gs_d, pl_d = dev(groups.group_start), dev(np.asarray(pl, dtype=np.int32))
    g = api.PrefixGroups(gs_d, pl_d, groups.max_group_size)
    plan = api.pa_decode_shared_plan(args, g, num_cus=num_cus)
    ws = api.SharedWorkspace(plan, args, qd.device)
    for _ in range(calls):
        out.fill_(float("nan"))
        api.pa_decode_shared(args, g, ws)
    torch.cuda.synchronize()
    return out, ws.counters.cpu().numpy()


def _check(api, x, groups, what, **kw):
    out, counters = _run_shared(api, x, groups, **kw)
    ref = oracle.attention_of(x)
    if kw.get("qsl") is not None:
        return out, counters, ref
    err = assert_parity(out, ref, x.dtype, what)
    assert not counters.any(), f"{what}: arrival counters not left at zero"
    return out, err, ref


CASES = [
    # (name, H_q, H_kv, L, D, ps, group_sizes, prefix_pages, suffix, query_lens)
    ("g4-ps16", 8, 2, 1, 128, 16, [3, 1, 2, 5], [4, 0, 1, 7], (1, 70), None),
    ("mha-ps128", 4, 4, 1, 128, 128, [4, 2], [2, 1], (1, 300), None),
    ("g8-d64", 16, 2, 1, 64, 16, [6, 1, 1], [3, 2, 0], (1, 50), None),
    ("l4-g2", 8, 4, 4, 128, 32, [3, 3], [2, 3], (4, 90), [4, 1, 3, 2, 4, 0]),
    ("l2-g4-qlens", 8, 2, 2, 128, 16, [2, 3, 1], [5, 2, 3], (2, 40), [2, 1, 2, 0, 1, 2]),
    ("ps8-lanes", 8, 2, 1, 128, 8, [4, 2], [3, 5], (1, 33), None),
    ("one-group", 32, 8, 1, 128, 16, [9], [40], (1, 400), None),
    ("long-prefix", 8, 2, 1, 128, 16, [5, 2], [256, 64], (1, 20), None),
]


@pytest.mark.parametrize("seed,case", list(enumerate(CASES, start=100)),
                         ids=[c[0] for c in CASES])
def test_shared_matches_oracle(api, seed, case):
    name, H_q, H_kv, L, D, ps, sizes, pages, suffix, qlens = case
    x, groups = make_shared(seed, H_q=H_q, H_kv=H_kv, L=L, D=D, page_size=ps,
                            group_sizes=sizes, prefix_pages=pages, suffix=suffix,
                            query_lens=qlens)
    print(f"shared case {name}: B={x.B} groups={groups.num_groups}", flush=True)
    _check(api, x, groups, name)


FP8_CASES = [c for c in CASES if c[4] == 128]  # fp8 pages: head_dim 128


@pytest.mark.parametrize("seed,case", list(enumerate(FP8_CASES, start=200)),
                         ids=[c[0] for c in FP8_CASES])
def test_shared_fp8_pages_match_oracle(api, seed, case):
    """fp8 (E4M3) pages with per-tensor scales: the prefix launch (the
    prefill kernel's fp8 build) and the decode launch both read the codes;
    their row states carry v_scale alike, so the merge is unchanged."""
    name, H_q, H_kv, L, D, ps, sizes, pages, suffix, qlens = case
    x, groups = make_shared(seed, H_q=H_q, H_kv=H_kv, L=L, D=D, page_size=ps,
                            group_sizes=sizes, prefix_pages=pages, suffix=suffix,
                            query_lens=qlens, kv_dtype="fp8_e4m3", kv_scales=(0.37, 1.7))
    print(f"shared fp8 case {name}: B={x.B} groups={groups.num_groups}", flush=True)
    _check(api, x, groups, f"fp8 {name}")


def test_shared_fp8_partial_page_prefix_and_unshared_agree(api):
    """fp8 pages, a prefix that ends inside a page, and the same inputs
    through pa_decode: both within the bar of the oracle, and of each other."""
    x, groups = make_shared(19, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[3, 2, 4], prefix_pages=[4, 2, 9], suffix=(9, 150),
                            kv_dtype="fp8_e4m3", kv_scales=(0.6, 0.45))
    pl = groups.prefix_lens + np.asarray([7, 15, 3], dtype=np.int32)
    out_s, _, ref = _check(api, x, groups, "fp8 partial page", prefix_lens=pl)
    out_u, _ = run_decode(api, DeviceInputs(x))
    assert_parity(out_u, ref, "bf16", "fp8 unshared")
    assert np.abs(host_f64(out_s) - host_f64(out_u)).max() <= 1.6e-2


def test_shared_equals_unshared_decode(api):
    """The same inputs through pa_decode (every request walks its prefix)
    agree with the shared path to bf16 rounding of the final output."""
    x, groups = make_shared(11, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[4, 3, 1], prefix_pages=[8, 3, 2], suffix=(1, 200))
    out_s, _ = _run_shared(api, x, groups)
    out_u, _ = run_decode(api, DeviceInputs(x))
    d = np.abs(host_f64(out_s) - host_f64(out_u))
    assert d.max() <= 1.6e-2, d.max()


def test_shared_prefix_read_through_first_member_only(api):
    """The prefix pages are read once per group, through the first member's
    table: with every other member's prefix entries pointed at a free page
    of garbage, the shared path still gives the attention of the intact
    inputs (a path that walked those entries would read the garbage)."""
    x, groups = make_shared(18, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[4, 3, 2], prefix_pages=[6, 3, 2], suffix=(1, 80),
                            extra_free_pages=2)
    ref = oracle.attention_of(x)
    used = set(x.block_table[x.block_table >= 0].tolist())
    free = [p for p in range(x.num_pages) if p not in used]
    assert free
    bt = x.block_table.copy()
    for k in range(groups.num_groups):
        s, e = int(groups.group_start[k]), int(groups.group_start[k + 1])
        P = int(groups.prefix_lens[k]) // x.page_size
        bt[s + 1:e, :P] = free[0]
    import dataclasses
    bad = dataclasses.replace(x, block_table=bt)
    out, counters = _run_shared(api, bad, groups)
    assert_parity(out, ref, "bf16", "first member's prefix only")
    assert not counters.any()


def test_shared_repeated_calls(api):
    """Calls in a row reuse one workspace (counters left zero each time) and
    give identical outputs."""
    import torch
    x, groups = make_shared(12, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[5, 2, 6], prefix_pages=[6, 2, 9], suffix=(1, 300))
    out1, c1 = _run_shared(api, x, groups, calls=1)
    out3, c3 = _run_shared(api, x, groups, calls=3)
    assert not c1.any() and not c3.any()
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    assert_parity(out3, oracle.attention_of(x), "bf16", "repeated")


def test_shared_partial_page_prefix(api):
    """A prefix length that ends inside a page shares only its whole pages
    (the rest is walked per request): the result is unchanged."""
    x, groups = make_shared(13, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[3, 2], prefix_pages=[4, 2], suffix=(9, 60))
    pl = groups.prefix_lens + np.asarray([7, 15], dtype=np.int32)  # into the members' own pages
    _check(api, x, groups, "partial page", prefix_lens=pl)


def test_shared_all_singletons_no_prefix(api):
    """Every request a group of its own with prefix 0: plain decode."""
    x, groups = make_shared(14, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[1] * 7, prefix_pages=[0] * 7, suffix=(1, 500))
    _check(api, x, groups, "singletons")


def test_shared_groups_then_unshared_requests(api):
    """Groups at the front, then requests in no group (group_start ends
    before the batch does), and the same batch with no groups at all."""
    x, groups = make_shared(17, H_q=8, H_kv=2, L=1, D=128, page_size=16,
                            group_sizes=[3, 2, 1, 1, 1], prefix_pages=[5, 2, 0, 0, 0],
                            suffix=(1, 90))
    from workloads import SharedGroups
    front = SharedGroups(groups.group_start[:3].copy(), groups.prefix_lens[:2].copy())
    assert front.group_start[-1] == 5 < x.B
    _check(api, x, front, "front groups")
    none = SharedGroups(np.zeros(1, dtype=np.int32), np.zeros(0, dtype=np.int32))
    _check(api, x, none, "no groups")


def test_shared_many_requests(api):
    """More than 256 requests: the group of each request comes from the scan
    over several requests per thread."""
    sizes = [7, 1, 40, 1, 1, 90, 3, 1, 120, 2, 1, 60]
    pages = [2, 0, 3, 1, 0, 1, 4, 0, 2, 1, 0, 5]
    x, groups = make_shared(15, H_q=8, H_kv=2, L=1, D=128, page_size=16, group_sizes=sizes,
                            prefix_pages=pages, suffix=(1, 40))
    assert x.B > 256
    _check(api, x, groups, "many requests")


def test_shared_packed_rows(api):
    """Packed query rows (query_start_loc) with a shared prefix."""
    x, groups = make_shared(16, H_q=8, H_kv=4, L=2, D=128, page_size=16,
                            group_sizes=[3, 1, 2], prefix_pages=[3, 1, 2], suffix=(2, 60),
                            query_lens=[2, 1, 2, 1, 0, 2])
    lens = [int(v) for v in x.rows_valid()]
    rows = [x.query[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)]
    qsl = np.zeros(x.B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    q = np.ascontiguousarray(np.concatenate(rows, axis=0))
    out, counters, ref = _check(api, x, groups, "packed", q=q, qsl=qsl)
    assert not counters.any()
    got = host_f64(out)
    full = np.zeros((x.B, x.H_q, x.L, x.D))
    for b in range(x.B):
        full[b, :, :lens[b]] = got[qsl[b]:qsl[b + 1]].transpose(1, 0, 2)
    import torch
    assert_parity(torch.from_numpy(full), ref, "bf16", "packed")


def test_shared_c5_decode(api):
    """The decode part of the mixed workload (48 requests, 11 of them sharing
    a 2048-key prefix of 16 pages of 128 keys) with the sharers as one group:
    whole output against the oracle."""
    m = make_c5()
    x, groups, _ = c5_decode_grouped(m)
    assert list(groups.group_start) == [0, 11] and list(groups.prefix_lens) == [2048]
    _check(api, x, groups, "C5 decode shared")
