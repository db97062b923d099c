"""GPU parity of the prefill path over fp8 (E4M3) K/V pages against the
oracle, through the C ABI.  The kv-cache dtype with per-tensor k/v scales
("Reading vLLM's PagedAttention Kernel", section 3.2) applies to every read
of the pages: pa_prefill (key split and unsplit; codes loaded into LDS
with one pool-wide buffer resource, per-row page offsets for page sizes
that are not a multiple of 16, or one resource per run for pools past
2 GiB, and widened at the operand reads; per-lane register staging for
pools past 2 GiB with such page sizes) and pa_attention's ragged route, whose
decode part and prefill part both read the codes.  The address trace of
the instrumented build is bit-exact; outputs are held to the bf16 bar, and
the LDS-load staging repeats bit for bit.  Marked gpu."""
import numpy as np
import pytest

import oracle
from tests._gpu import (DeviceInputs, assert_parity, dev, expected_visits, host_f64,
                        run_prefill)
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


def _fp8(seed, ctx, **kw):
    return make_random(seed, B=len(ctx), D=128, ctx=ctx, dtype="bf16", kv_dtype="fp8_e4m3",
                       extra_free_pages=5, **kw)


def _expect_trace_visits(x):
    tr = oracle.translate_of(x)
    v = expected_visits(x)
    for b in range(x.B):
        if x.rows_valid()[b] == 0:
            tr[b] = -1
            v[b] = 0
    return tr, v


CASES = [
    # seed, H_q, H_kv, L, ps, ctx, causal, query_lens, (k_scale, v_scale)
    (1, 8, 2, 100, 16, [100, 333], True, None, (0.37, 1.7)),
    (2, 32, 8, 256, 128, [300, 4096, 257], True, [256, 100, 1], (0.5, 0.25)),
    (3, 28, 4, 77, 5, [77, 200, 1000], True, None, (0.8, 0.6)),       # per-lane walk
    (4, 7, 1, 33, 1, [40, 33], True, None, (1.0, 1.0)),               # page size 1
    (5, 8, 8, 64, 48, [64, 600], False, None, (8.0, 0.3)),            # peaked scores
    (6, 16, 4, 200, 256, [200, 1500, 3001], True, [200, 150, 7], (0.3, 0.7)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_fp8_prefill_parity_and_trace(api, case):
    seed, Hq, Hkv, L, ps, ctx, causal, ql, scales = case
    print(f"[fp8 prefill] seed={seed} Hq={Hq} Hkv={Hkv} L={L} ps={ps} ctx={ctx} "
          f"causal={causal} qlens={ql} scales={scales}", flush=True)
    x = _fp8(seed, ctx, H_q=Hq, H_kv=Hkv, L=L, page_size=ps, causal=causal, query_lens=ql,
             kv_scales=scales)
    ref = oracle.attention_of(x)
    tr, v = _expect_trace_visits(x)
    for kw in (dict(), dict(num_cus=512), dict(split=False)):
        out, ex = run_prefill(api, DeviceInputs(x), **kw)
        assert_parity(out, ref, "bf16", f"fp8 prefill case{seed} {kw}")
        if "counters" in ex:
            assert not ex["counters"].any()
        if ql is not None:
            g = host_f64(out)
            for b, n in enumerate(ql):
                assert (g[b, :, n:] == 0).all()
        t_out, tex = run_prefill(api, DeviceInputs(x), trace=True, **kw)
        assert np.array_equal(tex["trace"], tr)
        assert np.array_equal(tex["visits"], v)
        assert_parity(t_out, ref, "bf16", f"fp8 prefill traced case{seed} {kw}")


@pytest.mark.parametrize("garbage", ["nan", "random"])
def test_fp8_prefill_stale_codes_bit_identical(api, garbage):
    """Codes past each request's context (NaN or random) change no output bit."""
    kw = dict(H_q=8, H_kv=2, L=100, page_size=16, causal=True)
    base, _ = run_prefill(api, DeviceInputs(_fp8(71, [100, 333], **kw)))
    o, _ = run_prefill(api, DeviceInputs(_fp8(71, [100, 333], garbage=garbage, **kw)))
    assert np.array_equal(host_f64(o), host_f64(base))


def test_fp8_prefill_pool_past_2gib(api):
    """fp8 pools of more than 2^31 bytes per K and V tensor: the runs stage
    through per-run buffer resources; the live pages sit at the top."""
    import torch
    x = _fp8(72, [40, 170, 333], H_q=8, H_kv=2, L=40, page_size=16, causal=True,
             kv_scales=(0.45, 1.3))
    page_bytes = x.H_kv * x.page_size * x.D
    n_big = (1 << 31) // page_bytes + 512
    assert n_big * page_bytes > (1 << 31)
    ids = np.arange(n_big - x.num_pages, n_big)
    kp = torch.full((n_big, x.H_kv, x.page_size, x.D), 0x7F, dtype=torch.uint8, device="cuda")
    vp = torch.full_like(kp, 0x7F)                       # NaN codes everywhere else
    idx = torch.from_numpy(ids).to("cuda")
    kp[idx] = dev(x.key_pages)
    vp[idx] = dev(x.value_pages)
    d = DeviceInputs(x, pages=(kp, vp))
    d.bt = dev(np.where(x.block_table >= 0, ids[np.maximum(x.block_table, 0)], -1).astype(np.int32))
    print(f"[fp8 bigpool] {n_big} pages x {page_bytes} B", flush=True)
    ref = oracle.attention_of(x)
    for split in (False, True):
        out, _ = run_prefill(api, d, split=split)
        assert_parity(out, ref, "bf16", f"fp8 prefill, pool past 2 GiB, split={split}")
    del kp, vp, d
    torch.cuda.empty_cache()


def _pack(x):
    lens = [int(n) for n in x.rows_valid()]
    rows = [x.query[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)]
    qsl = np.zeros(x.B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    return np.ascontiguousarray(np.concatenate(rows, axis=0)), qsl


RAGGED = [
    # seed, H_q, H_kv, L, ps, ctx, query_lens, scales
    (81, 32, 8, 40, 16, [40, 900, 1, 0, 77, 300], [40, 1, 1, 0, 2, 33], (0.5, 0.5)),
    (82, 16, 4, 300, 128, [300, 5000, 129, 2049], [300, 1, 129, 1], (0.37, 1.7)),
    (83, 8, 2, 20, 5, [20, 100, 1, 31], [20, 1, 1, 17], (1.0, 0.25)),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"seed{c[0]}" for c in RAGGED])
def test_fp8_ragged_one_call(api, case):
    """pa_attention over packed rows of fp8 pages: one-row requests through
    the decode kernel, the others through the prefill kernel, in one call;
    the instrumented kernels of the same call trace every key."""
    import torch
    seed, Hq, Hkv, L, ps, ctx, ql, scales = case
    print(f"[fp8 ragged] seed={seed} Hq={Hq} Hkv={Hkv} L={L} ps={ps} ctx={ctx} ql={ql}",
          flush=True)
    x = _fp8(seed, ctx, H_q=Hq, H_kv=Hkv, L=L, page_size=ps, causal=True, query_lens=ql,
             kv_scales=scales)
    q, qsl = _pack(x)
    ref = oracle.attention_of(x)
    qd = dev(q)
    kp, vp, bt, cl = dev(x.key_pages), dev(x.value_pages), dev(x.block_table), dev(x.context_lens)
    tr, v = _expect_trace_visits(x)
    for trace in (False, True):
        out = torch.full_like(qd, float("nan"))
        dbg_t = dbg_v = None
        if trace:
            cap = x.max_pages * x.page_size
            dbg_t = torch.full((x.B, cap, 2), -1, dtype=torch.int32, device="cuda")
            dbg_v = torch.zeros((x.B, x.H_kv, cap), dtype=torch.int32, device="cuda")
        args = api.make_args(qd, kp, vp, bt, cl, out, scale=x.scale, mask="causal",
                             query_start_loc=dev(qsl), max_query_len=x.L, debug_trace=dbg_t,
                             debug_visits=dbg_v, k_scale=x.k_scale, v_scale=x.v_scale)
        ap = api.pa_attention_plan(args)
        assert ap.route == api._lib.ROUTE_RAGGED
        ws = api.attention_workspace(ap, args, qd)
        api.pa_attention(args, ws)
        torch.cuda.synchronize()
        got = host_f64(out)
        full = np.zeros((x.B, x.H_q, x.L, x.D))
        for b in range(x.B):
            full[b, :, :qsl[b + 1] - qsl[b]] = got[qsl[b]:qsl[b + 1]].transpose(1, 0, 2)
        assert_parity(torch.from_numpy(full), ref, "bf16", f"fp8 ragged seed{seed} trace={trace}")
        assert not ws.counters.any().item()
        if trace:
            assert np.array_equal(dbg_t.cpu().numpy(), tr)
            assert np.array_equal(dbg_v.cpu().numpy(), v)


def test_fp8_c3_full_size(api):
    """The chunked prefill workload (4 requests x 512 rows after prefixes of
    up to 2048 keys, H_q 28, H_kv 4) over fp8 pages: whole output against the
    oracle in fp32 and fp64, split and unsplit, and the address trace."""
    from workloads import make_c3_fp8
    x = make_c3_fp8()
    print(f"[C3-fp8] seed={x.seed} ctx={x.context_lens.tolist()}", flush=True)
    ref = oracle.attention_of(x)
    ref64 = oracle.attention_of(x, precision="f64")
    tr, v = _expect_trace_visits(x)
    d = DeviceInputs(x)
    for kw in (dict(), dict(split=False)):
        out, ex = run_prefill(api, d, **kw)
        err = assert_parity(out, ref, "bf16", f"C3-fp8 {kw}")
        assert_parity(out, ref64, "bf16", f"C3-fp8 {kw} (fp64 oracle)")
        assert "counters" not in ex or not ex["counters"].any()
        print(f"[C3-fp8] {kw} max abs err {err:.3e}", flush=True)
        _, tex = run_prefill(api, d, trace=True, **kw)
        assert np.array_equal(tex["trace"], tr) and np.array_equal(tex["visits"], v)


def test_fp8_packed_rows_through_pa_prefill(api):
    """Packed query rows (query_start_loc) of fp8 pages through pa_prefill
    itself, with and without the key split."""
    import torch
    x = _fp8(91, [300, 45, 900, 130], H_q=16, H_kv=4, L=130, page_size=16, causal=True,
             query_lens=[130, 45, 2, 0], kv_scales=(0.6, 1.2))
    q, qsl = _pack(x)
    ref = oracle.attention_of(x)
    qd = dev(q)
    for split in (True, False):
        out = torch.full_like(qd, float("nan"))
        args = api.make_args(qd, dev(x.key_pages), dev(x.value_pages), dev(x.block_table),
                             dev(x.context_lens), out, scale=x.scale, mask="causal",
                             query_start_loc=dev(qsl), max_query_len=x.L, k_scale=x.k_scale,
                             v_scale=x.v_scale)
        ws = api.PrefillWorkspace.for_args(args, qd.device) if split else None
        api.pa_prefill(args, ws)
        torch.cuda.synchronize()
        got = host_f64(out)
        full = np.zeros((x.B, x.H_q, x.L, x.D))
        for b in range(x.B):
            full[b, :, :qsl[b + 1] - qsl[b]] = got[qsl[b]:qsl[b + 1]].transpose(1, 0, 2)
        assert_parity(torch.from_numpy(full), ref, "bf16", f"fp8 packed prefill split={split}")
        if ws is not None and ws.counters is not None:
            assert not ws.counters.any().item()


def test_fp8_checked_call_flags_out_of_pool_pages(api):
    """The contract check with fp8 pages: an out-of-pool entry is flagged
    (PA_DEBUG_BAD_PAGE, one count per call), the output stays untouched, and
    the same call on valid metadata gives the oracle's result with the
    error word zero."""
    import dataclasses
    import torch
    x = _fp8(92, [300, 41, 900], H_q=8, H_kv=2, L=40, page_size=16, causal=True,
             kv_scales=(0.5, 0.5))
    bt = x.block_table.copy()
    bt[2, 3] = x.num_pages
    bad = dataclasses.replace(x, block_table=bt)
    for inputs, want in ((bad, [1, 1]), (x, [0, 0])):
        err = torch.zeros(2, dtype=torch.int32, device="cuda")
        qd = dev(inputs.query)
        out = torch.full_like(qd, float("nan"))
        args = api.make_args(qd, dev(inputs.key_pages), dev(inputs.value_pages),
                             dev(inputs.block_table), dev(inputs.context_lens), out,
                             scale=inputs.scale, mask="causal", debug_errors=err,
                             k_scale=inputs.k_scale, v_scale=inputs.v_scale)
        ws = api.PrefillWorkspace.for_args(args, qd.device)
        api.pa_prefill(args, ws)
        torch.cuda.synchronize()
        assert err.cpu().tolist() == want
        if want[0]:
            assert torch.isnan(out).all()
        else:
            assert_parity(out, oracle.attention_of(x), "bf16", "fp8 checked prefill")
        if ws.counters is not None:
            assert not ws.counters.any().item()


@pytest.mark.parametrize("ps", [16, 5])
def test_fp8_lds_load_staging_repeats_bit_for_bit(api, ps):
    """The codes go straight into LDS (16-key runs in a page, or rows that
    resolve their own page): calls in a row (split or not) and the
    instrumented build give the same output bits."""
    import torch
    from workloads import make_c3_fp8
    x = make_c3_fp8() if ps == 16 else _fp8(93, [700, 200, 1500], H_q=28, H_kv=4, L=200,
                                            page_size=ps, causal=True, kv_scales=(0.5, 0.5))
    d = DeviceInputs(x)
    for kw in (dict(), dict(split=False)):
        outs = [run_prefill(api, d, **kw)[0] for _ in range(3)]
        outs.append(run_prefill(api, d, trace=True, **kw)[0])
        for o in outs[1:]:
            assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), kw
