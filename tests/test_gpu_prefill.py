"""GPU parity of the prefill path (pa_prefill) and of the mixed decode +
prefill batch against the oracle, through the C ABI."""
import dataclasses

import numpy as np
import pytest

import oracle
from tests._gpu import (DeviceInputs, assert_parity, expected_visits, host_f64, run_decode,
                        run_prefill)
from workloads import make_c3, make_c5, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def _expect_trace_visits(x):
    tr = oracle.translate_of(x)
    v = expected_visits(x)
    for b in range(x.B):
        if x.rows_valid()[b] == 0:
            tr[b] = -1
            v[b] = 0
    return tr, v


def _dma_staging(x):
    """Whether the bf16 prefill loads K/V tiles straight into LDS (pools
    under 2 GiB, any page size and head size): the staging of every
    benchmarked shape."""
    return x.dtype == "bf16"


def _traced_prefill_matches(api, d, x, out, **kw):
    """The instrumented build of the staging mode that produced `out` records
    the (page, slot) decoded from the address each key's load used and one
    visit per key under the kv head that address points at: both equal the
    oracle's translation exactly.  The LDS-load staging gives the same
    output bits traced and untraced (and call after call); the register
    staging (pools of 2 GiB and more with page sizes that are not a
    multiple of 8, none here) is not bitwise repeatable from call to call,
    and the fp32 path is held to the oracle as well."""
    t_out, tex = run_prefill(api, d, trace=True, **kw)
    tr, v = _expect_trace_visits(x)
    assert np.array_equal(tex["trace"], tr)
    assert np.array_equal(tex["visits"], v)
    if _dma_staging(x):
        assert np.array_equal(host_f64(t_out), host_f64(out)), "traced output differs"
    else:
        assert_parity(t_out, oracle.attention_of(x), x.dtype, "traced (per-lane staging)")


CASES = [
    # seed, dtype, D, H_q, H_kv, L, ps, ctx, causal, query_lens
    (1, "bf16", 128, 4, 4, 9, 16, [9, 100], True, None),
    (2, "bf16", 128, 28, 4, 77, 16, [77, 200, 1000], True, None),
    (3, "bf16", 64, 8, 2, 130, 4, [130, 131, 500], True, None),
    (4, "bf16", 128, 8, 8, 64, 128, [64, 600], False, None),
    (5, "bf16", 128, 7, 1, 33, 1, [40, 33], True, None),
    (6, "bf16", 128, 32, 8, 256, 128, [300, 4096, 257], True, [256, 100, 1]),
    (7, "bf16", 64, 3, 3, 50, 5, [50, 51, 120], True, [50, 0, 17]),
    (8, "f32", 128, 8, 2, 40, 16, [40, 300], True, None),
    (9, "f32", 64, 4, 4, 12, 3, [12, 13, 40], False, [12, 5, 0]),
    (10, "bf16", 128, 16, 2, 300, 24, [300, 1000], True, None),
    # page sizes that are multiples of 16: D 64 stages through registers,
    # D 128 loads straight into LDS (32-key tiles over 48- and 32-key pages)
    (11, "bf16", 64, 8, 2, 100, 16, [100, 700], True, None),
    (12, "bf16", 128, 16, 4, 200, 48, [200, 1500, 3001], True, [200, 150, 7]),
    (13, "bf16", 128, 12, 3, 65, 32, [65, 66, 2000], True, None),
    # 64- and 256-key pages: several 32-key tiles per page
    (14, "bf16", 128, 8, 2, 100, 64, [100, 1000], True, None),
    (15, "bf16", 128, 28, 4, 130, 256, [130, 300, 2600], True, [130, 64, 1]),
    (16, "bf16", 64, 8, 2, 70, 256, [70, 900], False, None),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_prefill_parity_random_shapes(api, case):
    seed, dt, D, Hq, Hkv, L, ps, ctx, causal, ql = case
    print(f"[prefill] seed={seed} dtype={dt} D={D} Hq={Hq} Hkv={Hkv} L={L} ps={ps} ctx={ctx} "
          f"causal={causal} qlens={ql}", flush=True)
    x = make_random(seed, B=len(ctx), H_q=Hq, H_kv=Hkv, L=L, D=D, page_size=ps, ctx=ctx,
                    dtype=dt, causal=causal, query_lens=ql, extra_free_pages=5)
    ref = oracle.attention_of(x)
    # the production kernels, with the key split (default plan, and one with
    # pieces as short as allowed) and without it; the arrival counters are
    # left at zero; each instrumented run traces the same staging mode
    for kw in (dict(), dict(num_cus=512), dict(split=False)):
        out, ex = run_prefill(api, DeviceInputs(x), **kw)
        assert_parity(out, ref, dt, f"prefill case{seed} {kw}")
        if "counters" in ex:
            assert not ex["counters"].any()
        if ql is not None:
            g = host_f64(out)
            for b, n in enumerate(ql):
                assert (g[b, :, n:] == 0).all()
        _traced_prefill_matches(api, DeviceInputs(x), x, out, **kw)


def test_prefill_stale_data_and_relabel_bit_identical(api):
    kw = dict(B=2, H_q=8, H_kv=2, L=100, D=128, page_size=16, ctx=[100, 333], dtype="bf16",
              causal=True, extra_free_pages=7)
    x = make_random(61, garbage=1e4, **kw)
    base, _ = run_prefill(api, DeviceInputs(x))
    y = make_random(61, garbage="nan", **kw)
    o, _ = run_prefill(api, DeviceInputs(y))
    assert np.array_equal(host_f64(o), host_f64(base))
    pi = np.random.default_rng(3).permutation(x.num_pages)
    kp2 = np.empty_like(x.key_pages)
    vp2 = np.empty_like(x.value_pages)
    kp2[pi], vp2[pi] = x.key_pages, x.value_pages
    z = dataclasses.replace(x, key_pages=kp2, value_pages=vp2,
                            block_table=np.where(x.block_table >= 0,
                                                 pi[np.maximum(x.block_table, 0)], -1).astype(np.int32))
    o, _ = run_prefill(api, DeviceInputs(z))
    assert np.array_equal(host_f64(o), host_f64(base))


def test_prefill_equals_decode_for_short_chunks(api):
    """The two schedules compute the same function: L <= 8 through both."""
    x = make_random(62, B=3, H_q=16, H_kv=4, L=6, D=128, page_size=16, ctx=[6, 50, 700],
                    dtype="bf16", causal=True)
    a, _ = run_prefill(api, DeviceInputs(x))
    b, _ = run_decode(api, DeviceInputs(x), partition_tokens=64)
    ref = oracle.attention_of(x)
    assert_parity(a, ref, "bf16", "prefill L=6")
    assert_parity(b, ref, "bf16", "decode L=6")


def test_c3_chunked_prefill_full_size(api):
    x = make_c3()
    print(f"[C3] seed={x.seed} ctx={x.context_lens.tolist()}", flush=True)
    ref = oracle.attention_of(x)
    ref64 = oracle.attention_of(x, precision="f64")
    d = DeviceInputs(x)
    for kw in (dict(), dict(split=False)):
        out, ex = run_prefill(api, d, **kw)
        err = assert_parity(out, ref, "bf16", f"C3 {kw}")
        assert_parity(out, ref64, "bf16", f"C3 {kw} (fp64 oracle)")
        assert "counters" not in ex or not ex["counters"].any()
        print(f"[C3] {kw} max abs err {err:.3e}", flush=True)
        _traced_prefill_matches(api, d, x, out, **kw)
        print(f"[C3] {kw} trace bit-exact", flush=True)


def test_key_split_matches_unsplit_and_repeats(api):
    """Pieces merged by the last one to arrive give the unsplit result to
    rounding, call after call on one workspace (the counters reset)."""
    import torch
    x = make_random(71, B=3, H_q=16, H_kv=2, L=200, D=128, page_size=16,
                    ctx=[3000, 200, 1500], dtype="bf16", causal=True)
    d = DeviceInputs(x)
    ref = oracle.attention_of(x)
    base, _ = run_prefill(api, d, split=False)
    out = d.out()
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask)
    plan = api.pa_prefill_plan(args, num_cus=512)
    ws = api.PrefillWorkspace(plan, x.D, d.q.device)
    for rep in range(3):
        out.zero_()
        api.pa_prefill(args, ws)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", f"split rep {rep}")
        assert not ws.counters.any().item()
        diff = np.abs(host_f64(out) - host_f64(base)).max()
        assert diff <= 2.0 ** -7, diff


def test_c5_mixed_batch_full_size(api):
    import torch
    m = make_c5()
    print(f"[C5] seed={m.seed} pool={m.decode.num_pages}", flush=True)
    dec = DeviceInputs(m.decode)
    pre = DeviceInputs(m.prefill, pages=(dec.kp, dec.vp))   # one pool, two calls
    out_d, ex = run_decode(api, dec)
    out_p, _ = run_prefill(api, pre)
    torch.cuda.synchronize()
    err_d = assert_parity(out_d, oracle.attention_of(m.decode), "bf16", "C5 decode")
    err_p = assert_parity(out_p, oracle.attention_of(m.prefill), "bf16", "C5 prefill")
    print(f"[C5] decode S={ex['S']} err {err_d:.3e}; prefill err {err_p:.3e}", flush=True)
    t_out, tex = run_decode(api, dec, trace=True)
    tr, v = _expect_trace_visits(m.decode)
    assert np.array_equal(tex["trace"], tr) and np.array_equal(tex["visits"], v)
    assert np.array_equal(host_f64(t_out), host_f64(out_d))
    _traced_prefill_matches(api, pre, m.prefill, out_p)
    print("[C5] traces bit-exact", flush=True)


def _plant_spike(x, b, j, coef):
    """Make logical key j of request b score far above every other key for
    the query rows of the kv head that share it: K[j] = coef * (sum of that
    group's last-row queries).  With coef 16 the row maxima sit about 2^200
    above the first key block's (base-2 units), past the fp32 range, so
    only an exact reference gives finite weights."""
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits
    G = x.H_q // x.H_kv
    ps = x.page_size
    page, slot = int(x.block_table[b, j // ps]), j % ps
    q = x.query if x.dtype == "f32" else bf16_bits_to_f32(x.query)
    for g in range(x.H_kv):
        lb = x.L - 1 if x.query_lens is None else int(x.query_lens[b]) - 1
        d = q[b, g * G:(g + 1) * G, lb, :].astype(np.float64).sum(axis=0)
        k = (coef * d).astype(np.float32)
        x.key_pages[page, g, slot, :] = k if x.dtype == "f32" else f32_to_bf16_bits(k)
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_late_score_spike_is_exact(api, dtype):
    """A key past the first block that scores more than 2^16 above the first
    block's maximum (in the base-2 units the kernel uses) must give the same
    result as any other input: the walk is redone from the exact maxima."""
    x = make_random(81, B=2, H_q=8, H_kv=2, L=130, D=128, page_size=16, ctx=[400, 200],
                    dtype=dtype, causal=True)
    x = _plant_spike(x, 0, 300, 16.0)
    x = _plant_spike(x, 1, 150, 16.0)
    ref = oracle.attention_of(x)
    for kw in (dict(), dict(num_cus=512), dict(split=False)):
        out, _ = run_prefill(api, DeviceInputs(x), **kw)
        assert_parity(out, ref, dtype, f"prefill spike {kw}")


def test_decode_late_score_spike_is_exact(api):
    x = make_random(82, B=3, H_q=16, H_kv=4, L=1, D=128, page_size=16, ctx=[900, 300, 2000],
                    dtype="bf16", causal=True)
    for b, j in ((0, 700), (1, 299), (2, 1999)):
        x = _plant_spike(x, b, j, 16.0)
    ref = oracle.attention_of(x)
    for kw in (dict(), dict(partition_tokens=64)):
        out, _ = run_decode(api, DeviceInputs(x), **kw)
        assert_parity(out, ref, "bf16", f"decode spike {kw}")


@pytest.mark.parametrize("L", [4096, 16384])
def test_long_prompt_prefill_whole_tiles(api, L):
    """The long-prompt causal prefill exactly as it is timed (one request,
    prefix 0, H 28/4, key-split workspace), checked on whole 128-row tiles:
    the first two, one in the middle and the last two.  A tile holds packed
    rows 128t .. 128t + 127 (packed row rho = position rho / 7 of head
    rho % 7 of a kv head), so every head of positions 128t // 7 ..
    (128t + 127) // 7 is compared; rows [i0, i1) of the call see the same
    keys as the call with those rows alone after a context of i1 tokens
    (bottom-right causal alignment), which the oracle finishes in seconds.
    The instrumented build of the same staging mode traces every key."""
    x = make_random(100 + L, B=1, H_q=28, H_kv=4, L=L, D=128, page_size=16, ctx=[L],
                    dtype="bf16", causal=True, extra_free_pages=16)
    print(f"[long L={L}] seed={x.seed}", flush=True)
    d = DeviceInputs(x)
    out, ex = run_prefill(api, d)
    assert not ex["counters"].any()
    got = host_f64(out)
    assert np.isfinite(got).all()
    G = x.H_q // x.H_kv
    nt = -(-G * L // 128)
    for t in sorted({0, 1, nt // 2, nt - 2, nt - 1}):
        i0, i1 = 128 * t // G, min(L, (128 * t + 127) // G + 1)
        sub = dataclasses.replace(x, L=i1 - i0, query=np.ascontiguousarray(x.query[:, :, i0:i1]),
                                  context_lens=np.array([i1], dtype=np.int32))
        ref = oracle.attention_of(sub)
        err = assert_parity(out[:, :, i0:i1], ref, "bf16", f"L={L} tile {t} rows {i0}..{i1}")
        print(f"[long L={L}] tile {t}: rows {i0}..{i1} max abs err {err:.3e}", flush=True)
    _traced_prefill_matches(api, d, x, out)
    print(f"[long L={L}] trace bit-exact", flush=True)
