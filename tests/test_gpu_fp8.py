"""GPU parity of fp8 (E4M3) K/V pages against the oracle, through the C ABI:
the decode path reading fp8 pages with per-tensor k/v scales (address trace
bit-exact, output within the bf16 bar), and the write path quantising bf16
rows into an fp8 pool (every byte of the pool equal to the oracle's codes).
Marked gpu: needs an MI355X and libpa.so."""
import numpy as np
import pytest

import oracle
from oracle.scatter import scatter_tokens_fp8
from tests._gpu import DeviceInputs, assert_parity, dev, expected_visits, host_f64, run_decode
from workloads import make_append, make_c2_fp8, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def _expect(x):
    tr = oracle.translate_of(x)
    v = expected_visits(x)
    for b in range(x.B):
        if x.rows_valid()[b] == 0:
            tr[b] = -1
            v[b] = 0
    return tr, v


def _check(api, x, **kw):
    d = DeviceInputs(x)
    out, ex = run_decode(api, d, **kw)
    err = assert_parity(out, oracle.attention_of(x), "bf16", f"fp8 {kw} S={ex['S']}")
    t_out, tex = run_decode(api, d, trace=True, **kw)
    tr, v = _expect(x)
    assert np.array_equal(tex["trace"], tr)
    assert np.array_equal(tex["visits"], v)
    assert np.array_equal(host_f64(t_out), host_f64(out)), "traced output differs"
    return out, err


CASES = [
    # seed, H_q, H_kv, L, ps, ctx, partition_tokens, causal, scales
    (1, 32, 8, 1, 16, [1, 15, 16, 17, 31, 32, 33, 100], 0, True, (0.5, 0.5)),
    (2, 8, 2, 2, 16, [2, 64, 700, 2049], 0, True, (0.37, 1.7)),
    (3, 16, 4, 1, 32, [5, 31, 32, 500], 64, True, (1.0, 0.25)),
    (4, 4, 4, 1, 128, [1, 128, 129, 1000], 256, False, (0.5, 0.5)),
    (5, 28, 4, 1, 5, [1, 9, 23, 61], 10, True, (0.8, 0.6)),     # per-lane walk
    (6, 7, 1, 1, 1, [3, 4, 17], 0, True, (0.5, 0.5)),           # page size 1
    (7, 64, 8, 1, 48, [1, 47, 48, 4097], 0, True, (8.0, 0.3)),     # peaked scores
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_fp8_decode_parity_and_trace(api, case):
    seed, Hq, Hkv, L, ps, ctx, P, causal, scales = case
    print(f"[fp8] seed={seed} Hq={Hq} Hkv={Hkv} L={L} ps={ps} ctx={ctx} P={P} scales={scales}",
          flush=True)
    x = make_random(seed, B=len(ctx), H_q=Hq, H_kv=Hkv, L=L, D=128, page_size=ps, ctx=ctx,
                    dtype="bf16", causal=causal, extra_free_pages=4, kv_dtype="fp8_e4m3",
                    kv_scales=scales)
    _check(api, x, partition_tokens=P)


def test_fp8_c2_full_size(api):
    x = make_c2_fp8()
    print(f"[C2-fp8] seed={x.seed}", flush=True)
    out, err = _check(api, x)
    print(f"[C2-fp8] max abs err {err:.3e}", flush=True)
    # the merge kernel and the fused merge agree
    b, _ = run_decode(api, DeviceInputs(x), fused=False)
    assert_parity(b, oracle.attention_of(x, precision="f64"), "bf16", "C2-fp8 merge kernel")


@pytest.mark.parametrize("garbage", ["nan", "random"])
def test_fp8_stale_codes_bit_identical(api, garbage):
    kw = dict(B=4, H_q=8, H_kv=2, L=1, D=128, page_size=16, ctx=[5, 33, 100, 250],
              dtype="bf16", causal=True, extra_free_pages=6, kv_dtype="fp8_e4m3")
    base, _ = run_decode(api, DeviceInputs(make_random(51, **kw)))
    o, _ = run_decode(api, DeviceInputs(make_random(51, garbage=garbage, **kw)))
    assert np.array_equal(host_f64(o), host_f64(base))


def test_fp8_noalloc_matches_workspace_decode(api):
    import torch
    x = make_random(61, B=6, H_q=32, H_kv=8, L=1, D=128, page_size=16,
                    ctx=[1, 300, 4096, 17, 999, 2048], dtype="bf16", causal=True,
                    kv_dtype="fp8_e4m3", kv_scales=(0.3, 0.7))
    d = DeviceInputs(x)
    ref, _ = run_decode(api, d)
    out = d.out()
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                         k_scale=x.k_scale, v_scale=x.v_scale)
    api.pa_decode_noalloc(args)
    torch.cuda.synchronize()
    assert np.array_equal(host_f64(out), host_f64(ref))


@pytest.mark.parametrize("shape", [
    dict(seed=2, B=64, H_kv=8, D=128, page_size=16, ctx_old=(127, 4095), n_new=[1] * 64),
    dict(seed=3, B=4, H_kv=4, D=128, page_size=16, ctx_old=(0, 2048), n_new=[512] * 4,
         pad_tokens=7),
    dict(seed=5, B=3, H_kv=2, D=64, page_size=5, ctx_old=[0, 3, 9], n_new=[7, 1, 12]),
])
def test_fp8_append_quantises_bit_exact(api, shape):
    """pa_append into an fp8 pool: every byte of both pools equals the
    oracle's codes of row / scale (untouched bytes included), with rows that
    plant ties, overflows and NaN beside the random ones."""
    import torch
    a = make_append(dtype="bf16", kv_dtype="fp8_e4m3", kv_scales=(0.37, 1.9), **shape)
    p = a.paged
    key = a.key.copy()
    # plant exact ties / saturation / NaN in the first live token (bf16 bits)
    from workloads import f32_to_bf16_bits
    t0 = int(np.nonzero(a.slot_mapping >= 0)[0][0])
    planted = np.array([1.0625, 1.1875, 1e4, -1e4, 2.0 ** -10, 3 * 2.0 ** -10], np.float32)
    key[t0, 0, :6] = f32_to_bf16_bits(planted * np.float32(0.37))
    key[t0, 0, 6] = 0x7FC0
    kp, vp = dev(p.key_pages), dev(p.value_pages)
    print(f"[fp8 append] seed {a.seed} T {a.num_tokens} H_kv {p.H_kv} D {p.D} ps {p.page_size}",
          flush=True)
    api.pa_append(dev(key), dev(a.value), dev(a.slot_mapping), kp, vp,
                  k_scale=p.k_scale, v_scale=p.v_scale)
    torch.cuda.synchronize()
    want_k, want_v = scatter_tokens_fp8(p.key_pages, p.value_pages, key, a.value,
                                        a.slot_mapping, p.k_scale, p.v_scale)
    assert np.array_equal(kp.cpu().numpy(), want_k)
    assert np.array_equal(vp.cpu().numpy(), want_v)
