"""Randomised parity sweep through the C ABI: decode, prefill and the K/V
write on shapes drawn from seeded generators (dtype, head size, GQA group,
page size from 1 to 256, ragged query lengths, empty contexts, explicit
partitions, the balanced schedule on small grids, the key split on and off)
against the oracle, at the same bars as the hand-picked cases."""
import numpy as np
import pytest

import oracle
from oracle.scatter import scatter_tokens
from tests._gpu import DeviceInputs, assert_parity, dev, run_decode, run_prefill
from workloads import make_append, make_random

pytestmark = pytest.mark.gpu

KINDS = ("decode", "prefill", "append")
SEEDS = range(31000, 31060)


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def _shape(seed):
    r = np.random.default_rng(seed)
    kind = KINDS[seed % 3]
    s = dict(kind=kind, dt="bf16" if r.random() < 0.8 else "f32", D=int(r.choice([64, 128])),
             Hkv=int(r.choice([1, 2, 4, 8])), G=int(r.integers(1, 9)),
             ps=int(r.choice([1, 3, 8, 16, 16, 16, 32, 48, 64, 128, 256])),
             B=int(r.integers(1, 7)))
    B = s["B"]
    if kind == "append":
        s.update(ctx_old=[int(v) for v in r.integers(0, 600, B)],
                 n_new=[int(v) for v in r.integers(0, 300, B)], pad=int(r.integers(0, 3)))
        return s
    causal = bool(r.random() < 0.8)
    L = int(r.integers(1, 9)) if kind == "decode" else int(r.choice([1, 5, 17, 64, 100, 129, 250]))
    ql = [int(v) for v in r.integers(0, L + 1, B)] if r.random() < 0.3 else None
    rows = ql if ql is not None else [L] * B
    ctx = [int(max(rows[b] if causal else 0, v)) for b, v in enumerate(r.integers(0, 3000, B))]
    if r.random() < 0.2:
        ctx[0] = rows[0] if causal else 0
    s.update(causal=causal, L=L, ql=ql, ctx=ctx, free=int(r.integers(0, 9)),
             P=0 if r.random() < 0.6 else s["ps"] * int(r.integers(1, 40)),
             cus_dec=int(r.choice([0, 1, 3, 16])), fused=bool(r.random() < 0.7),
             split=bool(r.random() < 0.7), cus_pre=int(r.choice([0, 2, 512])))
    return s


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape(api, seed):
    import torch
    s = _shape(seed)
    print(f"[sweep] seed={seed} {s}", flush=True)
    if s["kind"] == "append":
        a = make_append(seed, B=s["B"], H_kv=s["Hkv"], D=s["D"], page_size=s["ps"],
                        ctx_old=s["ctx_old"], n_new=s["n_new"], dtype=s["dt"], pad_tokens=s["pad"])
        kp, vp = dev(a.paged.key_pages), dev(a.paged.value_pages)
        if a.num_tokens > 0:
            api.pa_append(dev(a.key), dev(a.value), dev(a.slot_mapping), kp, vp)
        torch.cuda.synchronize()
        want_k, want_v = scatter_tokens(a.paged.key_pages, a.paged.value_pages, a.key, a.value,
                                        a.slot_mapping)
        if s["dt"] == "bf16":
            got_k = kp.view(torch.int16).cpu().numpy().view(np.uint16)
            got_v = vp.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            got_k, got_v = kp.cpu().numpy(), vp.cpu().numpy()
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)
        return
    x = make_random(seed, B=s["B"], H_q=s["G"] * s["Hkv"], H_kv=s["Hkv"], L=s["L"], D=s["D"],
                    page_size=s["ps"], ctx=s["ctx"], dtype=s["dt"], causal=s["causal"],
                    query_lens=s["ql"], extra_free_pages=s["free"])
    ref = oracle.attention_of(x)
    d = DeviceInputs(x)
    if s["kind"] == "decode":
        out, ex = run_decode(api, d, partition_tokens=s["P"], num_cus=s["cus_dec"],
                             fused=s["fused"])
        assert_parity(out, ref, s["dt"], f"sweep decode seed {seed} S={ex['S']}")
    else:
        out, ex = run_prefill(api, d, split=s["split"], num_cus=s["cus_pre"])
        assert_parity(out, ref, s["dt"], f"sweep prefill seed {seed}")
        if "counters" in ex:
            assert not ex["counters"].any()
