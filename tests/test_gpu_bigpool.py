"""Page pools past 2 GiB: the live pages sit at the top of a pool of more than
2^31 bytes per K and V tensor, where byte offsets no longer fit 31 bits (the
prefill then stages through per-run buffer resources instead of one
pool-wide resource).  Results must not depend on where the pages live
(physical relabelling is invisible to attention), so the oracle runs on the
compact pool.  Marked gpu: needs an MI355X (about 4.1 GiB of device memory)."""
import numpy as np
import pytest

import oracle
from tests._gpu import DeviceInputs, assert_parity, dev, run_decode, run_prefill
from workloads import make_append, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()  # fail loudly if the library is missing
    return a


def _big(x, extra=512):
    """Device pools of more than 2 GiB each holding x's pages at the top, and
    the block table relabelled to match (fp8 pools: NaN codes elsewhere)."""
    import torch
    fp8 = getattr(x, "kv_dtype", None) == "fp8_e4m3"
    page_bytes = x.H_kv * x.page_size * x.D * (1 if fp8 else 2)
    n_big = (1 << 31) // page_bytes + extra
    assert n_big * page_bytes > (1 << 31)
    ids = np.arange(n_big - x.num_pages, n_big)          # compact page i -> ids[i]
    if fp8:
        kp = torch.full((n_big, x.H_kv, x.page_size, x.D), 0x7F, dtype=torch.uint8, device="cuda")
    else:
        garbage = torch.tensor([9984.0], dtype=torch.bfloat16).item()
        kp = torch.full((n_big, x.H_kv, x.page_size, x.D), garbage, dtype=torch.bfloat16,
                        device="cuda")
    vp = torch.full_like(kp, kp.flatten()[0].item())
    idx = torch.from_numpy(ids).to("cuda")
    kp[idx] = dev(x.key_pages)
    vp[idx] = dev(x.value_pages)
    bt = np.where(x.block_table >= 0, ids[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    d = DeviceInputs(x, pages=(kp, vp))
    d.bt = dev(bt)
    print(f"[bigpool] {x.name} pool {n_big} pages x {page_bytes} B = {n_big * page_bytes / 2**30:.3f} GiB",
          flush=True)
    return d, ids


@pytest.mark.parametrize("split", [False, True])
def test_prefill_pool_past_2gib(api, split):
    x = make_random(61, B=3, H_q=8, H_kv=2, L=40, D=128, page_size=16, ctx=[40, 170, 333],
                    dtype="bf16", causal=True, name="bigpool_prefill")
    d, _ = _big(x)
    out, _ = run_prefill(api, d, split=split)
    assert_parity(out, oracle.attention_of(x), "bf16", "prefill, pool past 2 GiB")


@pytest.mark.parametrize("shape", [
    dict(seed=64, D=128, page_size=5, kv=None),     # per-lane register staging
    dict(seed=65, D=128, page_size=5, kv="fp8_e4m3"),
    dict(seed=66, D=64, page_size=16, kv=None),     # one buffer resource per 8-key run
])
def test_prefill_pool_past_2gib_other_shapes(api, shape):
    """Pools past 2 GiB with a page size that is not a multiple of 8 (the
    only calls that still stage through registers, bf16 and fp8) and with
    D = 64 (per-run resources): against the oracle, split and unsplit."""
    kv = shape["kv"]
    x = make_random(shape["seed"], B=3, H_q=8, H_kv=2, L=40, D=shape["D"],
                    page_size=shape["page_size"], ctx=[40, 170, 333], dtype="bf16", causal=True,
                    name="bigpool_prefill_other", kv_dtype=kv, kv_scales=(0.45, 1.3))
    d, _ = _big(x)
    ref = oracle.attention_of(x)
    for split in (False, True):
        out, _ = run_prefill(api, d, split=split)
        assert_parity(out, ref, "bf16", f"prefill past 2 GiB {shape} split={split}")
    del d
    import torch
    torch.cuda.empty_cache()


def test_decode_pool_past_2gib(api):
    x = make_random(62, B=4, H_q=8, H_kv=2, L=1, D=128, page_size=16, ctx=[1, 77, 900, 2050],
                    dtype="bf16", causal=True, name="bigpool_decode")
    d, _ = _big(x)
    out, _ = run_decode(api, d)
    assert_parity(out, oracle.attention_of(x), "bf16", "decode, pool past 2 GiB")


def test_append_pool_past_2gib(api):
    import torch
    a = make_append(63, B=2, H_kv=2, D=128, page_size=16, ctx_old=[10, 40], n_new=[20, 9],
                    dtype="bf16", pad_tokens=2, name="bigpool_append")
    d, ids = _big(a.paged)
    sm = np.where(a.slot_mapping >= 0,
                  ids[np.maximum(a.slot_mapping, 0) // 16] * 16 + np.maximum(a.slot_mapping, 0) % 16,
                  -1).astype(np.int32)
    api.pa_append(dev(a.key), dev(a.value), dev(sm), d.kp, d.vp)
    torch.cuda.synchronize()
    for t in np.flatnonzero(sm >= 0):
        page, off = divmod(int(sm[t]), 16)
        got_k = d.kp[page, :, off, :].view(torch.int16).cpu().numpy().view(np.uint16)
        got_v = d.vp[page, :, off, :].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got_k, a.key[t]) and np.array_equal(got_v, a.value[t])
