"""Binding checks that need device tensors: a host tensor mixed into a GPU
call, and metadata shapes that disagree with the query, are refused before
anything is launched."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_96_amd import api as a
    a._lib.lib()
    return a


def test_mixed_devices_and_bad_shapes_are_refused(api):
    import torch
    q = torch.zeros(2, 4, 1, 64, device="cuda")
    kp = torch.zeros(8, 2, 16, 64, device="cuda")
    bt = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    cl = torch.ones(2, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    api.make_args(q, kp, kp.clone(), bt, cl, out)  # consistent: accepted
    with pytest.raises(ValueError, match="block_table is on cpu"):
        api.make_args(q, kp, kp.clone(), bt.cpu(), cl, out)
    with pytest.raises(ValueError, match="context_lens"):
        api.make_args(q, kp, kp.clone(), bt, torch.ones(1, dtype=torch.int32, device="cuda"), out)
    with pytest.raises(ValueError, match="block_table"):
        api.make_args(q, kp, kp.clone(), bt[:1], cl, out)
    with pytest.raises(ValueError, match="query_lens"):
        api.make_args(q, kp, kp.clone(), bt, cl, out,
                      query_lens=torch.ones(3, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="slot_mapping is on cpu"):
        api.pa_append(torch.zeros(3, 2, 64, device="cuda"), torch.zeros(3, 2, 64, device="cuda"),
                      torch.zeros(3, dtype=torch.int32), kp, kp.clone())
    torch.cuda.synchronize()
