"""dory_op_argmax_noalloc (partials in the library's own device array, for
callers that cannot allocate) against dory_op_argmax (caller scratch): the
same greedy ids bit for bit, on two calls in a row with the second smaller,
plus ties, +-0 and +-inf, and the capacity limit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import looped_ngpt_amd as dory  # noqa: E402


def _reference(logits):
    B, V = logits.shape
    out = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(dory.argmax_scratch_bytes(B, V), dtype=torch.uint8, device="cuda")
    dory.op_argmax(logits, out, scratch)
    return out


def _noalloc(logits):
    out = torch.full((logits.shape[0],), -1, dtype=torch.int32, device="cuda")
    dory.op_argmax_noalloc(logits, out)
    return out


def _logits(B, V, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(B, V, generator=g)
    # ties on the maximum (lowest index wins), signed zeros, infinities
    x[0, V // 3] = x[0].max() + 1
    x[0, V // 2] = x[0, V // 3]
    if B > 1:
        x[1] = -0.0
        x[1, 7] = 0.0
    if B > 2:
        x[2, V - 1] = float("inf")
        x[2, 5] = float("inf")
    return x.cuda()


def test_noalloc_argmax_matches_scratch_argmax_two_calls():
    big = _logits(64, 131072, 1)                    # the array's full size: 64 x 128 partials
    small = _logits(3, 1000, 2)                     # then a smaller input (one partial per row)
    print("noalloc argmax: 64 x 131072 then 3 x 1000", flush=True)
    for x in (big, small):
        ref = _reference(x)
        got = _noalloc(x)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
        np.testing.assert_array_equal(got.cpu().numpy(), np.argmax(x.cpu().numpy(), axis=-1))
    # the first call's partials are still in the array: a third, larger call
    # must not read them
    mid = _logits(5, 50000, 3)
    np.testing.assert_array_equal(_noalloc(mid).cpu().numpy(), _reference(mid).cpu().numpy())


def test_noalloc_argmax_limits():
    x = torch.zeros(65, 131072, device="cuda")      # 65 x 128 partials > 8192
    out = torch.empty(65, dtype=torch.int32, device="cuda")
    with pytest.raises(dory.DoryError) as e:
        dory.op_argmax_noalloc(x, out)
    assert e.value.status == dory.DORY_E_CAPACITY
    y = torch.zeros(1, 8192 * 1024, device="cuda")  # one row at the limit
    y[0, 8192 * 1024 - 2] = 1.0
    out1 = torch.empty(1, dtype=torch.int32, device="cuda")
    dory.op_argmax_noalloc(y, out1)
    assert int(out1.item()) == 8192 * 1024 - 2
