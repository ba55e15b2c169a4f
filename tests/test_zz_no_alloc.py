"""The forward that allocates nothing, against dbf_linear_forward.

dbf_linear_forward_noalloc runs the kernels of dbf_linear_forward with their
scratch in the library's static device array.  Each case calls both entry
points through the C ABI on the same handle and inputs, twice in a row with
the second input smaller than the first (so the second call finds the first
one's leftovers in the array), and requires:

* identical fp16 bits (the same kernels and arithmetic; the parity of the
  forward itself against the oracle is covered by the parity suites),
* no change of the device's free memory across the no-allocation calls,
* DBF_ERR_SHAPE, and untouched outputs, for a batch whose scratch exceeds
  the array.

Every case prints its name before it touches the GPU.
"""

import sys

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf
from tests import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _both(torch, H, X):
    """(dbf_linear_forward output, dbf_linear_forward_noalloc output, free bytes before, after)."""
    x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    batch = X.shape[0]
    y_ref = torch.empty((batch, H.n), dtype=torch.float16, device="cuda")
    y_na = torch.full((batch, H.n), float("nan"), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    dbf.dbf_linear_forward(H.handle, x.data_ptr(), y_ref.data_ptr(), batch, stream)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    dbf.dbf_linear_forward_noalloc(H.handle, x.data_ptr(), y_na.data_ptr(), batch, stream)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return y_ref.cpu().numpy(), y_na.cpu().numpy(), free0, free1


# (name, n, m, k, first batch, second batch): prefill then the batch-1 int8
# decode; the matrix-core decode with its stage-1 reduction cut into parts
# (wide m: tickets and partials in the array), then batch 1; decode batch 16
# then 3.
CASES = [
    ("prefill300_then_decode1", 1000, 1300, 600, 300, 1),
    ("decode9_parts_then_decode1", 256, 10240, 1024, 9, 1),
    ("decode16_then_decode3", 333, 257, 129, 16, 3),
]


@pytest.mark.parametrize("name,n,m,k,b1,b2", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_forward(gpu, name, n, m, k, b1, b2):
    import torch
    _say(f"noalloc {name} n={n} m={m} k={k} batches {b1},{b2}")
    L = inputs.random_layer(name, n, m, k, 41, 0.05, 1.0, 0.05, (b1, b2))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=max(b1, b2))
    try:
        # one call first: resolves the array's address on this device
        x0 = torch.from_numpy(np.ascontiguousarray(L.X[b2])).cuda()
        y0 = torch.empty((b2, n), dtype=torch.float16, device="cuda")
        dbf.dbf_linear_forward_noalloc(H.handle, x0.data_ptr(), y0.data_ptr(), b2,
                                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for b in (b1, b2):
            y_ref, y_na, free0, free1 = _both(torch, H, L.X[b])
            assert np.array_equal(y_ref.view(np.uint16), y_na.view(np.uint16)), f"{name} batch {b}: outputs differ"
            assert free1 == free0, f"{name} batch {b}: free device memory changed ({free0} -> {free1})"
    finally:
        H.close()


def test_noalloc_rejects_oversized_scratch(gpu):
    import torch
    # k_pad 16384 at batch 2100: the prefill intermediate alone is 2 * 2100 *
    # 16384 bytes, more than the 64 MiB array
    n, m, k, b = 64, 64, 16384, 2100
    _say(f"noalloc oversized n={n} m={m} k={k} batch {b}")
    L = inputs.random_layer("big", n, m, k, 43, 0.05, 1.0, 0.05, (b,))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=b)
    try:
        x = torch.from_numpy(L.X[b]).cuda()
        y = torch.zeros((b, n), dtype=torch.float16, device="cuda")
        with pytest.raises(dbf.DbfError) as e:
            dbf.dbf_linear_forward_noalloc(H.handle, x.data_ptr(), y.data_ptr(), b,
                                           torch.cuda.current_stream().cuda_stream)
        assert e.value.status == dbf.DBF_ERR_SHAPE
        torch.cuda.synchronize()
        assert not torch.any(y != 0).item()
        # the same call through dbf_linear_forward (the handle's own workspace) works
        dbf.dbf_linear_forward(H.handle, x.data_ptr(), y.data_ptr(), b, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all().item()
    finally:
        H.close()
