"""rvq_encode_noalloc (the encoder with the library's own device scratch as
its workspace), called through the C ABI, against rvq_encode with a
caller workspace: the same IDs and residual bits on two calls in a row,
the second smaller, and a host-side error for inputs whose workspace
exceeds the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import parity
import workloads

pytestmark = pytest.mark.gpu


def _raw(rvq, x, cb, prep, ids, res, dev):
    L, K, d = cb.shape
    return rvq.raw_library().rvq_encode_noalloc(
        ctypes.c_void_p(x.data_ptr()), 1 if x.dtype == torch.bfloat16 else 0, x.shape[0], d,
        ctypes.c_void_p(cb.data_ptr()), ctypes.c_void_p(prep.data_ptr()), L, K,
        ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(res.data_ptr()) if res is not None else None,
        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))


def test_noalloc_matches_the_workspace_encoder():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import residual_vector_quantization_rvq_amd as rvq
    dev = torch.device("cuda:0")
    # a native-resolution image of 84 x 84 patches at the benchmark shape
    # (the largest the scratch holds), then a smaller ragged problem
    cases = [(61, 7056, 1152, 8, 8192, "bf16"), (62, 777, 200, 3, 700, "f32")]
    for seed, n, d, L, K, dt in cases:
        w = workloads.random_problem(seed, n, d, L, K, x_dtype=dt)
        x = parity.x_to_device(w, dev)
        cb = torch.from_numpy(w.codebooks).to(dev)
        prep = rvq.rvq_prepare_codebooks(cb)
        ids_a, res_a = rvq.rvq_encode(x, cb, prep, residual=True)
        ids_b = torch.full((n, L), -1, dtype=torch.int32, device=dev)
        res_b = torch.full((n, d), float("nan"), dtype=torch.float32, device=dev)
        st = _raw(rvq, x, cb, prep, ids_b, res_b, dev)
        torch.cuda.synchronize()
        print(f"[noalloc] n={n} d={d} L={L} K={K} {dt}: status {st}", flush=True)
        assert st == 0, rvq.raw_library().rvq_last_error().decode()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(res_a.view(torch.int32), res_b.view(torch.int32))
        sel = np.arange(0, n, max(1, n // 64))
        sub = w.rows(sel)
        parity.check_ids(ids_b.cpu().numpy()[sel], sub.x, dt, w.codebooks)
    # beyond the scratch: refused on the host, nothing written
    w = workloads.random_problem(63, 40000, 1152, 2, 256, x_dtype="bf16")
    x = parity.x_to_device(w, dev)
    cb = torch.from_numpy(w.codebooks).to(dev)
    prep = rvq.rvq_prepare_codebooks(cb)
    ids = torch.full((40000, 2), -1, dtype=torch.int32, device=dev)
    st = _raw(rvq, x, cb, prep, ids, None, dev)
    torch.cuda.synchronize()
    assert st == 2 and "scratch" in rvq.raw_library().rvq_last_error().decode()
    assert torch.all(ids == -1)
