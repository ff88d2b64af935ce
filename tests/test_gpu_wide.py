"""Rows wider than 1280 features (1281 to 8192), which rvq_encode encodes
with exact fp32 distances on the vector ALUs, against the fp64 oracle: the
IDs under both parity rules on every row, the residual, determinism and
batch invariance, and the maximum width."""
import numpy as np
import pytest
import torch

import parity
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rvq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import residual_vector_quantization_rvq_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.mark.parametrize("seed,n,d,L,K,dt", [
    (61, 300, 1281, 3, 200, "f32"),     # one past the matrix-core width, ragged rows and tiles
    (62, 129, 1536, 4, 513, "bf16"),
    (63, 65, 2048, 2, 1000, "f32"),
    (64, 37, 3001, 3, 64, "bf16"),      # width not a multiple of 16
    (65, 1, 1300, 5, 1, "f32"),         # one row, one codeword
    (66, 70, 8192, 2, 130, "f32"),      # the largest width
])
def test_wide_rows_against_the_oracle(rvq, dev, seed, n, d, L, K, dt):
    w = workloads.random_problem(seed, n, d, L, K, x_dtype=dt)
    x = parity.x_to_device(w, dev)
    cb = torch.from_numpy(w.codebooks).to(dev)
    prep = rvq.rvq_prepare_codebooks(cb)
    ids, res = rvq.rvq_encode(x, cb, prep, residual=True)
    ids2, res2 = rvq.rvq_encode(x, cb, prep, residual=True)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    print(f"[wide] seed {seed} n {n} d {d} L {L} K {K} {dt}",
          parity.check_ids(ids_h, w.x, dt, w.codebooks), flush=True)
    parity.check_residual(res.cpu().numpy(), w.x, dt, ids_h, w.codebooks)
    # deterministic, and a row's result does not depend on the other rows
    assert torch.equal(ids, ids2) and torch.equal(res.view(torch.int32), res2.view(torch.int32))
    a, b = n // 3, max(n // 3 + 1, (2 * n) // 3)
    ids_s, res_s = rvq.rvq_encode(x[a:b].contiguous(), cb, prep, residual=True)
    torch.cuda.synchronize()
    assert torch.equal(ids_s, ids[a:b])
    assert torch.equal(res_s.view(torch.int32), res[a:b].view(torch.int32))


def test_wide_duplicate_codewords_pick_the_lowest_index(rvq, dev):
    # every row's nearest codeword is present three times: the lowest index wins
    g = np.random.default_rng(67)
    d, K = 1600, 40
    cb = (g.standard_normal((1, K, d)) / np.sqrt(d)).astype(np.float32)
    cb[0, 31] = cb[0, 7]
    cb[0, 35] = cb[0, 7]
    x = np.repeat(cb[0, 7:8], 5, axis=0) + np.float32(1e-3) * g.standard_normal((5, d)).astype(np.float32)
    cbt = torch.from_numpy(cb).to(dev)
    ids = rvq.rvq_encode(torch.from_numpy(x).to(dev), cbt, rvq.rvq_prepare_codebooks(cbt))
    torch.cuda.synchronize()
    assert (ids.cpu().numpy()[:, 0] == 7).all()


def test_wide_random_shapes(rvq, dev):
    # random wide shapes, every row against the oracle (RVQ_WIDE_SHAPES sets
    # the count, default 12)
    import os
    g = np.random.default_rng(68)
    for i in range(int(os.environ.get("RVQ_WIDE_SHAPES", "12"))):
        d = int(g.integers(1281, 4097))
        n = int(g.integers(1, 200))
        L = int(g.integers(1, 5))
        K = int(g.integers(1, 900))
        dt = "bf16" if g.random() < 0.5 else "f32"
        w = workloads.random_problem(6800 + i, n, d, L, K, x_dtype=dt)
        x = parity.x_to_device(w, dev)
        cb = torch.from_numpy(w.codebooks).to(dev)
        ids, res = rvq.rvq_encode(x, cb, rvq.rvq_prepare_codebooks(cb), residual=True)
        torch.cuda.synchronize()
        ids_h = ids.cpu().numpy()
        tag = f"seed {6800 + i} n {n} d {d} L {L} K {K} {dt}"
        try:
            st = parity.check_ids(ids_h, w.x, dt, w.codebooks)
            parity.check_residual(res.cpu().numpy(), w.x, dt, ids_h, w.codebooks)
        except AssertionError as e:
            raise AssertionError(f"{tag}: {e}") from None
        print(f"[wide sweep] {tag}: {st['decisions']} decisions ok", flush=True)


def test_wide_rows_through_the_streaming_and_no_allocation_encoders(rvq, dev):
    # the streaming tokeniser (host rows in chunks) and rvq_encode_noalloc
    # (the library's own scratch) take wide rows too, bit for bit as
    # rvq_encode
    import ctypes
    n, d, L, K = 700, 2000, 3, 300
    w = workloads.random_problem(69, n, d, L, K, x_dtype="bf16")
    x = parity.x_to_device(w, dev)
    cb = torch.from_numpy(w.codebooks).to(dev)
    prep = rvq.rvq_prepare_codebooks(cb)
    ids, res = rvq.rvq_encode(x, cb, prep, residual=True)
    torch.cuda.synchronize()
    host = x.cpu()
    sids, done = rvq.rvq_stream_encode(host, cb, prep, chunk_rows=256)
    assert done == 3
    assert torch.equal(sids, ids.cpu())
    ids_b = torch.full((n, L), -1, dtype=torch.int32, device=dev)
    res_b = torch.full((n, d), float("nan"), dtype=torch.float32, device=dev)
    st = rvq.raw_library().rvq_encode_noalloc(
        ctypes.c_void_p(x.data_ptr()), 1, n, d, ctypes.c_void_p(cb.data_ptr()),
        ctypes.c_void_p(prep.data_ptr()), L, K, ctypes.c_void_p(ids_b.data_ptr()),
        ctypes.c_void_p(res_b.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, rvq.raw_library().rvq_last_error().decode()
    assert torch.equal(ids_b, ids)
    assert torch.equal(res_b.view(torch.int32), res.view(torch.int32))
