"""The step's entry points under HIP graph capture: prepare, encode (both
encoder modes) and the fused decode + statistics pass are captured once and
replayed several times, with other eager work and synchronisations between
the replays, and every replay must reproduce the eager results bit for bit.
The library issues no memset, allocation or host synchronisation inside
these calls, which is what makes them capturable."""
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


def _step(rvq, x, cb, ws, ids):
    prep = rvq.rvq_prepare_codebooks(cb)
    _, res = rvq.rvq_encode(x, cb, prep, residual=True, workspace=ws, ids_out=ids)
    dec, hist, msr = rvq.rvq_decode_level_stats(ids, x, cb, torch.bfloat16)
    return res, dec, hist, msr


CASES = {
    # 1024 rows: the split plan, 2 launches per level
    "single_image": lambda: workloads.single_image(),
    # enough rows for all levels in one launch
    "fused": lambda: workloads.random_problem(53, 20000, 256, 3, 500, x_dtype="bf16"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_replays_from_a_graph(rvq, dev, name):
    w = CASES[name]()
    x = parity.x_to_device(w, dev)
    cb = torch.from_numpy(w.codebooks).to(dev)
    n, d, L, K = w.N, w.D, w.L, w.K
    ws = torch.empty(rvq.rvq_encode_workspace_size(n, d, L, K), dtype=torch.uint8, device=dev)
    ids = torch.empty((n, L), dtype=torch.int32, device=dev)
    ref = [t.clone() for t in _step(rvq, x, cb, ws, ids)]
    ref_ids = ids.clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream(device=dev)          # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):                 # warm-up on the capture stream's side
        _step(rvq, x, cb, ws, ids)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = _step(rvq, x, cb, ws, ids)

    for rep in range(4):
        # eager work between replays: clobber the outputs, run another encode
        ids.fill_(-1)
        for t in out:
            t.zero_()
        other = rvq.rvq_encode(x[: min(n, 300)].contiguous(), cb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids), f"replay {rep}: ids"
        assert torch.equal(other, ref_ids[: min(n, 300)])
        for a, b, what in zip(out, ref, ("residual", "decode", "counts", "msr")):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {what}"
    print(f"[graph {name}] 4 replays bit-exact")
