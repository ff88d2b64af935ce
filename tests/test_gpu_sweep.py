"""Random shapes against the fp64 oracle: widths 1 to 1280, 1 to 12 levels,
1 to 6000 codewords, fp32 and bf16 rows, both encoder modes.  On sampled
rows the IDs must equal the oracle's wherever its best-to-second gap exceeds
1e-4 ||r||^2 (and be within that of the nearest everywhere), and residuals
must match the fp64 ones.  The number of shapes is RVQ_SWEEP_SHAPES (default
40) and the seed of the shape draw RVQ_SWEEP_SEED (default 2024); the test
stops at the first shape that breaks a rule."""
import os

import numpy as np
import pytest
import torch

import oracle
import parity
import workloads

pytestmark = pytest.mark.gpu


def _shapes(count: int, seed: int = 2024):
    g = np.random.default_rng(seed)
    # (problem seeds differ between shape draws, so no problem repeats)
    base = 5000 if seed == 2024 else 100000 + 1000 * (seed % 1000)
    for i in range(count):
        d = int(g.choice([g.integers(1, 65), g.integers(65, 600), g.integers(600, 1281)]))
        L = int(g.integers(1, 13))
        K = int(g.choice([g.integers(1, 300), g.integers(300, 6001)]))
        fused = g.random() < 0.3 and d * K * L <= 6e7
        n = int(g.integers(19712, 24000)) if fused else int(g.integers(1, 3000))
        dt = "bf16" if g.random() < 0.5 else "f32"
        yield base + i, n, d, L, K, dt


def test_random_shapes_against_the_oracle():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import residual_vector_quantization_rvq_amd as rvq
    dev = torch.device("cuda:0")
    count = int(os.environ.get("RVQ_SWEEP_SHAPES", "40"))
    shape_seed = int(os.environ.get("RVQ_SWEEP_SEED", "2024"))
    decisions = strict = 0
    for seed, n, d, L, K, dt in _shapes(count, shape_seed):
        w = workloads.random_problem(seed, n, d, L, K, x_dtype=dt)
        x = parity.x_to_device(w, dev)
        cb = torch.from_numpy(w.codebooks).to(dev)
        ids, res = rvq.rvq_encode(x, cb, rvq.rvq_prepare_codebooks(cb), residual=True)
        torch.cuda.synchronize()
        rows = min(n, int(max(16, min(256, 4e9 / (3.0 * L * K * d)))))
        sel = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).choice(n, rows, replace=False)]))
        sub = w.rows(sel)
        ids_h = ids.cpu().numpy()[sel]
        ref = oracle.encode(sub.x, sub.codebooks, x_dtype=dt)
        tag = f"seed {seed} n {n} d {d} L {L} K {K} {dt}"
        try:
            st = parity.check_ids(ids_h, sub.x, dt, w.codebooks, ref=ref)
            parity.check_residual(res[torch.from_numpy(sel).to(dev)].cpu().numpy(), sub.x, dt,
                                  ids_h, w.codebooks)
        except AssertionError as e:
            raise AssertionError(f"{tag}: {e}") from None
        decisions += st["decisions"]
        strict += st["strict_decisions"]
        print(f"[sweep] {tag}: {st['decisions']} decisions ok", flush=True)
    print(f"[sweep] {count} shapes, {decisions} sampled decisions, {strict} strict; none broke a rule")
