"""GPU-vs-oracle parity rules shared by the GPU tests.

IDs: bit-exact wherever the oracle's best-to-second gap exceeds 1e-4 times
the squared norm of the residual the decision is made for.  Operationally:
  strict prefix  -- per row, GPU IDs equal the oracle's for every level
                    before the first near-tie level of the oracle's path;
  teacher-forced -- along the GPU's own IDs (recomputed in fp64), every
                    chosen codeword is within 1e-4 * ||rho||^2 of the best,
                    which covers the near-tie level and everything after a
                    legitimate divergence.
Reconstructions: fp32 output within 1e-5 relative L2 per row of the fp64
sum.  bf16 output: per element, within one bf16 step of the fp64 sum rounded
to bf16, plus the error bound of an fp32 sum of L terms taken in level order,
(L-1) * 2^-24 * sum_l |c_l,i| (this term only matters where the codewords
cancel to far below their own size, e.g. a sum of O(1) terms that is 1e-6);
per row, within 2^-8 relative L2 of the fp64 sum.
Residual: within 1e-5 of (||x|| + sum ||c||) of x minus the fp64 sum of the
GPU's codewords.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

GAP_REL = 1e-4
RECON_REL = 1e-5


def x_to_device(w, dev) -> torch.Tensor:
    if w.x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w.x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(w.x)).to(dev)


def bf16_tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_strict_prefix(gpu_ids: np.ndarray, ref: dict) -> dict:
    """Strict-prefix rule; returns counts for reporting."""
    strict = ref["gap"] > GAP_REL * ref["rn2"]
    n, L = strict.shape
    near = ~strict
    first = np.where(near.any(axis=1), near.argmax(axis=1), L)
    bad = []
    for i in range(n):
        l = first[i]
        if not np.array_equal(gpu_ids[i, :l], ref["ids"][i, :l]):
            bad.append(i)
    assert not bad, (f"{len(bad)} rows differ from the oracle before their first near-tie level; "
                     f"first: row {bad[0]} gpu {gpu_ids[bad[0]]} oracle {ref['ids'][bad[0]]}")
    return {"rows": n, "rows_all_strict": int((first == L).sum()),
            "strict_decisions": int(strict.sum()), "decisions": int(strict.size),
            "equal_decisions": int((gpu_ids == ref["ids"]).sum())}


def check_ids(gpu_ids: np.ndarray, x, x_dtype, codebooks, ref: dict = None) -> dict:
    """Both ID rules against the fp64 oracle: the strict prefix (ref is the
    oracle's encode of the same rows, computed here when not given) and the
    teacher-forced rule along the GPU's own IDs."""
    if ref is None:
        ref = oracle.encode(x, codebooks, x_dtype=x_dtype)
    stats = check_strict_prefix(gpu_ids, ref)
    stats["worst_excess"] = check_teacher_forced(x, x_dtype, gpu_ids, codebooks)
    return stats


def check_teacher_forced(x, x_dtype, gpu_ids, codebooks) -> float:
    tf = oracle.teacher_forced(x, gpu_ids, codebooks, x_dtype=x_dtype)
    ratio = tf["excess"] / np.maximum(tf["rho2"], 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= GAP_REL, f"an ID is {worst:.3g}*||rho||^2 worse than the nearest codeword"
    return worst


def check_decode_f32(out: np.ndarray, ids: np.ndarray, codebooks, levels=None) -> float:
    ref = oracle.decode(ids, codebooks, levels=levels)
    num = np.linalg.norm(out.astype(np.float64) - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= RECON_REL, f"decode relative L2 error {worst:.3g} > {RECON_REL}"
    return worst


def _bf16_step(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), 0.0)


def check_decode_bf16(out_bits: np.ndarray, ids: np.ndarray, codebooks, levels=None) -> int:
    exact = oracle.decode(ids, codebooks, levels=levels)
    ref = oracle.round_to_bf16(exact)
    got = oracle.widen_bf16(out_bits).astype(np.float64)
    cb = np.asarray(codebooks)
    nlev = cb.shape[0] if levels is None else int(levels)
    abs_sum = np.zeros_like(exact)
    for l in range(nlev):
        abs_sum += np.abs(cb[l][ids[:, l]].astype(np.float64))
    fp32_sum_bound = max(nlev - 1, 0) * 2.0 ** -24 * abs_sum
    tol = np.maximum(_bf16_step(ref), _bf16_step(got)) + fp32_sum_bound
    diff = np.abs(got - ref)
    bad = np.argwhere(diff > tol)
    assert len(bad) == 0, (f"{len(bad)} bf16 elements off by more than one bf16 step plus the fp32 "
                           f"sum bound; first {tuple(bad[0])}: got {got[tuple(bad[0])]!r} "
                           f"want {ref[tuple(bad[0])]!r}")
    num = np.linalg.norm(got - exact, axis=1)
    den = np.linalg.norm(exact, axis=1)
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    assert rel.size == 0 or rel.max() <= 2.0 ** -8, f"bf16 decode row error {rel.max():.3g}"
    return int((diff > 0).sum())


def check_residual(res: np.ndarray, x, x_dtype, ids: np.ndarray, codebooks) -> float:
    x64 = oracle.as_f64(x, x_dtype)
    rec = oracle.decode(ids, codebooks)
    cb = np.asarray(codebooks, dtype=np.float64)
    L = cb.shape[0]
    scale = np.linalg.norm(x64, axis=1)
    for l in range(L):
        scale = scale + np.linalg.norm(cb[l][ids[:, l]], axis=1)
    err = np.linalg.norm(res.astype(np.float64) - (x64 - rec), axis=1)
    worst = float((err / np.maximum(scale, 1e-300)).max()) if err.size else 0.0
    assert worst <= RECON_REL, f"residual error {worst:.3g} (relative to ||x|| + sum ||c||)"
    return worst


def check_msr(msr: np.ndarray, x, x_dtype, ids, codebooks) -> float:
    ref = oracle.msr(x, ids, codebooks, x_dtype=x_dtype)
    rel = np.abs(msr - ref) / np.maximum(np.abs(ref), 1e-300)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= RECON_REL, f"msr relative error {worst:.3g}"
    return worst
