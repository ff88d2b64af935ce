"""Seeded synthetic inputs for residual vector quantization (RVQ).

This module is shared by the fp64 oracle (``oracle/``), the tests and
``bench.py``.  It only draws random numbers and lays them out; it holds none
of the quantizer's arithmetic (no distance, argmin, residual or decode step).
The one arithmetic step it performs is building the "structured" rows of the
tiny workload as a plain fp64 sum of one codeword per level, which is the
workload's own recipe for inputs whose generating IDs are known.

Every generator uses ``numpy.random.Generator(PCG64(seed))`` and a fixed draw
order: codebooks first (level 0..L-1), then inputs, then IDs.  fp64 draws are
rounded to fp32; bf16 inputs are the fp32 values rounded to nearest-even on
the upper 16 bits.  bf16 arrays are stored as ``uint16`` bit patterns.

Shapes follow the pages' setting: native-resolution visual features turned
into multi-level discrete tokens ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
section "Visual Primitive Modeling", paragraph "Discrete
Native Resolution Vision Transformer" and Figure 1: images of different
resolutions, so token counts per image are ragged).  The pages give no D, K,
L or value distributions; the five workloads below are synthetic stand-ins
with the sizes the build is measured on.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "tiny_structured",
    "single_image",
    "native_batch",
    "bulk_tokenisation",
    "decode_heavy",
    "mixed_sequence",
    "random_problem",
    "WORKLOADS",
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs must be finite.  Works in chunks so multi-GB arrays stay bounded.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        flat_out[s:s + step] = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic problem.

    x          : [N, D] fp32 array, or uint16 bf16 bits when x_dtype == "bf16"
    codebooks  : [L, K, D] fp32, one codebook per level
    gen_ids    : [N, L] int32 generating IDs where known (-1 = unknown row)
    ids        : [N_ids, L] int32 given IDs (decode/statistics workloads)
    offsets    : int64 [n_images + 1] row offsets of a ragged image batch
    """

    name: str
    codebooks: np.ndarray
    x: Optional[np.ndarray] = None
    x_dtype: str = "f32"
    gen_ids: Optional[np.ndarray] = None
    ids: Optional[np.ndarray] = None
    offsets: Optional[np.ndarray] = None
    out_dtype: str = "f32"
    notes: str = ""

    @property
    def L(self) -> int:
        return int(self.codebooks.shape[0])

    @property
    def K(self) -> int:
        return int(self.codebooks.shape[1])

    @property
    def D(self) -> int:
        return int(self.codebooks.shape[2])

    @property
    def N(self) -> int:
        return 0 if self.x is None else int(self.x.shape[0])

    def x_f32(self) -> np.ndarray:
        """Input rows widened exactly to fp32."""
        if self.x_dtype == "bf16":
            return f32_from_bf16_bits(self.x)
        return self.x

    def rows(self, sel) -> "Workload":
        """The same problem restricted to a subset of input rows."""
        sel = np.asarray(sel)
        return dataclasses.replace(
            self,
            x=None if self.x is None else np.ascontiguousarray(self.x[sel]),
            gen_ids=None if self.gen_ids is None else np.ascontiguousarray(self.gen_ids[sel]),
            offsets=None,
        )


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _gaussian_codebooks(g, L, K, D, std_of_level) -> np.ndarray:
    """Per-level fp32 Gaussian codebooks, level-major draw order."""
    cb = np.empty((L, K, D), dtype=np.float32)
    for l in range(L):
        cb[l] = (g.standard_normal((K, D)) * std_of_level(l)).astype(np.float32)
    return cb


def _normal_rows_f32(g, n, d, chunk=1 << 16) -> np.ndarray:
    out = np.empty((n, d), dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = g.standard_normal((e - s, d)).astype(np.float32)
    return out


def tiny_structured(seed: int = 1) -> Workload:
    """Tiny encode+decode: N=256, D=64, L=4, K=256.

    Codebook of level l is 4^-l * N(0,1)/sqrt(D) in fp32, so consecutive
    levels are scaled 4x apart.  Rows 0..127 are fp32 N(0,1).  Rows 128..255
    are fp32(sum over l of C_l[g_l]) with the sum taken in fp64 and g drawn
    uniformly; their generating IDs are kept in ``gen_ids``.
    """
    N, D, L, K = 256, 64, 4, 256
    g = _rng(seed)
    cb = _gaussian_codebooks(g, L, K, D, lambda l: 4.0 ** (-l) / math.sqrt(D))
    half = N // 2
    x = np.empty((N, D), dtype=np.float32)
    x[:half] = g.standard_normal((half, D)).astype(np.float32)
    gen = g.integers(0, K, size=(half, L), dtype=np.int64).astype(np.int32)
    cb64 = cb.astype(np.float64)
    acc = np.zeros((half, D), dtype=np.float64)
    for l in range(L):
        acc += cb64[l][gen[:, l]]
    x[half:] = acc.astype(np.float32)
    gen_ids = np.full((N, L), -1, dtype=np.int32)
    gen_ids[half:] = gen
    return Workload("tiny_structured", cb, x, "f32", gen_ids=gen_ids, out_dtype="f32",
                    notes="N=256 D=64 L=4 K=256; rows 128..255 are exact codeword sums")


def single_image(seed: int = 2, literal_std: bool = False) -> Workload:
    """One 32x32 image: N=1024, D=1152, L=8, K=4096, fp32 rows of unit L2 norm.

    Rows are N(0,1) draws normalised in fp64, then rounded to fp32.  Codebook
    entries of level l have std 0.7^l times s0, with s0 = 1/sqrt(D) so the
    codebooks live on the same scale as unit-norm rows (``literal_std=True``
    takes s0 = 1).
    """
    N, D, L, K = 1024, 1152, 8, 4096
    g = _rng(seed)
    s0 = 1.0 if literal_std else 1.0 / math.sqrt(D)
    cb = _gaussian_codebooks(g, L, K, D, lambda l: s0 * 0.7 ** l)
    z = g.standard_normal((N, D))
    x = (z / np.sqrt((z * z).sum(axis=1, keepdims=True))).astype(np.float32)
    return Workload("single_image", cb, x, "f32", out_dtype="f32",
                    notes=f"N=1024 D=1152 L=8 K=4096 std0={'1' if literal_std else '1/sqrt(D)'}")


def native_batch(seed: int = 3) -> Workload:
    """Ragged native-resolution batch: 16 images, H and W in patches uniform on
    14..84 inclusive, packed flat with int64 offsets.  D=1152 bf16 N(0,1)
    rows; L=8 levels of K=8192 fp32 codewords with std 0.7^l."""
    D, L, K = 1152, 8, 8192
    g = _rng(seed)
    cb = _gaussian_codebooks(g, L, K, D, lambda l: 0.7 ** l)
    hw = g.integers(14, 85, size=(16, 2), dtype=np.int64)
    counts = hw[:, 0] * hw[:, 1]
    offsets = np.zeros(17, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    N = int(offsets[-1])
    x = bf16_bits_from_f32(_normal_rows_f32(g, N, D))
    return Workload("native_batch", cb, x, "bf16", offsets=offsets, out_dtype="bf16",
                    notes=f"16 images, N={N}, D=1152 bf16, L=8, K=8192")


def bulk_tokenisation(seed: int = 4, n: int = 1 << 20) -> Workload:
    """Offline bulk tokenisation: D=1280 bf16 rows from a 64-component Gaussian
    mixture (equal weights, component means N(0,I), within-component std 0.3);
    L=16 levels of K=16384 fp32 codewords with std 0.8^l.  ``n`` defaults to
    1,048,576 rows."""
    D, L, K, C = 1280, 16, 16384, 64
    g = _rng(seed)
    cb = _gaussian_codebooks(g, L, K, D, lambda l: 0.8 ** l)
    mu = g.standard_normal((C, D))
    comp = g.integers(0, C, size=n, dtype=np.int64)
    x = np.empty((n, D), dtype=np.uint16)
    chunk = 1 << 15
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        rows = mu[comp[s:e]] + 0.3 * g.standard_normal((e - s, D))
        x[s:e] = bf16_bits_from_f32(rows.astype(np.float32))
    return Workload("bulk_tokenisation", cb, x, "bf16", out_dtype="bf16",
                    notes=f"N={n} D=1280 bf16 mixture of 64, L=16, K=16384")


def decode_heavy(seed: int = 5, n_ids: int = 4_194_304, n_msr: int = 65_536) -> Workload:
    """Decode-heavy workload with statistics.

    IDs [n_ids, 8] uniform on 0..8191, with floor(0.1*n_ids) rows (sampled
    without replacement) forced to ID 0 at every level; codebooks D=1152 fp32,
    std 0.7^l.  ``x`` is a separate [n_msr, 1152] fp32 N(0,1) subset that is
    encoded at L=8 for the mean-squared-residual statistics.
    """
    D, L, K = 1152, 8, 8192
    g = _rng(seed)
    cb = _gaussian_codebooks(g, L, K, D, lambda l: 0.7 ** l)
    x = _normal_rows_f32(g, n_msr, D)
    ids = g.integers(0, K, size=(n_ids, L), dtype=np.int64).astype(np.int32)
    hot = g.choice(n_ids, size=int(math.floor(0.1 * n_ids)), replace=False)
    ids[hot] = 0
    return Workload("decode_heavy", cb, x, "f32", ids=ids, out_dtype="bf16",
                    notes=f"ids {n_ids}x8 (10% hot rows at ID 0), msr subset {n_msr}x1152 fp32")


@dataclasses.dataclass
class MixedSequence:
    """A mixed text / visual token sequence and its embedding tables (bf16
    bit patterns): ids [T, L] int32, is_visual [T] uint8, text_table [V, D],
    level_tables [L, K, D]."""
    ids: np.ndarray
    is_visual: np.ndarray
    text_table: np.ndarray
    level_tables: np.ndarray
    notes: str = ""


def mixed_sequence(seed: int = 6, d_model: int = 4096, vocab: int = 65536) -> MixedSequence:
    """16 images as visual tokens (H and W in patches uniform on 14..84, as in
    the native batch; L=8 level IDs uniform on 0..8191), each after a text
    segment of 32..512 tokens (IDs uniform on 0..vocab-1); embedding tables
    of width d_model, bf16 N(0, 0.02^2).  Draw order: tables (levels, then
    text), image sizes, segment lengths, then IDs in sequence order."""
    L, K = 8, 8192
    g = _rng(seed)
    level = np.empty((L, K, d_model), dtype=np.uint16)
    for l in range(L):
        level[l] = bf16_bits_from_f32((0.02 * g.standard_normal((K, d_model), dtype=np.float32)))
    text = np.empty((vocab, d_model), dtype=np.uint16)
    chunk = 8192
    for s in range(0, vocab, chunk):
        e = min(vocab, s + chunk)
        text[s:e] = bf16_bits_from_f32(0.02 * g.standard_normal((e - s, d_model), dtype=np.float32))
    sizes = g.integers(14, 85, size=(16, 2), dtype=np.int64)
    counts = sizes[:, 0] * sizes[:, 1]
    seg = g.integers(32, 513, size=16, dtype=np.int64)
    T = int(seg.sum() + counts.sum())
    ids = np.zeros((T, L), dtype=np.int32)
    vis = np.zeros(T, dtype=np.uint8)
    t = 0
    for i in range(16):
        ids[t:t + seg[i], 0] = g.integers(0, vocab, size=int(seg[i]))
        t += int(seg[i])
        ids[t:t + counts[i]] = g.integers(0, K, size=(int(counts[i]), L))
        vis[t:t + counts[i]] = 1
        t += int(counts[i])
    return MixedSequence(ids, vis, text, level,
                         notes=f"T={T} ({int(counts.sum())} visual, {int(seg.sum())} text), "
                               f"L=8, K=8192, V={vocab}, D_model={d_model}, bf16 tables")


def random_problem(seed: int, n: int, d: int, L: int, K: int, x_dtype: str = "f32",
                   decay: float = 0.7, cb_scale: float = 1.0, x_scale: float = 1.0) -> Workload:
    """A generic Gaussian problem for parity tests at intermediate sizes."""
    g = _rng(seed)
    cb = _gaussian_codebooks(g, L, K, d, lambda l: cb_scale * decay ** l)
    x = (_normal_rows_f32(g, n, d) * np.float32(x_scale)).astype(np.float32)
    if x_dtype == "bf16":
        x = bf16_bits_from_f32(x)
    return Workload(f"random_s{seed}_n{n}_d{d}_L{L}_K{K}", cb, x, x_dtype,
                    out_dtype=x_dtype)


WORKLOADS = {
    "tiny_structured": tiny_structured,
    "single_image": single_image,
    "native_batch": native_batch,
    "bulk_tokenisation": bulk_tokenisation,
    "decode_heavy": decode_heavy,
}
