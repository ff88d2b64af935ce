"""fp64 CPU oracle for residual vector quantization (RVQ).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.
It shares no code, header, table or helper with the HIP library.

The arithmetic lives in ``rvq_oracle.c`` (plain C, fp64, sequential sums,
OpenMP over rows only), built here with gcc.  This wrapper converts inputs to
fp64 exactly (fp32 and bf16 values are all representable in fp64) and takes
the plain means and roundings that the definitions call for.

Sources (pages' titles and sections):
  * "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", section "Visual
    Primitive Modeling": RVQ turns native-resolution features into
    multi-level discrete tokens; Figure 1: tokens are reconstructed.
  * "LongCat-2.5 Open Source Release: Meituan's 1.6T Multimodal Agent Model
    with 1M Context", section "02 Visual Coding and 3D": residual
    quantization adds detail level by level.
  * "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", paragraph "Offline Visual
    Preprocessing": a fixed tokenizer.

Per-function pins live in ``tests/test_oracle.py``, and
``tests/test_oracle_mutants.py`` plants mistakes in the C source that those
pins must catch; ``packing.py`` (the packing objective and its exhaustive
search) is pinned by ``tests/test_oracle_packing.py``.  Every function is
pinned (no "parity unpinned" entry).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rvq_oracle.c")
_LIB = os.path.join(_HERE, "librvq_oracle.so")

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction); with
    force=False only when the library is missing or older than its source."""
    stale = not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str) -> ctypes.CDLL:
    """Load a built oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.rvq_oracle_encode.argtypes = [p, i64, i32, p, i32, i32, p, p, p, p, p, i32]
    lib.rvq_oracle_decode.argtypes = [p, i64, p, i32, i32, i32, i32, p, i32]
    lib.rvq_oracle_hist.argtypes = [p, i64, i32, i32, p]
    lib.rvq_oracle_row_sq_residual.argtypes = [p, p, i64, i32, p, i32, i32, p, i32]
    lib.rvq_oracle_teacher_forced.argtypes = [p, p, i64, i32, p, i32, i32, p, p, i32]
    lib.rvq_oracle_embed.argtypes = [p, p, i64, i32, p, i64, p, i32, i32, p, i32]
    for f in ("rvq_oracle_encode", "rvq_oracle_decode", "rvq_oracle_hist",
              "rvq_oracle_row_sq_residual", "rvq_oracle_teacher_forced", "rvq_oracle_embed"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """Exact conversion of fp32 / bf16-bits / fp64 rows to fp64."""
    if dtype == "bf16":
        a = widen_bf16(a)
    a = np.ascontiguousarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle inputs must be finite")
    return a


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def encode(x: np.ndarray, codebooks: np.ndarray, x_dtype: str = "f32",
           threads: int = 0) -> dict:
    """Greedy RVQ in fp64.  Returns ids [n,L] int32, gap/rn2/ms [n,L] fp64 and
    the final residual res [n,d] fp64 (see rvq_oracle.c for definitions)."""
    lib = _load()
    x64 = as_f64(x, x_dtype)
    cb = as_f64(codebooks)
    L, K, d = cb.shape
    n = x64.shape[0]
    if x64.ndim != 2 or x64.shape[1] != d:
        raise ValueError("x must be [n, d] with the codebooks' d")
    ids = np.empty((n, L), dtype=np.int32)
    gap = np.empty((n, L), dtype=np.float64)
    rn2 = np.empty((n, L), dtype=np.float64)
    ms = np.empty((n, L), dtype=np.float64)
    res = np.empty((n, d), dtype=np.float64)
    _check(lib.rvq_oracle_encode(_ptr(x64), n, d, _ptr(cb), L, K, _ptr(ids), _ptr(gap),
                                 _ptr(rn2), _ptr(ms), _ptr(res), int(threads)), "encode")
    return {"ids": ids, "gap": gap, "rn2": rn2, "ms": ms, "res": res}


def decode(ids: np.ndarray, codebooks: np.ndarray, levels: Optional[int] = None,
           threads: int = 0) -> np.ndarray:
    """fp64 sum of the chosen codewords, level order; ``levels`` = prefix length."""
    lib = _load()
    cb = as_f64(codebooks)
    L, K, d = cb.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = ids.shape[0]
    if ids.ndim != 2 or ids.shape[1] != L:
        raise ValueError("ids must be [n, L]")
    levels = L if levels is None else int(levels)
    out = np.empty((n, d), dtype=np.float64)
    _check(lib.rvq_oracle_decode(_ptr(ids), n, _ptr(cb), L, K, d, levels, _ptr(out),
                                 int(threads)), "decode")
    return out


def embed(ids: np.ndarray, level_tables: np.ndarray, is_visual: Optional[np.ndarray] = None,
          text_table: Optional[np.ndarray] = None, table_dtype: str = "f32",
          threads: int = 0) -> np.ndarray:
    """fp64 token embeddings [T, D] of a mixed sequence: a visual token sums
    its level rows in level order, a text token is row ids[t, 0] of the text
    table.  Tables are fp32, or bf16 bit patterns with table_dtype="bf16"."""
    lib = _load()
    vis = as_f64(level_tables, table_dtype)
    L, K, D = vis.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    if ids.ndim != 2 or ids.shape[1] != L:
        raise ValueError("ids must be [T, L]")
    T = ids.shape[0]
    flags = None if is_visual is None else np.ascontiguousarray(is_visual, dtype=np.uint8)
    txt = None if text_table is None else as_f64(text_table, table_dtype)
    V = 0 if txt is None else txt.shape[0]
    if txt is not None and txt.shape[1] != D:
        raise ValueError("text table width differs from the level tables'")
    out = np.empty((T, D), dtype=np.float64)
    _check(lib.rvq_oracle_embed(_ptr(ids), _ptr(flags), T, L, _ptr(txt), V, _ptr(vis), K, D,
                                _ptr(out), int(threads)), "embed")
    return out


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), one
    rounding; returned as fp64 holding the bf16 value.  Uses v = m * 2^e with
    0.5 <= |m| < 1; bf16 keeps 8 significant bits, so m is rounded to a
    multiple of 2^-8 (numpy.rint rounds halves to even)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def bf16_bits_of(v_bf16_valued: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp64 values that are exactly bf16 values."""
    f = np.ascontiguousarray(v_bf16_valued, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def hist(ids: np.ndarray, K: int) -> np.ndarray:
    """Per-level codeword usage counts [L, K] int64."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, L = ids.shape
    h = np.empty((L, K), dtype=np.int64)
    _check(lib.rvq_oracle_hist(_ptr(ids), n, L, int(K), _ptr(h)), "hist")
    return h


def row_sq_residual(x: np.ndarray, ids: np.ndarray, codebooks: np.ndarray,
                    x_dtype: str = "f32", threads: int = 0) -> np.ndarray:
    """ms[n, l] = ||x_n - sum_{j<=l} C_j[ids[n,j]]||^2 in fp64."""
    lib = _load()
    x64 = as_f64(x, x_dtype)
    cb = as_f64(codebooks)
    L, K, d = cb.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = x64.shape[0]
    if ids.shape != (n, L):
        raise ValueError("ids must be [n, L]")
    ms = np.empty((n, L), dtype=np.float64)
    _check(lib.rvq_oracle_row_sq_residual(_ptr(x64), _ptr(ids), n, d, _ptr(cb), L, K,
                                          _ptr(ms), int(threads)), "row_sq_residual")
    return ms


def msr(x: np.ndarray, ids: np.ndarray, codebooks: np.ndarray, x_dtype: str = "f32",
        threads: int = 0) -> np.ndarray:
    """Per-level mean squared residual [L]: the mean over rows of
    row_sq_residual, summed sequentially over rows in fp64."""
    ms = row_sq_residual(x, ids, codebooks, x_dtype, threads)
    n, L = ms.shape
    out = np.zeros(L, dtype=np.float64)
    if n == 0:
        return out
    for l in range(L):
        s = 0.0
        for v in ms[:, l].tolist():
            s += v
        out[l] = s / n
    return out


def teacher_forced(x: np.ndarray, ids: np.ndarray, codebooks: np.ndarray,
                   x_dtype: str = "f32", threads: int = 0) -> dict:
    """Along the given IDs: excess[n,l] = dist(chosen) - min dist, and the
    squared norm rho2[n,l] of the residual the choice was made for."""
    lib = _load()
    x64 = as_f64(x, x_dtype)
    cb = as_f64(codebooks)
    L, K, d = cb.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = x64.shape[0]
    if ids.shape != (n, L):
        raise ValueError("ids must be [n, L]")
    excess = np.empty((n, L), dtype=np.float64)
    rho2 = np.empty((n, L), dtype=np.float64)
    _check(lib.rvq_oracle_teacher_forced(_ptr(x64), _ptr(ids), n, d, _ptr(cb), L, K,
                                         _ptr(excess), _ptr(rho2), int(threads)),
           "teacher_forced")
    return {"excess": excess, "rho2": rho2}
