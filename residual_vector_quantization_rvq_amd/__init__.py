"""Residual vector quantization (RVQ) on MI355X (gfx950).

Thin Python binding of ``librvq.so`` (the C ABI in ``include/rvq.h``).  It
only marshals arguments: torch allocates device memory (outputs and
workspaces) and supplies the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing, importing this package raises.

Functions keep the C names:
  rvq_prepare_codebooks(codebooks)            -> prepared buffer (uint8 tensor)
  rvq_encode(x, codebooks, prepared)          -> ids [n, L] int32 (, residual)
  rvq_decode(ids, codebooks, out_dtype, ...)  -> reconstruction [n, d]
  rvq_level_stats(ids, K, x, codebooks)       -> (hist [L, K] int64, msr [L] fp64)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

__all__ = [
    "RVQError", "library_path", "exported_symbols", "RVQ_F32", "RVQ_BF16",
    "rvq_prepared_size", "rvq_prepare_codebooks", "rvq_encode_workspace_size", "rvq_encode",
    "rvq_encode_noalloc", "rvq_decode", "rvq_level_stats_workspace_size", "rvq_level_stats",
    "rvq_decode_level_stats",
    "rvq_embed_tokens", "rvq_idcache_resume", "rvq_idcache_append", "rvq_idcache_read",
    "rvq_stream_workspace_size", "rvq_stream_encode", "rvq_stream_encode_to_cache",
    "rvq_pack_ranks", "rvq_mfma_rate", "rvq_status_string",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "librvq.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "rvq.h")

RVQ_OK, RVQ_ERR_INVALID_ARGUMENT, RVQ_ERR_UNSUPPORTED, RVQ_ERR_WORKSPACE_TOO_SMALL, RVQ_ERR_HIP = range(5)
RVQ_F32, RVQ_BF16 = 0, 1


class RVQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(_LIB_PATH)
_i32, _i64, _sz, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_psz = ctypes.POINTER(ctypes.c_size_t)

_lib.rvq_status_string.argtypes = [ctypes.c_int]
_lib.rvq_status_string.restype = ctypes.c_char_p
_lib.rvq_last_error.argtypes = []
_lib.rvq_last_error.restype = ctypes.c_char_p
_lib.rvq_prepared_size.argtypes = [_i32, _i32, _i32, _psz]
_lib.rvq_prepare_codebooks.argtypes = [_p, _i32, _i32, _i32, _p, _sz, _p]
_lib.rvq_encode_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _psz]
_lib.rvq_encode.argtypes = [_p, ctypes.c_int, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _p, _sz, _p]
_lib.rvq_encode_profiled.argtypes = [_p, ctypes.c_int, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _p,
                                     _sz, _p, _p, ctypes.POINTER(ctypes.c_int32)]
_lib.rvq_encode_noalloc.argtypes = [_p, ctypes.c_int, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _p]
_lib.rvq_decode.argtypes = [_p, _i64, _p, _i32, _i32, _i32, _i32, _p, ctypes.c_int, _p, _p]
_lib.rvq_level_stats_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _psz]
_lib.rvq_level_stats.argtypes = [_p, _i64, _i32, _i32, _p, _p, ctypes.c_int, _i32, _p, _p, _p,
                                 _p, _sz, _p]
_lib.rvq_decode_level_stats.argtypes = [_p, _i64, _p, _i32, _i32, _i32, _p, ctypes.c_int, _p, _p,
                                        ctypes.c_int, _p, _p, _p, _sz, _p]
_lib.rvq_embed_tokens.argtypes = [_p, _p, _i64, _i32, _p, _i64, _p, _i32, _i32, ctypes.c_int,
                                  _p, ctypes.c_int, _p, _p]
_pi64 = ctypes.POINTER(ctypes.c_int64)
_lib.rvq_idcache_resume.argtypes = [ctypes.c_char_p, _i64, _i32, _i32, _i64, _pi64]
_lib.rvq_idcache_append.argtypes = [ctypes.c_char_p, _i64, _i32, _i32, _i64, _i64, _p]
_lib.rvq_idcache_read.argtypes = [ctypes.c_char_p, _i64, _i32, _i32, _i64, _p, _pi64]
_CHUNK_CB = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                             ctypes.c_int64, ctypes.c_void_p)
_lib.rvq_pack_ranks.argtypes = [_p, _p, _i64, _i32, _i64, _i32, _p, _p]
_lib.rvq_stream_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _psz]
_lib.rvq_stream_encode.argtypes = [_p, ctypes.c_int, _i64, _i32, _p, _p, _i32, _i32, _p, _i64,
                                   _i64, _i64, _p, _p, _p, _sz, _p, _pi64]
_lib.rvq_stream_encode_to_cache.argtypes = [ctypes.c_char_p, _p, ctypes.c_int, _i64, _i32, _p,
                                            _p, _i32, _i32, _p, _i64, _i64, _p, _sz, _p, _pi64]
_lib.rvq_mfma_rate_workspace_size.argtypes = [_i32]
_lib.rvq_mfma_rate_workspace_size.restype = ctypes.c_size_t
_lib.rvq_mfma_rate.argtypes = [_i32, _i32, _i32, _p, _sz, _p, ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(ctypes.c_double)]
for _f in ("rvq_mfma_rate", "rvq_prepared_size", "rvq_prepare_codebooks", "rvq_encode_workspace_size",
           "rvq_encode", "rvq_encode_noalloc", "rvq_encode_profiled", "rvq_decode",
           "rvq_level_stats_workspace_size", "rvq_level_stats", "rvq_decode_level_stats", "rvq_embed_tokens", "rvq_idcache_resume",
           "rvq_idcache_append", "rvq_idcache_read", "rvq_stream_workspace_size",
           "rvq_stream_encode", "rvq_stream_encode_to_cache", "rvq_pack_ranks"):
    getattr(_lib, _f).restype = ctypes.c_int


def raw_library() -> ctypes.CDLL:
    """The loaded ctypes library (for callers passing raw pointers)."""
    return _lib


def exported_symbols() -> list:
    """Function names declared in include/rvq.h."""
    with open(_HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rvq_\w+)\s*\(", text, re.M)))


def rvq_status_string(status: int) -> str:
    return _lib.rvq_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != RVQ_OK:
        raise RVQError(status, f"{rvq_status_string(status)}: {_lib.rvq_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return RVQ_F32
    if dt == torch.bfloat16:
        return RVQ_BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def _need_cuda(name: str, t: torch.Tensor, device: Optional[torch.device] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_codebooks(codebooks: torch.Tensor, device: Optional[torch.device] = None):
    """Codebooks are a float32 [L, K, d] device tensor; returns (L, K, d)."""
    _need_cuda("codebooks", codebooks, device)
    if codebooks.dtype != torch.float32 or codebooks.dim() != 3:
        raise ValueError("codebooks must be float32 [L, K, d]")
    return tuple(int(v) for v in codebooks.shape)


def _need_shape(name: str, t: torch.Tensor, shape: tuple, dtype: torch.dtype,
                device: torch.device) -> None:
    _need_cuda(name, t, device)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} {list(shape)} (got {t.dtype} {list(t.shape)})")


def _need_bytes(name: str, t: torch.Tensor, nbytes: int, device: torch.device) -> None:
    _need_cuda(name, t, device)
    if t.dtype != torch.uint8 or t.dim() != 1 or t.numel() < nbytes:
        raise ValueError(f"{name} must be a uint8 buffer of at least {nbytes} bytes")


def rvq_prepared_size(L: int, K: int, d: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.rvq_prepared_size(L, K, d, ctypes.byref(out)))
    return out.value


def rvq_prepare_codebooks(codebooks: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Norms and bf16 copy of a fixed [L, K, d] fp32 codebook set."""
    L, K, d = _need_codebooks(codebooks)
    nbytes = rvq_prepared_size(L, K, d)
    if out is not None:
        _need_bytes("out", out, nbytes, codebooks.device)
    prepared = out if out is not None else torch.empty(nbytes, dtype=torch.uint8,
                                                       device=codebooks.device)
    _check(_lib.rvq_prepare_codebooks(_ptr(codebooks), L, K, d, _ptr(prepared), prepared.numel(),
                                      _stream(codebooks.device)))
    return prepared


def rvq_encode_workspace_size(n: int, d: int, L: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.rvq_encode_workspace_size(n, d, L, K, ctypes.byref(out)))
    return out.value


def rvq_encode(x: torch.Tensor, codebooks: torch.Tensor, prepared: Optional[torch.Tensor] = None,
               residual: bool = False, workspace: Optional[torch.Tensor] = None,
               ids_out: Optional[torch.Tensor] = None, events=None, launches=None):
    """Greedy RVQ encode of rows x [n, d] (fp32 or bf16).  Returns ids [n, L]
    int32, and the fp32 final residual [n, d] when ``residual`` is true.
    ``events``: optional ctypes array of 2*L hipEvent_t recorded around each
    distance launch; ``launches``: optional ctypes.c_int32 receiving the
    number of launches recorded (rvq_encode_profiled)."""
    _need_cuda("x", x)
    dev = x.device
    L, K, d = _need_codebooks(codebooks, dev)
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError("x must be [n, d] with the codebooks' d")
    _dtype_code(x.dtype)
    n = x.shape[0]
    if prepared is None:
        prepared = rvq_prepare_codebooks(codebooks)
    _need_bytes("prepared", prepared, rvq_prepared_size(L, K, d), dev)
    if ids_out is not None:
        _need_shape("ids_out", ids_out, (n, L), torch.int32, dev)
    ids = ids_out if ids_out is not None else torch.empty((n, L), dtype=torch.int32, device=dev)
    res = torch.empty((n, d), dtype=torch.float32, device=dev) if residual else None
    wbytes = rvq_encode_workspace_size(n, d, L, K)
    if workspace is not None:
        _need_cuda("workspace", workspace, dev)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a uint8 [bytes] tensor")
    if workspace is None or workspace.numel() < wbytes:
        workspace = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    _check(_lib.rvq_encode_profiled(_ptr(x), _dtype_code(x.dtype), n, d, _ptr(codebooks),
                                    _ptr(prepared), L, K, _ptr(ids), _ptr(res), _ptr(workspace),
                                    workspace.numel(), _stream(dev), events,
                                    None if launches is None else ctypes.byref(launches)))
    return (ids, res) if residual else ids


def rvq_encode_noalloc(x: torch.Tensor, codebooks: torch.Tensor, prepared: torch.Tensor,
                       ids_out: torch.Tensor, residual_out: Optional[torch.Tensor] = None) -> None:
    """rvq_encode into caller-given outputs with the library's own device
    scratch as workspace (no device allocation in the call)."""
    _need_cuda("x", x)
    dev = x.device
    L, K, d = _need_codebooks(codebooks, dev)
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError("x must be [n, d] with the codebooks' d")
    n = x.shape[0]
    _need_bytes("prepared", prepared, rvq_prepared_size(L, K, d), dev)
    _need_shape("ids_out", ids_out, (n, L), torch.int32, dev)
    if residual_out is not None:
        _need_shape("residual_out", residual_out, (n, d), torch.float32, dev)
    _check(_lib.rvq_encode_noalloc(_ptr(x), _dtype_code(x.dtype), n, d, _ptr(codebooks),
                                   _ptr(prepared), L, K, _ptr(ids_out), _ptr(residual_out),
                                   _stream(dev)))


def rvq_decode(ids: torch.Tensor, codebooks: torch.Tensor, out_dtype: torch.dtype = torch.float32,
               levels: Optional[int] = None, bad_ids: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sum of the chosen codewords of the first ``levels`` levels (default all)."""
    _need_cuda("ids", ids)
    dev = ids.device
    L, K, d = _need_codebooks(codebooks, dev)
    n = ids.shape[0]
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[1] != L:
        raise ValueError("ids must be int32 [n, L]")
    levels = L if levels is None else int(levels)
    _dtype_code(out_dtype)
    if bad_ids is not None:
        _need_shape("bad_ids", bad_ids, (1,), torch.int32, dev)
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=dev)
    _need_shape("out", out, (n, d), out_dtype, dev)
    _check(_lib.rvq_decode(_ptr(ids), n, _ptr(codebooks), L, K, d, levels, _ptr(out),
                           _dtype_code(out.dtype), _ptr(bad_ids), _stream(ids.device)))
    return out


def rvq_embed_tokens(ids: torch.Tensor, level_tables: torch.Tensor,
                     is_visual: Optional[torch.Tensor] = None,
                     text_table: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32,
                     bad_ids: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One embedding row per token of a mixed sequence: a visual token sums its
    rows of the per-level tables [L, K, D], a text token (is_visual == 0) is
    row ids[t, 0] of text_table [V, D].  Tables are float32 or bfloat16."""
    _need_cuda("ids", ids)
    dev = ids.device
    _need_cuda("level_tables", level_tables, dev)
    if level_tables.dim() != 3:
        raise ValueError("level_tables must be [L, K, D]")
    L, K, D = level_tables.shape
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[1] != L:
        raise ValueError("ids must be int32 [T, L]")
    T = ids.shape[0]
    _dtype_code(out_dtype)
    if bad_ids is not None:
        _need_shape("bad_ids", bad_ids, (1,), torch.int32, dev)
    tdt = _dtype_code(level_tables.dtype)
    V = 0
    if text_table is not None:
        _need_cuda("text_table", text_table, dev)
        if text_table.dtype != level_tables.dtype or text_table.dim() != 2 or text_table.shape[1] != D:
            raise ValueError("text_table must be [V, D] in the level tables' dtype")
        V = text_table.shape[0]
    if is_visual is not None:
        _need_cuda("is_visual", is_visual, dev)
        if is_visual.dtype == torch.bool:
            is_visual = is_visual.view(torch.uint8)
        if is_visual.dtype != torch.uint8 or is_visual.shape != (T,):
            raise ValueError("is_visual must be uint8 or bool [T]")
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype, device=dev)
    _need_shape("out", out, (T, D), out_dtype, dev)
    _check(_lib.rvq_embed_tokens(_ptr(ids), _ptr(is_visual), T, L, _ptr(text_table), V,
                                 _ptr(level_tables), K, D, tdt, _ptr(out), _dtype_code(out.dtype),
                                 _ptr(bad_ids), _stream(ids.device)))
    return out


def rvq_idcache_resume(path: str, n: int, L: int, K: int, chunk_rows: int) -> int:
    """Create the ID cache file, or check and trim an existing one; returns the
    number of leading chunks it holds."""
    done = ctypes.c_int64()
    _check(_lib.rvq_idcache_resume(os.fsencode(path), n, L, K, chunk_rows, ctypes.byref(done)))
    return done.value


def rvq_idcache_append(path: str, n: int, L: int, K: int, chunk_rows: int, chunk: int,
                       ids) -> None:
    """Append chunk ``chunk``: a host int32 array (numpy or CPU tensor) of its
    rows x L IDs."""
    import numpy as np
    a = np.ascontiguousarray(ids.numpy() if isinstance(ids, torch.Tensor) else ids, dtype=np.int32)
    _check(_lib.rvq_idcache_append(os.fsencode(path), n, L, K, chunk_rows, chunk,
                                   a.ctypes.data_as(ctypes.c_void_p)))


def rvq_idcache_read(path: str, n: int, L: int, K: int, chunk_rows: int):
    """(ids [n, L] int32 numpy array, number of valid leading chunks); rows of
    missing chunks are -1."""
    import numpy as np
    ids = np.full((n, L), -1, dtype=np.int32)
    done = ctypes.c_int64()
    _check(_lib.rvq_idcache_read(os.fsencode(path), n, L, K, chunk_rows,
                                 ids.ctypes.data_as(ctypes.c_void_p), ctypes.byref(done)))
    return ids, done.value


def rvq_pack_ranks(text_tokens, image_tokens, ranks: int, capacity: int, exact_max: int = 12):
    """Assign samples (text and image token counts, host sequences) to
    `ranks` data-parallel ranks of at most `capacity` tokens each, keeping
    every rank's visual share close to the batch's.  Returns (rank of each
    sample as an int32 numpy array, summary): summary holds "dev" (max over
    ranks of |V_r - p N_r| times N, an integer), "N" and "max_load"."""
    import numpy as np
    t = np.ascontiguousarray(text_tokens, dtype=np.int64)
    v = np.ascontiguousarray(image_tokens, dtype=np.int64)
    if t.ndim != 1 or t.shape != v.shape:
        raise ValueError("text_tokens and image_tokens must be 1-D and of one length")
    out = np.empty(t.shape[0], dtype=np.int32)
    summ = np.zeros(3, dtype=np.int64)
    _check(_lib.rvq_pack_ranks(t.ctypes.data_as(ctypes.c_void_p), v.ctypes.data_as(ctypes.c_void_p),
                               t.shape[0], int(ranks), int(capacity), int(exact_max),
                               out.ctypes.data_as(ctypes.c_void_p),
                               summ.ctypes.data_as(ctypes.c_void_p)))
    return out, {"dev": int(summ[0]), "N": int(summ[1]), "max_load": int(summ[2])}


def rvq_stream_workspace_size(chunk_rows: int, d: int, L: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.rvq_stream_workspace_size(chunk_rows, d, L, K, ctypes.byref(out)))
    return out.value


def _stream_args(x_host: torch.Tensor, codebooks: torch.Tensor, prepared: torch.Tensor,
                 chunk_rows: int, ids_out: Optional[torch.Tensor],
                 workspace: Optional[torch.Tensor]):
    if x_host.is_cuda or not x_host.is_contiguous() or x_host.dim() != 2:
        raise ValueError("x_host must be a contiguous [n, d] host tensor")
    L, K, d = _need_codebooks(codebooks)
    n = x_host.shape[0]
    if x_host.shape[1] != d:
        raise ValueError("x_host width differs from the codebooks'")
    _dtype_code(x_host.dtype)
    _need_bytes("prepared", prepared, rvq_prepared_size(L, K, d), codebooks.device)
    if ids_out is None:
        ids_out = torch.empty((n, L), dtype=torch.int32, pin_memory=x_host.is_pinned())
    if ids_out.is_cuda or ids_out.dtype != torch.int32 or ids_out.shape != (n, L):
        raise ValueError("ids_out must be a host int32 [n, L] tensor")
    wbytes = rvq_stream_workspace_size(chunk_rows, d, L, K)
    if workspace is None:
        workspace = torch.empty(wbytes, dtype=torch.uint8, device=codebooks.device)
    _need_bytes("workspace", workspace, wbytes, codebooks.device)
    return n, d, L, K, ids_out, workspace


def rvq_stream_encode(x_host: torch.Tensor, codebooks: torch.Tensor, prepared: torch.Tensor,
                      chunk_rows: int, ids_out: Optional[torch.Tensor] = None,
                      first_chunk: int = 0, max_chunks: int = 0, on_chunk=None,
                      workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """Encode host rows chunk by chunk with overlapped copies; returns the host
    IDs [n, L] and the number of chunks done.  on_chunk(chunk, row0, rows)
    is called after each chunk's IDs are in ids; a true return stops."""
    n, d, L, K, ids_out, workspace = _stream_args(x_host, codebooks, prepared, chunk_rows,
                                                  ids_out, workspace)
    errors = []

    def relay(_user, chunk, row0, rows, _ids):
        try:
            return 1 if on_chunk(int(chunk), int(row0), int(rows)) else 0
        except BaseException as e:  # an exception cannot cross the C frame
            errors.append(e)
            return 1
    cb = _CHUNK_CB(relay) if on_chunk is not None else None
    done = ctypes.c_int64()
    _check(_lib.rvq_stream_encode(_ptr(x_host), _dtype_code(x_host.dtype), n, d, _ptr(codebooks),
                                  _ptr(prepared), L, K, _ptr(ids_out), chunk_rows, first_chunk,
                                  max_chunks, ctypes.cast(cb, ctypes.c_void_p) if cb else None,
                                  None, _ptr(workspace), workspace.numel(),
                                  _stream(codebooks.device), ctypes.byref(done)))
    if errors:
        raise errors[0]
    return ids_out, done.value


def rvq_stream_encode_to_cache(path: str, x_host: torch.Tensor, codebooks: torch.Tensor,
                               prepared: torch.Tensor, chunk_rows: int,
                               ids_out: Optional[torch.Tensor] = None, max_chunks: int = 0,
                               workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """rvq_stream_encode into the resumable ID cache at path (continues a
    partial file); returns the host IDs of the chunks run and the number of
    chunks the file holds."""
    n, d, L, K, ids_out, workspace = _stream_args(x_host, codebooks, prepared, chunk_rows,
                                                  ids_out, workspace)
    done = ctypes.c_int64()
    _check(_lib.rvq_stream_encode_to_cache(os.fsencode(path), _ptr(x_host),
                                           _dtype_code(x_host.dtype), n, d, _ptr(codebooks),
                                           _ptr(prepared), L, K, _ptr(ids_out), chunk_rows,
                                           max_chunks, _ptr(workspace), workspace.numel(),
                                           _stream(codebooks.device), ctypes.byref(done)))
    return ids_out, done.value


def rvq_level_stats_workspace_size(n: int, L: int, K: int, d: int, with_msr: bool) -> int:
    out = ctypes.c_size_t()
    _check(_lib.rvq_level_stats_workspace_size(n, L, K, d, 1 if with_msr else 0, ctypes.byref(out)))
    return out.value


def rvq_level_stats(ids: torch.Tensor, K: int, x: Optional[torch.Tensor] = None,
                    codebooks: Optional[torch.Tensor] = None,
                    bad_ids: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Per-level usage counts [L, K] int64 and, when x is given, the per-level
    mean squared residual [L] fp64."""
    _need_cuda("ids", ids)
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise ValueError("ids must be int32 [n, L]")
    n, L = ids.shape
    dev = ids.device
    if bad_ids is not None:
        _need_shape("bad_ids", bad_ids, (1,), torch.int32, dev)
    hist = torch.empty((L, K), dtype=torch.int64, device=dev)
    msr = None
    d = 1
    xdt = RVQ_F32
    if x is not None:
        _need_cuda("x", x, dev)
        if codebooks is None:
            raise ValueError("codebooks are required with x")
        if x.dim() != 2 or x.shape[0] != n:
            raise ValueError("x must be [n, d] with the IDs' n")
        d = x.shape[1]
        if _need_codebooks(codebooks, dev) != (L, K, d):
            raise ValueError(f"codebooks must be float32 [{L}, {K}, {d}] (the IDs' L, K and x's d)")
        xdt = _dtype_code(x.dtype)
        msr = torch.empty((L,), dtype=torch.float64, device=dev)
    wbytes = rvq_level_stats_workspace_size(n, L, K, d, x is not None)
    if workspace is not None:
        _need_cuda("workspace", workspace, dev)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a uint8 [bytes] tensor")
    if workspace is None or workspace.numel() < wbytes:
        workspace = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    _check(_lib.rvq_level_stats(_ptr(ids), n, L, K, _ptr(hist), _ptr(x), xdt, d, _ptr(codebooks),
                                _ptr(msr), _ptr(bad_ids), _ptr(workspace), workspace.numel(),
                                _stream(dev)))
    return hist, msr


def rvq_decode_level_stats(ids: torch.Tensor, x: torch.Tensor, codebooks: torch.Tensor,
                           out_dtype: torch.dtype = torch.float32,
                           bad_ids: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None
                           ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Full decode [n, d], usage counts [L, K] int64 and mean squared residual
    [L] fp64 of the same IDs in one gather pass (the same bits as rvq_decode
    followed by rvq_level_stats)."""
    _need_cuda("ids", ids)
    dev = ids.device
    _need_cuda("x", x, dev)
    L, K, d = _need_codebooks(codebooks, dev)
    n = ids.shape[0]
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[1] != L:
        raise ValueError("ids must be int32 [n, L]")
    if x.dim() != 2 or x.shape[0] != n or x.shape[1] != d:
        raise ValueError("x must be [n, d] with the codebooks' d")
    _dtype_code(x.dtype)
    _dtype_code(out_dtype)
    if bad_ids is not None:
        _need_shape("bad_ids", bad_ids, (1,), torch.int32, dev)
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=dev)
    _need_shape("out", out, (n, d), out_dtype, dev)
    hist = torch.empty((L, K), dtype=torch.int64, device=dev)
    msr = torch.empty((L,), dtype=torch.float64, device=dev)
    wbytes = rvq_level_stats_workspace_size(n, L, K, d, True)
    if workspace is not None:
        _need_cuda("workspace", workspace, dev)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a uint8 [bytes] tensor")
    if workspace is None or workspace.numel() < wbytes:
        workspace = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    _check(_lib.rvq_decode_level_stats(_ptr(ids), n, _ptr(codebooks), L, K, d, _ptr(out),
                                       _dtype_code(out.dtype), _ptr(hist), _ptr(x),
                                       _dtype_code(x.dtype), _ptr(msr), _ptr(bad_ids),
                                       _ptr(workspace), workspace.numel(), _stream(dev)))
    return out, hist, msr


def rvq_mfma_rate(blocks: int, iters: int, zero_operands: bool = False,
                  device: Optional[torch.device] = None):
    """The matrix cores' achievable bf16 rate: a register-only loop of
    v_mfma_f32_32x32x16_bf16 on `blocks` four-wave workgroups (one per
    compute unit for one wave per SIMD), on random or all-zero operands.
    Waits for the run.  Returns (TFLOP/s, shader clock in GHz)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    ws = torch.empty(int(_lib.rvq_mfma_rate_workspace_size(blocks)), dtype=torch.uint8, device=dev)
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    _check(_lib.rvq_mfma_rate(blocks, iters, 1 if zero_operands else 0, _ptr(ws), ws.numel(),
                              _stream(dev), ctypes.byref(tf), ctypes.byref(ghz)))
    return tf.value, ghz.value
