"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/rvq.h, sizes workspaces as documented and rejects bad
arguments on the host before any HIP call."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "residual_vector_quantization_rvq_amd", "librvq.so")


@pytest.fixture(scope="module")
def rvq():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._builder().build()
    import residual_vector_quantization_rvq_amd as m
    return m


def test_exports_every_declared_symbol(rvq):
    names = rvq.exported_symbols()
    assert {"rvq_encode", "rvq_decode", "rvq_level_stats", "rvq_prepare_codebooks",
            "rvq_status_string", "rvq_last_error"} <= set(names)
    lib = ctypes.CDLL(rvq.library_path())
    for name in names:
        assert hasattr(lib, name), f"{name} declared in rvq.h but not exported"


def test_header_is_plain_c(rvq, tmp_path):
    # a C11 program (gcc, no C++) includes rvq.h, links librvq.so and calls
    # host-side entry points
    src = tmp_path / "use.c"
    src.write_text(
        "#include <stdio.h>\n#include \"rvq.h\"\n"
        "int main(void) {\n"
        "  size_t b = 0;\n"
        "  rvq_status st = rvq_prepared_size(1, 128, 640, &b);\n"
        "  rvq_status bad = rvq_decode(NULL, 4, NULL, 2, 3, 4, 2, NULL, RVQ_F32, NULL, NULL);\n"
        "  printf(\"%d %zu %d %s\\n\", (int)st, b, (int)bad, rvq_last_error());\n"
        "  return 0;\n}\n")
    exe = tmp_path / "use"
    libdir = os.path.dirname(rvq.library_path())
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
                    "-L", libdir, "-lrvq", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    al = lambda v: (v + 255) // 256 * 256
    assert out[0] == "0" and int(out[1]) == al(128 * 4) + al(4096 + 12 * 16384) + al(8) + al(16)
    assert out[2] == "1" and "NULL" in " ".join(out[3:])


def test_status_strings(rvq):
    assert rvq.rvq_status_string(0) == "RVQ_OK"
    assert rvq.rvq_status_string(3) == "RVQ_ERR_WORKSPACE_TOO_SMALL"
    assert rvq.rvq_status_string(99) == "RVQ_ERR_UNKNOWN"


def test_prepared_size_layout(rvq):
    # norms [L][K rounded up to 128] fp32, then per level and 128-codeword
    # tile a 4 KB norm k-step and one 16 KB stage per 64 features (stage
    # counts 1, 2, 4, 8, 12, 16, 18, 20), the band bound's codebook terms per
    # tile [L][tiles][2] and per level [L][4] fp32, each part rounded up to
    # 256 bytes
    al = lambda v: (v + 255) // 256 * 256
    L, K, d = 8, 8192, 1152
    T = K // 128
    assert rvq.rvq_prepared_size(L, K, d) == (L * K * 4 + L * T * (4096 + 18 * 16384)
                                              + al(L * T * 8) + al(L * 16))
    # d = 70: 2 stages; rows not a multiple of 16 wide also get an fp32
    # codebook copy with row stride 80
    L, K, d = 3, 300, 70
    assert rvq.rvq_prepared_size(L, K, d) == (al(L * 384 * 4) + al(L * 3 * (4096 + 2 * 16384))
                                              + al(L * 3 * 8) + al(L * 16) + al(L * K * 80 * 4))
    # d = 640 needs 10 stages, padded to the next instantiated count (12)
    assert rvq.rvq_prepared_size(1, 128, 640) == al(128 * 4) + al(4096 + 12 * 16384) + al(8) + al(16)
    # rows wider than 1280 features take the exact fp32 encoder: no stages
    # (a norm block per tile is still reserved), the padded fp32 copy when
    # d is not a multiple of 16; up to 8192 features
    assert rvq.rvq_prepared_size(2, 300, 1281) == (al(2 * 384 * 4) + al(2 * 3 * 4096)
                                                   + al(2 * 3 * 8) + al(2 * 16)
                                                   + al(2 * 300 * 1296 * 4))
    assert rvq.rvq_prepared_size(1, 128, 8192) == al(128 * 4) + al(4096) + al(8) + al(16)
    with pytest.raises(rvq.RVQError) as e:
        rvq.rvq_prepared_size(1, 128, 8193)
    assert e.value.status == 2


def test_encode_workspace_size(rvq):
    # two fp32 residuals [n rounded up to 128][d rounded up to 16], repair
    # codes [n][L] int32 and, when some device (up to 1024 compute units)
    # may run n rows in the per-level split plan: 7 float4 records per row,
    # split and row half for min(tiles, ceil(2048 / row blocks)) splits, a
    # bf16 copy of the rows and (||r_b||^2, ||dr||^2) per row
    al = lambda v: (v + 255) // 256 * 256
    n, d, L, K = 1000, 64, 4, 256
    assert rvq.rvq_encode_workspace_size(n, d, L, K) == (
        2 * al(1024 * 64 * 4) + al(n * L * 4) + al(n * 2 * 2 * 7 * 16) + al(1024 * 64 * 2)
        + al(n * 8))
    assert rvq.rvq_encode_workspace_size(10, 70, 2, 300) == (
        2 * al(128 * 80 * 4) + al(10 * 2 * 4) + al(10 * 3 * 2 * 7 * 16) + al(128 * 80 * 2)
        + al(10 * 8))
    # 30,834 rows (241 row blocks): 9 splits at most
    n = 30834
    assert rvq.rvq_encode_workspace_size(n, 1152, 8, 8192) == (
        2 * al(30848 * 1152 * 4) + al(n * 8 * 4) + al(n * 9 * 2 * 7 * 16) + al(30848 * 1152 * 2)
        + al(n * 8))
    # rows wider than 1280 features use the same layout (the exact fp32
    # encoder keeps its codeword-slice minima in the split plan's records)
    n, d, L, K = 1000, 2048, 4, 256
    assert rvq.rvq_encode_workspace_size(n, d, L, K) == (
        2 * al(1024 * 2048 * 4) + al(n * L * 4) + al(n * 2 * 2 * 7 * 16) + al(1024 * 2048 * 2)
        + al(n * 8))
    # 80,000 rows fill any device: no split-plan buffers
    assert rvq.rvq_encode_workspace_size(80000, 1280, 16, 16384) == (
        2 * al(80000 * 1280 * 4) + al(80000 * 16 * 4))
    assert rvq.rvq_encode_workspace_size(0, d, L, K) == 256


def test_encode_codebook_level_limit(rvq):
    # one level of codewords (K x d rounded up to 16, fp32) must stay below 4 GiB
    assert rvq.rvq_encode_workspace_size(1, 1280, 1, 800_000) > 0
    with pytest.raises(rvq.RVQError) as e:
        rvq.rvq_encode_workspace_size(1, 1280, 1, 1 << 20)
    assert e.value.status == 2


@pytest.mark.parametrize("n,d,L,K,err", [
    (-1, 4, 1, 1, 1), (1, 0, 1, 1, 1), (1, 4, 0, 1, 1), (1, 4, 1, 0, 1),
    (1 << 26, 4, 1, 1, 2),
])
def test_shape_validation(rvq, n, d, L, K, err):
    with pytest.raises(rvq.RVQError) as e:
        rvq.rvq_encode_workspace_size(n, d, L, K)
    assert e.value.status == err


def _call_encode(rvq, **kw):
    lib = rvq.raw_library()
    a = dict(x=256, x_dtype=0, n=10, d=4, cb=256, prep=256, L=2, K=3, ids=256, res=None,
             ws=256, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    p = ctypes.c_void_p
    return lib.rvq_encode(p(a["x"]), a["x_dtype"], a["n"], a["d"], p(a["cb"]), p(a["prep"]),
                          a["L"], a["K"], p(a["ids"]), p(a["res"]) if a["res"] else None,
                          p(a["ws"]), a["ws_bytes"], p(a["stream"]) if a["stream"] else None)


def test_encode_rejects_bad_arguments_before_any_hip_call(rvq):
    # fake, never-dereferenced addresses: validation must fail first
    assert _call_encode(rvq, x_dtype=7) == 1
    assert _call_encode(rvq, x=0) == 1
    assert _call_encode(rvq, x=258) == 1        # fp32 rows not 4-byte aligned
    assert _call_encode(rvq, x=257, x_dtype=1) == 1   # bf16 rows not 2-byte aligned
    assert _call_encode(rvq, cb=0) == 1
    assert _call_encode(rvq, prep=128) == 1     # prepared must be 256-byte aligned
    assert _call_encode(rvq, ids=0) == 1
    assert _call_encode(rvq, res=258) == 1      # residual_out not 4-byte aligned
    assert _call_encode(rvq, ws=0) == 1
    assert _call_encode(rvq, ws_bytes=10) == 3
    assert "workspace" in rvq.raw_library().rvq_last_error().decode()
    # n == 0 is a no-op once the arguments are valid (no HIP call made)
    assert _call_encode(rvq, n=0, x=0, ids=0) == 0


def test_decode_and_stats_reject_bad_arguments(rvq):
    lib = rvq.raw_library()
    p = ctypes.c_void_p
    # levels out of range, bad dtype, L above the gather limit, null out
    assert lib.rvq_decode(p(256), 4, p(256), 2, 3, 4, 3, p(256), 1, None, None) == 1
    assert lib.rvq_decode(p(256), 4, p(256), 2, 3, 4, 2, p(256), 5, None, None) == 1
    assert lib.rvq_decode(p(256), 4, p(256), 65, 3, 4, 2, p(256), 1, None, None) == 2
    assert lib.rvq_decode(p(256), 4, p(256), 2, 3, 4, 2, None, 1, None, None) == 1
    assert lib.rvq_decode(None, 0, p(256), 2, 3, 4, 2, None, 1, None, None) == 0
    # level stats: hist required; x without codebooks; short workspace
    assert lib.rvq_level_stats(p(256), 4, 2, 3, None, None, 0, 1, None, None, None,
                               p(256), 1 << 20, None) == 1
    assert lib.rvq_level_stats(p(256), 4, 2, 3, p(256), p(256), 0, 4, None, p(256), None,
                               p(256), 1 << 20, None) == 1
    assert lib.rvq_level_stats(p(256), 4, 2, 3, p(256), None, 0, 1, None, None, None,
                               p(256), 1, None) == 3


def test_prepare_rejects_small_buffer(rvq):
    lib = rvq.raw_library()
    p = ctypes.c_void_p
    assert lib.rvq_prepare_codebooks(p(256), 2, 3, 4, p(256), 16, None) == 3
    assert lib.rvq_prepare_codebooks(None, 2, 3, 4, p(256), 1 << 20, None) == 1


def test_embed_tokens_rejects_bad_arguments(rvq):
    lib = rvq.raw_library()
    p = ctypes.c_void_p
    # (ids, is_visual, T, L, text, V, tables, K, D, table_dtype, out, out_dtype, bad, stream)
    args = [p(256), None, 4, 2, p(256), 5, p(256), 3, 8, 0, p(256), 1, None, None]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.rvq_embed_tokens(*a)
    assert call(a9=7) == 1                 # unknown table dtype
    assert call(a11=4) == 1                # unknown out dtype
    assert call(a3=0) == 1                 # L >= 1
    assert call(a3=65) == 2                # L above the gather limit
    assert call(a5=-1) == 1                # V >= 0
    assert call(a4=None) == 1              # text table required when V > 0
    assert call(a6=p(8)) == 1              # level tables misaligned
    assert call(a10=None) == 1             # out required when T > 0
    assert call(a12=p(2)) == 1             # bad_ids misaligned
    assert call(a2=-1) == 1                # T >= 0
    assert call(a2=0, a0=None, a10=None) == 0   # empty sequence: nothing to do
    assert call(a2=0, a4=None, a5=0) == 0       # no text table with V == 0


def test_stream_encode_rejects_bad_arguments(rvq):
    lib = rvq.raw_library()
    p = ctypes.c_void_p
    done = ctypes.c_int64(-1)
    need = ctypes.c_size_t()
    assert lib.rvq_stream_workspace_size(1000, 64, 4, 256, ctypes.byref(need)) == 0
    enc = ctypes.c_size_t()
    assert lib.rvq_encode_workspace_size(1000, 64, 4, 256, ctypes.byref(enc)) == 0
    al = lambda v: (v + 255) // 256 * 256
    # two row buffers (4-byte features), two ID buffers, the encoder's workspace
    assert need.value == 2 * al(1000 * 64 * 4) + 2 * al(1000 * 4 * 4) + enc.value
    assert lib.rvq_stream_workspace_size(0, 64, 4, 256, ctypes.byref(need)) == 1
    # (x, x_dtype, n, d, cb, prepared, L, K, ids, chunk_rows, first, max, cb, user, ws,
    #  ws_bytes, stream, chunks_done)
    args = [p(256), 0, 5000, 64, p(256), p(256), 4, 256, p(256), 1000, 0, 0, None, None,
            p(256), 1 << 30, None, ctypes.byref(done)]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.rvq_stream_encode(*a)
    assert call(a17=None) == 1             # chunks_done required
    assert call(a1=7) == 1                 # unknown x dtype
    assert call(a9=0) == 1                 # chunk_rows >= 1
    assert call(a10=-1) == 1               # first_chunk >= 0
    assert call(a0=None) == 1              # host rows required
    assert call(a14=p(8)) == 1             # workspace misaligned
    assert call(a15=1024) == 3             # workspace too small
    assert call(a2=0) == 0 and done.value == 0          # nothing to do
    assert call(a10=5) == 0 and done.value == 5         # every chunk already done
    assert call(a10=9) == 0 and done.value == 5         # resume point past the end


def test_decode_level_stats_rejects_bad_arguments(rvq):
    lib = rvq.raw_library()
    p = ctypes.c_void_p
    # (ids, n, cb, L, K, d, out, out_dtype, hist, x, x_dtype, msr, bad, ws, ws_bytes, stream)
    args = [p(256), 4, p(256), 2, 3, 4, p(256), 1, p(256), p(256), 0, p(256), None, p(256),
            1 << 20, None]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.rvq_decode_level_stats(*a)
    assert call(a7=5) == 1                 # unknown out dtype
    assert call(a10=9) == 1                # unknown x dtype
    assert call(a11=None) == 1             # msr required
    assert call(a6=None) == 1              # out required when n > 0
    assert call(a9=p(2)) == 1              # fp32 x not 4-byte aligned
    assert call(a9=p(1), a10=1) == 1       # bf16 x not 2-byte aligned
    assert call(a14=1) == 3                # workspace too small
    assert call(a3=65) == 2                # L above the gather limit


def test_mfma_rate_rejects_bad_arguments(rvq):
    lib = rvq.raw_library()
    p = ctypes.c_void_p
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    need = int(lib.rvq_mfma_rate_workspace_size(4))
    assert need == 4 * (16 + 256 * 4)
    assert lib.rvq_mfma_rate_workspace_size(0) == 0
    # fake, never-dereferenced addresses: validation fails before any HIP call
    call = lambda blocks, iters, ws, nbytes: lib.rvq_mfma_rate(
        blocks, iters, 0, p(ws) if ws else None, nbytes, None, ctypes.byref(tf), ctypes.byref(ghz))
    assert call(0, 100, 256, need) == 1
    assert call(70000, 100, 256, need) == 1
    assert call(4, 5, 256, need) == 1
    assert call(4, 100, 0, need) == 1
    assert call(4, 100, 260, need) == 1      # not 8-byte aligned
    assert call(4, 100, 256, need - 1) == 3
    assert lib.rvq_mfma_rate(4, 100, 0, p(256), need, None, None, ctypes.byref(ghz)) == 1
