"""The resumable ID cache (host code of the library, no GPU): round trip,
resume after a torn or corrupt tail, and rejection of mismatched headers and
out-of-order appends.  The record layout and CRC-32 are checked against an
independent reading of the file written with Python's zlib.crc32."""
import os
import struct
import zlib

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "residual_vector_quantization_rvq_amd", "librvq.so")

N, L, K, CH = 1000, 3, 500, 300     # 4 chunks: 300, 300, 300, 100 rows


@pytest.fixture(scope="module")
def rvq():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._builder().build()
    import residual_vector_quantization_rvq_amd as m
    return m


def _ids():
    return np.random.default_rng(3).integers(0, K, size=(N, L)).astype(np.int32)


def _write(rvq, path, ids, chunks):
    assert rvq.rvq_idcache_resume(path, N, L, K, CH) == 0
    for c in range(chunks):
        rvq.rvq_idcache_append(path, N, L, K, CH, c, ids[c * CH:(c + 1) * CH])


def test_round_trip_and_layout(rvq, tmp_path):
    path = str(tmp_path / "ids.bin")
    ids = _ids()
    _write(rvq, path, ids, 4)
    got, done = rvq.rvq_idcache_read(path, N, L, K, CH)
    assert done == 4
    np.testing.assert_array_equal(got, ids)
    # independent reading of the format: header, then records with CRC-32
    raw = open(path, "rb").read()
    assert raw[:8] == b"RVQIDC01"
    n, l, k, ch, crc = struct.unpack_from("<qiiqI", raw, 8)
    assert (n, l, k, ch) == (N, L, K, CH) and crc == zlib.crc32(raw[:32])
    off = 64
    for c in range(4):
        rows = min(CH, N - c * CH)
        rc, rr = struct.unpack_from("<qq", raw, off)
        body = 16 + rows * L * 4
        assert (rc, rr) == (c, rows)
        assert struct.unpack_from("<I", raw, off + body)[0] == zlib.crc32(raw[off:off + body])
        off += body + 8
    assert off == len(raw)
    assert rvq.rvq_idcache_resume(path, N, L, K, CH) == 4


def test_resume_drops_torn_and_corrupt_tails(rvq, tmp_path):
    path = str(tmp_path / "ids.bin")
    ids = _ids()
    _write(rvq, path, ids, 3)
    size3 = os.path.getsize(path)
    rec = 16 + CH * L * 4 + 8
    # a torn third record: two chunks survive and the file is cut back
    with open(path, "r+b") as f:
        f.truncate(size3 - 5)
    assert rvq.rvq_idcache_resume(path, N, L, K, CH) == 2
    assert os.path.getsize(path) == 64 + 2 * rec
    rvq.rvq_idcache_append(path, N, L, K, CH, 2, ids[2 * CH:3 * CH])
    rvq.rvq_idcache_append(path, N, L, K, CH, 3, ids[3 * CH:])
    got, done = rvq.rvq_idcache_read(path, N, L, K, CH)
    assert done == 4
    np.testing.assert_array_equal(got, ids)
    # one flipped ID byte in the second record: only the first chunk is valid
    with open(path, "r+b") as f:
        f.seek(64 + rec + 16 + 7)
        b = f.read(1)
        f.seek(64 + rec + 16 + 7)
        f.write(bytes([b[0] ^ 0x10]))
    got, done = rvq.rvq_idcache_read(path, N, L, K, CH)
    assert done == 1
    np.testing.assert_array_equal(got[:CH], ids[:CH])
    assert (got[CH:] == -1).all()
    assert rvq.rvq_idcache_resume(path, N, L, K, CH) == 1


def test_rejects_mismatch_and_out_of_order(rvq, tmp_path):
    path = str(tmp_path / "ids.bin")
    ids = _ids()
    _write(rvq, path, ids, 1)
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_resume(path, N, L, K, CH + 1)      # other chunking
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_read(path, N, L + 1, K, CH)        # other level count
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_append(path, N, L, K, CH, 2, ids[2 * CH:3 * CH])   # skips chunk 1
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_append(path, N, L, K, CH, 0, ids[:CH])             # chunk 0 again
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_append(path, N, L, K, CH, 4, ids[:CH])             # no such chunk
    other = str(tmp_path / "other.bin")
    with open(other, "wb") as f:
        f.write(b"not an ID cache" + bytes(100))
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_resume(other, N, L, K, CH)
    with pytest.raises(rvq.RVQError):
        rvq.rvq_idcache_read(str(tmp_path / "missing.bin"), N, L, K, CH)
    # an empty cache (n == 0) has no chunks
    empty = str(tmp_path / "empty.bin")
    assert rvq.rvq_idcache_resume(empty, 0, L, K, CH) == 0
    got, done = rvq.rvq_idcache_read(empty, 0, L, K, CH)
    assert done == 0 and got.shape == (0, L)
