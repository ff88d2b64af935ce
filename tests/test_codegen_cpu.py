"""Compiles the encoder's device code to gfx950 assembly (no GPU needed) and
checks it for reads of inline-asm MFMA results that the compiler issued too
early (see asm_scan)."""
import concurrent.futures
import glob
import os
import subprocess
import tempfile

import pytest

import asm_scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "residual_vector_quantization_rvq_amd", "csrc")


def _device_asm(src: str, out_dir: str) -> str:
    import __graft_entry__
    _build = __graft_entry__._builder()
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    subprocess.run([_build.HIPCC, *_build.FLAGS, "-S", "--cuda-device-only", src, "-o", out],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def encoder_asm():
    srcs = sorted(glob.glob(os.path.join(CSRC, "encode_s*.hip")))
    assert srcs
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            return list(ex.map(lambda s: _device_asm(s, d), srcs))


def test_no_early_reads_of_mfma_results(encoder_asm):
    kernels = {}
    for asm in encoder_asm:
        kernels.update(asm_scan.kernel_bodies(asm, "_ZN3rvq12sweep_kernel"))
    # every stage count, fused and split
    assert len(kernels) >= 16, sorted(kernels)
    bad = {name: hits for name, body in kernels.items()
           if (hits := asm_scan.early_mfma_reads(body))}
    assert not bad, {k: v[:3] for k, v in bad.items()}


def test_scanner_flags_an_early_copy():
    # a register copy two instructions after an asm MFMA must be reported,
    # one after the explicit wait must not
    body = [
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]",
        ";;#ASMEND",
        "s_add_u32 s4, s4, 16",
        "v_mov_b64_e32 v[32:33], v[0:1]",
        ";;#ASMSTART",
        "s_nop 7",
        "s_nop 7",
        "s_nop 7",
        ";;#ASMEND",
        "v_mov_b64_e32 v[34:35], v[2:3]",
        "s_endpgm",
    ]
    hits = asm_scan.early_mfma_reads(body)
    assert [h[0] for h in hits] == [5]
