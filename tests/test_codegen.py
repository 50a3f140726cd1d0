"""Properties of the gfx950 code the build emits (device assembly of each
kernel source, compiled with the build's own flags): no packed-fp32 vector
arithmetic (the flags switch its selection off, and every fp32 operation
must round on its own), and no writes through the scalar data cache (all
stores are vector stores).  Runs on the host; needs hipcc."""

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from momentum_compression_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists(
    "/opt/rocm/bin/hipcc"), reason="hipcc not available")

KERNEL_SOURCES = [s for s in B.SOURCES if s != "api.hip"] + [B.PROBE_SRC]
PACKED_FP32 = re.compile(r"^\s+v_pk_(add|mul|fma)_f32\b", re.M)
SCALAR_WRITE = re.compile(r"^\s+s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb)", re.M)
KERNEL = re.compile(r"^\s+\.amdhsa_kernel\s+(\S+)", re.M)


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm")

    def one(src):
        dst = out / (src + ".s")
        cmd = [B.hipcc(), *B.FLAGS, "--cuda-device-only", "-S",
               os.path.join(B.CSRC, src), "-o", str(dst)]
        subprocess.run(cmd, check=True, capture_output=True)
        return src, dst.read_text()

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(one, KERNEL_SOURCES))


def test_every_source_emits_kernels(device_asm):
    for src, text in device_asm.items():
        assert KERNEL.search(text), f"{src}: no kernel in the device assembly"


def test_no_packed_fp32_arithmetic(device_asm):
    for src, text in device_asm.items():
        m = PACKED_FP32.search(text)
        assert m is None, f"{src}: {m.group(0).strip()}"


def test_no_scalar_cache_writes(device_asm):
    for src, text in device_asm.items():
        m = SCALAR_WRITE.search(text)
        assert m is None, f"{src}: {m.group(0).strip()}"
