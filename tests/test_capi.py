"""The C ABI from plain C: the header compiles as C99 and as C++17, and the
C test program (tests/capi/capi_roundtrip.c, built by the package build
against libonebit.so and the HIP runtime only) links and starts.  Without a
GPU it reports so (exit 2); with one, tests/test_gpu_capi.py runs it."""

import os
import shutil
import subprocess

import pytest

from momentum_compression_amd import build as B

HEADER = os.path.join(B.INCLUDE, "onebit.h")


def _rocm_include():
    return os.path.join(B._rocm(), "include")


@pytest.mark.parametrize("lang,std,cc", [("c", "c99", "gcc"), ("c++", "c++17", "g++")])
def test_header_compiles(tmp_path, lang, std, cc):
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} not available")
    src = tmp_path / ("h.c" if lang == "c" else "h.cpp")
    src.write_text('#include "onebit.h"\nint main(void) { return (int)onebit_workspace_bytes(0, 1, 0); }\n')
    res = subprocess.run([cc, "-x", lang, f"-std={std}", "-Wall", "-Wextra", "-Werror",
                          "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", f"-I{_rocm_include()}",
                          f"-I{B.INCLUDE}", str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_c_program_links_and_starts():
    if not os.path.exists(B.CAPI_BIN):
        pytest.fail("the C test program is not built: run python -m momentum_compression_amd.build")
    res = subprocess.run([B.CAPI_BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode in (0, 2), res.stdout + res.stderr
    assert res.stdout.strip() in ("capi ok", "no GPU")


def test_struct_mirror_matches_the_c_compiler(tmp_path):
    """Every field offset and the size of onebit_frozen_v_args as gcc lays
    them out from the header, against the binding's ctypes mirror."""
    import ctypes

    from momentum_compression_amd import onebit as ob

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    names = [f[0] for f in ob.FrozenVArgs._fields_]
    lines = "\n".join(f'    printf("{n} %zu\\n", offsetof(onebit_frozen_v_args, {n}));' for n in names)
    src = tmp_path / "off.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "onebit.h"\nint main(void) {\n'
                   f'{lines}\n    printf("sizeof %zu\\n", sizeof(onebit_frozen_v_args));\n'
                   '    return 0;\n}\n')
    exe = tmp_path / "off"
    res = subprocess.run(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", f"-I{_rocm_include()}",
                          f"-I{B.INCLUDE}", str(src), "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                       text=True).stdout.splitlines())
    for n in names:
        assert int(out[n]) == getattr(ob.FrozenVArgs, n).offset, n
    assert int(out["sizeof"]) == ctypes.sizeof(ob.FrozenVArgs)
