"""The C interface from plain C: include/attn.h compiles as C11 without warnings, and a
C program linked to libattn.so runs its host-side calls (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

import exact_attention_prefill_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_and_library_from_c(tmp_path):
    src = os.path.join(ROOT, "tests", "c", "abi_host.c")
    exe = str(tmp_path / "abi_host")
    libdir = os.path.dirname(ea.LIB_PATH)
    subprocess.run(
        ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), src, "-o", exe,
         "-L", libdir, "-lattn", f"-Wl,-rpath,{libdir}"],
        check=True, capture_output=True, text=True,
    )
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr
