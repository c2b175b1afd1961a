"""The boundary from plain C: a C99 program that includes only
include/q4_0.h and links libq4amd.so (no Python, no torch) sizes buffers and
gets validation errors back.  Runs without a GPU: every call it makes fails
validation (or is M = 0) before the library touches the HIP runtime."""

import os
import shutil
import subprocess

import pytest

import q4_weight_only_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "q4_0.h"

int main(void) {
    int bad = 0;
    /* 131072 x 3072: 216 MiB, the GGUF size (18 bytes per 32 weights) */
    if (q4_0_packed_bytes(131072, 3072) != (size_t)131072 * 3072 / 32 * 18) bad |= 1;
    if (q4_0_packed_bytes(16, 48) != 0) bad |= 2;                     /* K % 32 != 0 */
    if (strlen(q4_status_str(Q4_ERR_SHAPE)) == 0) bad |= 4;
    /* validation failures, no device memory involved */
    void *fake = (void *)(uintptr_t)0x10000;
    if (q4_0_linear(fake, 1, fake, 16, 48, (float *)fake, NULL) != Q4_ERR_SHAPE) bad |= 8;
    if (q4_0_linear(NULL, 1, fake, 16, 64, (float *)fake, NULL) != Q4_ERR_NULL) bad |= 16;
    if (q4_0_linear(fake, 0, fake, 16, 64, (float *)fake, NULL) != Q4_OK) bad |= 32;  /* M = 0: no-op */
    q4_0_segment segs[2] = {{fake, 16, (float *)fake}, {fake, 0, (float *)fake}};
    if (q4_0_linear_multi(fake, 1, 64, segs, 2, NULL) != Q4_ERR_SHAPE) bad |= 64;
    if (q4_0_linear_multi(fake, 1, 64, segs, 9, NULL) != Q4_ERR_SEGMENTS) bad |= 128;
    int64_t ns[1] = {4096};
    const char *name = q4_0_linear_kernel(1, 3072, ns, 1);
    if (strncmp(name, "gemv_kernel<", 12) != 0) bad |= 256;
    printf("c consumer: %s %d\n", name, bad);
    return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_plain_c_program_uses_the_abi(tmp_path):
    lib = q4.library_path()
    if not os.path.exists(lib):
        subprocess.run(["python", "-m", "q4_weight_only_amd.build"], check=True, cwd=ROOT)
    src = tmp_path / "consumer.c"
    exe = tmp_path / "consumer"
    src.write_text(PROGRAM)
    libdir = os.path.dirname(lib)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
                    str(src), "-o", str(exe), f"-L{libdir}", "-l:libq4amd.so", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    assert "c consumer: gemv_kernel<" in out.stdout
