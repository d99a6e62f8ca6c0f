"""The C boundary used from a plain C program on the GPU, with no Python or
PyTorch in the process: device memory from the HIP runtime, then
atlas_cube_reorder and atlas_cube_unorder on fp32 rows, checked bit for bit
(each cube-order row is the raster row of the permutation of "Technische
Samenvatting: AtlasVid", Methodologie 1, Fase 2, re-derived in the program;
the unorder restores the input)."""
import os
import shutil
import subprocess

import pytest

import windowed_global_local_amd as atlas

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"

C_SRC = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "atlas.h"

#define HIPCHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    printf("hip error %d at line %d\n", (int)e_, __LINE__); return 1; } } while (0)

int main(void)
{
    const atlas_dim3 grid = {6, 12, 16}, cube = {3, 6, 8};
    const int32_t heads = 3, hd = 64;
    const int64_t T = 6, H = 12, W = 16, ct = 3, ch = 6, cw = 8;
    const int64_t N = T * H * W, V = ct * ch * cw, nH = H / ch, nW = W / cw;
    const int64_t row = (int64_t)heads * hd;
    const size_t bytes = (size_t)(N * row) * sizeof(float);
    float *src = malloc(bytes), *out = malloc(bytes), *back = malloc(bytes);
    void *d_src = NULL, *d_dst = NULL, *d_back = NULL;
    int64_t i, p;
    int rc;
    if (!src || !out || !back) { puts("malloc"); return 1; }
    for (i = 0; i < N * row; ++i)
        src[i] = (float)(i % 9973) * 0.25f - 17.0f;
    HIPCHECK(hipMalloc(&d_src, bytes));
    HIPCHECK(hipMalloc(&d_dst, bytes));
    HIPCHECK(hipMalloc(&d_back, bytes));
    HIPCHECK(hipMemcpy(d_src, src, bytes, hipMemcpyHostToDevice));
    rc = atlas_cube_reorder(d_dst, d_src, grid, cube, heads, hd, ATLAS_F32, NULL);
    if (rc != ATLAS_OK) { printf("reorder: %s\n", atlas_status_string(rc)); return 1; }
    rc = atlas_cube_unorder(d_back, d_dst, grid, cube, heads, hd, ATLAS_F32, NULL);
    if (rc != ATLAS_OK) { printf("unorder: %s\n", atlas_status_string(rc)); return 1; }
    HIPCHECK(hipDeviceSynchronize());
    HIPCHECK(hipMemcpy(out, d_dst, bytes, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(back, d_back, bytes, hipMemcpyDeviceToHost));
    for (p = 0; p < N; ++p) {
        /* cube c = p / V in raster order over the cube grid, offset o = p % V
           in raster order inside the cube */
        const int64_t c = p / V, o = p % V;
        const int64_t a = c / (nH * nW), b = (c / nW) % nH, e = c % nW;
        const int64_t dt = o / (ch * cw), dh = (o / cw) % ch, dw = o % cw;
        const int64_t r = ((a * ct + dt) * H + (b * ch + dh)) * W + (e * cw + dw);
        if (memcmp(out + p * row, src + r * row, (size_t)row * sizeof(float)) != 0) {
            printf("reorder row %lld\n", (long long)p);
            return 1;
        }
    }
    if (memcmp(back, src, bytes) != 0) { puts("round trip"); return 1; }
    HIPCHECK(hipFree(d_src));
    HIPCHECK(hipFree(d_dst));
    HIPCHECK(hipFree(d_back));
    free(src); free(out); free(back);
    puts("ok");
    return 0;
}
"""


def test_c_program_reorder_round_trip(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    assert os.path.exists(atlas.LIB_PATH), "libatlas.so not built"
    src = tmp_path / "reorder_c.c"
    src.write_text(C_SRC)
    exe = tmp_path / "reorder_c"
    libdir = os.path.dirname(atlas.LIB_PATH)
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    str(src), "-o", str(exe), atlas.LIB_PATH, "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                   check=True, capture_output=True, text=True)
    print("[gpu-test] C program: reorder + unorder, 1152 tokens x 3 heads x 64, fp32", flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
