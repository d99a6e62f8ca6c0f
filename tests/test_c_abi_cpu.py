"""The boundary as a C program sees it, on the CPU: include/atlas.h compiles as
strict C11, a C program links libatlas.so, and the host-only entry points
(version, status strings, the FLOP helper, argument checks that return before
any HIP call) behave as the header states."""
import os
import shutil
import subprocess

import pytest

import windowed_global_local_amd as atlas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "atlas.h"

int main(void)
{
    const atlas_dim3 grid = {21, 136, 240}, cube = {3, 17, 24}, gp = {21, 30, 52};
    const atlas_dim3 bad_cube = {5, 17, 24};          /* 5 does not divide 21 */
    double f;
    int rc;
    if (atlas_version() != 10200) { puts("version"); return 1; }
    if (atlas_status_string(ATLAS_OK) == NULL || atlas_status_string(12345) == NULL) { puts("status"); return 1; }
    /* useful FLOPs of the 4K workload: 4 D heads (N (V + G) + G^2) */
    f = atlas_hier_attn_useful_flops(grid, cube, gp, 40, 128);
    if (fabs(f - 4.0 * 128 * 40 * (685440.0 * (1224 + 32760) + 32760.0 * 32760)) > 1.0) { puts("flops"); return 1; }
    /* argument checks return before any HIP call */
    rc = atlas_cube_reorder(NULL, NULL, grid, cube, 40, 128, ATLAS_BF16, NULL);
    if (rc != ATLAS_ERR_NULL) { printf("null %d\n", rc); return 1; }
    rc = atlas_cube_reorder((void *)0x7f0000000000, (const void *)0x7f1000000000, grid, bad_cube, 40, 128,
                            ATLAS_BF16, NULL);
    if (rc != ATLAS_ERR_SHAPE) { printf("shape %d\n", rc); return 1; }
    rc = atlas_cube_reorder((void *)0x7f0000000000, (const void *)0x7f1000000000, grid, cube, 40, 96,
                            ATLAS_BF16, NULL);
    if (rc != ATLAS_ERR_UNSUPPORTED) { printf("head_dim %d\n", rc); return 1; }
    rc = atlas_cube_reorder((void *)0x7f0000000000, (const void *)0x7f1000000000, grid, cube, 40, 128, 7, NULL);
    if (rc != ATLAS_ERR_DTYPE) { printf("dtype %d\n", rc); return 1; }
    if (atlas_last_hip_error() != 0) { puts("hip error"); return 1; }
    puts("ok");
    return 0;
}
"""


def test_header_compiles_as_c11_and_links(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(atlas.LIB_PATH):
        pytest.skip("libatlas.so not built")
    src = tmp_path / "use_atlas.c"
    src.write_text(C_SRC)
    exe = tmp_path / "use_atlas"
    libdir = os.path.dirname(atlas.LIB_PATH)
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    atlas.LIB_PATH, "-Wl,-rpath," + libdir, "-lm"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
