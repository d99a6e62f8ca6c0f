"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

Only invalid argument sets are passed here (with fake but aligned pointer
values): validation returns before anything is launched, so no pointer is ever
dereferenced.  Valid calls live in the GPU tests.
"""
import math
import os
import re

import numpy as np
import pytest

import windowed_global_local_amd as atlas
from windowed_global_local_amd import Dim3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "atlas.h")

P = 0x7F0000000000          # fake, 16-byte aligned "device" addresses
Q = P + (1 << 36)
R = P + (2 << 36)
BF16, F32 = 0, 1
OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_ALIAS, E_HIP, E_VALUE, E_SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)

GRID, CUBE, GP = Dim3(4, 8, 8), Dim3(2, 4, 4), Dim3(2, 4, 4)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(atlas.LIB_PATH):
        pytest.skip("libatlas.so not built")
    return atlas.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(atlas_\w+)\s*\(", src)))


def test_header_and_exports(lib):
    names = declared_functions()
    assert set(names) == set(atlas.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.atlas_version() == 10200
    assert lib.atlas_last_hip_error() == 0
    for code in (OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_ALIAS, E_HIP, E_VALUE, E_SCRATCH, 99):
        assert isinstance(lib.atlas_status_string(code), bytes)


def test_useful_flops_closed_forms(lib):
    f = lib.atlas_hier_attn_useful_flops
    # full attention (one cube = whole volume, no proxy) costs O((HWT)^2):
    # doubling T, H and W multiplies it by 64 ("Technische Samenvatting:
    # AtlasVid", Probleemstelling)
    a = f(Dim3(3, 4, 5), Dim3(3, 4, 5), Dim3(0, 0, 0), 2, 64)
    b = f(Dim3(6, 8, 10), Dim3(6, 8, 10), Dim3(0, 0, 0), 2, 64)
    assert b / a == 64.0
    assert a == 4 * 64 * 2 * 60 ** 2
    # with a fixed proxy the hierarchical cost is linear in the detail tokens
    g = Dim3(21, 30, 52)
    c1 = f(Dim3(21, 136, 240), Dim3(3, 17, 24), g, 40, 128)
    c2 = f(Dim3(42, 136, 240), Dim3(3, 17, 24), g, 40, 128)
    N, V, G = 21 * 136 * 240, 3 * 17 * 24, 21 * 30 * 52
    assert c2 - c1 == pytest.approx(4 * 128 * 40 * N * (V + G), rel=1e-15)
    assert c1 == pytest.approx(4.9904e14, rel=1e-4)
    assert f(Dim3(21, 45, 80), Dim3(3, 15, 16), Dim3(6, 23, 40), 40, 128) == pytest.approx(1.0285e13, rel=1e-4)
    assert f(Dim3(4, 8, 8), Dim3(2, 4, 4), Dim3(2, 4, 4), 2, 64) == pytest.approx(8.913e6, rel=1e-4)
    assert f(Dim3(4, 8, 8), Dim3(3, 4, 4), Dim3(0, 0, 0), 2, 64) == -1.0


def test_reorder_validation(lib):
    for fn in (lib.atlas_cube_reorder, lib.atlas_cube_unorder):
        assert fn(None, P, GRID, CUBE, 2, 64, BF16, None) == E_NULL
        assert fn(P, None, GRID, CUBE, 2, 64, BF16, None) == E_NULL
        assert fn(Q, P, GRID, Dim3(3, 4, 4), 2, 64, BF16, None) == E_SHAPE    # 3 does not divide 4
        assert fn(Q, P, Dim3(0, 8, 8), CUBE, 2, 64, BF16, None) == E_SHAPE
        assert fn(Q, P, GRID, Dim3(-2, 4, 4), 2, 64, BF16, None) == E_SHAPE
        assert fn(Q, P, GRID, CUBE, 0, 64, BF16, None) == E_SHAPE
        assert fn(Q, P, GRID, CUBE, 2, 64, 2, None) == E_DTYPE
        assert fn(Q, P, GRID, CUBE, 2, 96, BF16, None) == E_UNSUP
        assert fn(Q + 8, P, GRID, CUBE, 2, 64, BF16, None) == E_ALIGN
        assert fn(Q, P + 4, GRID, CUBE, 2, 64, F32, None) == E_ALIGN
        assert fn(P, P, GRID, CUBE, 2, 64, BF16, None) == E_ALIAS
        assert fn(P + 256 * 2 * 64 * 2 - 16, P, GRID, CUBE, 2, 64, BF16, None) == E_ALIAS
        # element count past 2^31 tokens
        assert fn(Q, P, Dim3(65536, 65536, 2), Dim3(1, 1, 1), 1, 64, BF16, None) == E_SHAPE


def test_rope_validation(lib):
    fn = lib.atlas_rope3d
    assert fn(None, None, GRID, CUBE, GP, 4.0, 1e4, 2, 64, BF16, None) == E_NULL
    assert fn(P, Q, GRID, CUBE, Dim3(0, 0, 0), 4.0, 1e4, 2, 64, BF16, None) == E_SHAPE
    assert fn(P, Q, GRID, CUBE, Dim3(2, 0, 4), 4.0, 1e4, 2, 64, BF16, None) == E_SHAPE
    assert fn(P, Q, GRID, CUBE, GP, float("nan"), 1e4, 2, 64, BF16, None) == E_VALUE
    assert fn(P, Q, GRID, CUBE, GP, 0.0, 1e4, 2, 64, BF16, None) == E_VALUE
    assert fn(P, Q, GRID, CUBE, GP, 4.0, 1.0, 2, 64, BF16, None) == E_VALUE
    assert fn(P, Q, GRID, CUBE, GP, 4.0, float("inf"), 2, 64, BF16, None) == E_VALUE
    assert fn(P, Q, GRID, CUBE, GP, 4.0, 1e4, 2, 128 + 64, BF16, None) == E_UNSUP
    assert fn(P, Q, GRID, CUBE, GP, 4.0, 1e4, 2, 64, 5, None) == E_DTYPE
    assert fn(P + 2, Q, GRID, CUBE, GP, 4.0, 1e4, 2, 64, BF16, None) == E_ALIGN
    assert fn(P, P + 64, GRID, CUBE, GP, 4.0, 1e4, 2, 64, BF16, None) == E_ALIAS


def test_attention_validation(lib):
    fn = lib.atlas_hier_attn

    def call(od=R, og=R + (1 << 30), qd=P, kd=P + (1 << 30), vd=P + (2 << 30), qg=Q, kg=Q + (1 << 30),
             vg=Q + (2 << 30), grid=GRID, cube=CUBE, gp=GP, heads=2, hd=64, scale=0.0, dt=BF16):
        return fn(od, og, qd, kd, vd, qg, kg, vg, grid, cube, gp, heads, hd, scale, dt, None)

    assert call(od=None) == E_NULL
    assert call(kd=None) == E_NULL
    assert call(og=None) == E_NULL
    assert call(vg=None) == E_NULL
    assert call(grid=Dim3(4, 8, 9)) == E_SHAPE
    assert call(gp=Dim3(1, 0, 1)) == E_SHAPE
    assert call(hd=32) == E_UNSUP
    assert call(dt=-1) == E_DTYPE
    assert call(scale=float("nan")) == E_VALUE
    assert call(scale=float("-inf")) == E_VALUE
    assert call(qd=P + 8) == E_ALIGN
    assert call(vg=Q + 4) == E_ALIGN
    assert call(od=P) == E_ALIAS                 # output on top of q_d
    assert call(og=Q + (2 << 30) + 64) == E_ALIAS   # output inside v_g
    assert call(og=R + 128) == E_ALIAS           # outputs overlap each other


def test_python_binding_requires_gpu_tensors():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("CPU-only check")
    x = torch.zeros(256, 2, 64)
    with pytest.raises(ValueError):
        atlas.atlas_cube_reorder(torch.empty_like(x), x, (4, 8, 8), (2, 4, 4))


def test_error_type_carries_status(lib):
    err = atlas.AtlasError(E_SHAPE, "x")
    assert err.code == E_SHAPE and "ATLAS_ERR_SHAPE" in str(err)
    assert math.isfinite(lib.atlas_hier_attn_useful_flops(GRID, CUBE, GP, 2, 64))


def test_attention_fwd_lse_validation(lib):
    fn = lib.atlas_hier_attn_fwd
    G1 = 1 << 30

    def call(od=R, og=R + G1, ld=R + 2 * G1, lg=R + 3 * G1, qd=P, kd=P + G1, vd=P + 2 * G1, qg=Q,
             kg=Q + G1, vg=Q + 2 * G1, gp=GP):
        return fn(od, og, ld, lg, qd, kd, vd, qg, kg, vg, GRID, CUBE, gp, 2, 64, 0.0, BF16, None)

    assert call(ld=None) == E_NULL
    assert call(lg=None) == E_NULL
    assert call(ld=R + 2 * G1 + 4) == E_ALIGN
    assert call(ld=P + 64) == E_ALIAS             # lse on top of q_d
    assert call(lg=R + 2 * G1 + 512) == E_ALIAS   # the two lse buffers overlap
    assert call(ld=R + 64) == E_ALIAS             # lse inside o_detail


def test_attention_bwd_validation(lib):
    fn = lib.atlas_hier_attn_bwd
    N, G, heads, hd = 256, 32, 2, 64
    need = lib.atlas_hier_attn_bwd_workspace_bytes(GRID, CUBE, GP, heads, hd)
    assert need == 4 * heads * (N + G)
    assert lib.atlas_hier_attn_bwd_workspace_bytes(GRID, CUBE, Dim3(0, 0, 0), heads, hd) == 4 * heads * N
    assert lib.atlas_hier_attn_bwd_workspace_bytes(GRID, Dim3(3, 4, 4), GP, heads, hd) == -1
    G1 = 1 << 30
    base = {"dqd": R, "dkd": R + G1, "dvd": R + 2 * G1, "dqg": R + 3 * G1, "dkg": R + 4 * G1,
            "dvg": R + 5 * G1, "qd": P, "kd": P + G1, "vd": P + 2 * G1, "qg": P + 3 * G1,
            "kg": P + 4 * G1, "vg": P + 5 * G1, "od": Q, "og": Q + G1, "dod": Q + 2 * G1,
            "dog": Q + 3 * G1, "ld": Q + 4 * G1, "lg": Q + 5 * G1, "ws": Q + 6 * G1}
    order = ("dqd", "dkd", "dvd", "dqg", "dkg", "dvg", "qd", "kd", "vd", "qg", "kg", "vg", "od",
             "og", "dod", "dog", "ld", "lg", "ws")

    def call(ws_bytes=need, gp=GP, hd=hd, scale=0.0, dt=BF16, **kw):
        p = dict(base)
        p.update(kw)
        return fn(*(p[k] for k in order), ws_bytes, GRID, CUBE, gp, heads, hd, scale, dt, None)

    assert call(dqd=None) == E_NULL
    assert call(ws=None) == E_NULL
    assert call(ld=None) == E_NULL
    assert call(lg=None) == E_NULL
    assert call(dog=None) == E_NULL
    assert call(gp=Dim3(0, 1, 1)) == E_SHAPE
    assert call(hd=32) == E_UNSUP
    assert call(dt=7) == E_DTYPE
    assert call(scale=float("nan")) == E_VALUE
    assert call(ws_bytes=need - 4) == E_VALUE
    assert call(kd=P + G1 + 8) == E_ALIGN
    assert call(ws=Q + 6 * G1 + 4) == E_ALIGN
    assert call(dqd=P) == E_ALIAS                     # dq_d on top of q_d
    assert call(dkg=R + 3 * G1 + 64) == E_ALIAS       # two outputs overlap
    assert call(ws=Q + 4 * G1 + 16) == E_ALIAS        # workspace inside lse_detail
    assert call(ws=R + 2 * G1 + 16) == E_ALIAS        # workspace inside dv_d


def test_attention_bwd_noalloc_validation(lib):
    """The no-allocation backward checks every argument (and the size of its
    fixed array) before it looks up that array or launches anything."""
    fn = lib.atlas_hier_attn_bwd_noalloc
    heads, hd = 2, 64
    G1 = 1 << 30
    base = [R, R + G1, R + 2 * G1, R + 3 * G1, R + 4 * G1, R + 5 * G1, P, P + G1, P + 2 * G1,
            P + 3 * G1, P + 4 * G1, P + 5 * G1, Q, Q + G1, Q + 2 * G1, Q + 3 * G1, Q + 4 * G1,
            Q + 5 * G1]

    def call(grid=GRID, cube=CUBE, gp=GP, heads=heads, hd=hd, scale=0.0, dt=BF16, **kw):
        p = list(base)
        for i, v in kw.items():
            p[int(i[1:])] = v
        return fn(*p, grid, cube, gp, heads, hd, scale, dt, None)

    assert call(a0=None) == E_NULL
    assert call(a16=None) == E_NULL
    assert call(gp=Dim3(0, 1, 1)) == E_SHAPE
    assert call(cube=Dim3(3, 4, 4)) == E_SHAPE
    assert call(hd=32) == E_UNSUP
    assert call(dt=7) == E_DTYPE
    assert call(scale=float("inf")) == E_VALUE
    assert call(a7=P + G1 + 8) == E_ALIGN
    assert call(a0=P) == E_ALIAS
    # long 4K latent grid with 40 heads: 4 * 40 * (N + G) bytes exceed the array
    big = dict(grid=Dim3(42, 136, 240), cube=Dim3(3, 17, 24), gp=Dim3(21, 30, 52), heads=40, hd=128)
    assert (lib.atlas_hier_attn_bwd_workspace_bytes(big["grid"], big["cube"], big["gp"], 40, 128)
            > atlas.NOALLOC_SCRATCH_BYTES)
    assert call(**big) == E_SCRATCH
    # the 4K latent grid fits
    fit = dict(grid=Dim3(21, 136, 240), cube=Dim3(3, 17, 24), gp=Dim3(21, 30, 52))
    assert (lib.atlas_hier_attn_bwd_workspace_bytes(fit["grid"], fit["cube"], fit["gp"], 40, 128)
            <= atlas.NOALLOC_SCRATCH_BYTES)
    assert lib.atlas_last_hip_error() == 0


@pytest.mark.parametrize("grid,cube,gp,rt", [
    ((4, 4, 4), (2, 2, 2), (2, 2, 2), 2.0),
    ((21, 45, 80), (3, 15, 16), (6, 23, 40), 4.0),
    ((21, 136, 240), (3, 17, 24), (21, 30, 52), 4.0),
    ((8, 270, 480), (2, 27, 24), (8, 30, 52), 4.0),
    ((8, 270, 480), (4, 10, 32), (8, 30, 52), 4.0),
    ((3, 4, 10), (1, 2, 5), (3, 4, 10), 1.0),
    ((1, 1, 6), (1, 1, 3), (1, 1, 4), 1.5),
])
def test_aligned_subset_equals_oracle(grid, cube, gp, rt):
    """The library's co-located lists (per-cube index ranges) equal the
    oracle's brute-force scan over (cube, proxy token) pairs."""
    import oracle
    goff, gidx = atlas.atlas_aligned_subset(grid, cube, gp, rt)
    ro, ri = oracle.aligned_subset(grid, cube, gp, rt)
    np.testing.assert_array_equal(goff.astype(np.int64), ro)
    np.testing.assert_array_equal(gidx, ri)


def test_aligned_subset_errors(lib):
    f = lib.atlas_aligned_subset
    assert f(None, None, 0, GRID, Dim3(3, 4, 4), GP, 4.0) == E_SHAPE
    assert f(None, None, 0, GRID, CUBE, Dim3(1, 0, 1), 4.0) == E_SHAPE
    assert f(None, None, 0, GRID, CUBE, GP, 0.0) == E_VALUE
    assert f(None, None, 0, GRID, CUBE, GP, float("nan")) == E_VALUE
    n = f(None, None, 0, GRID, CUBE, GP, 4.0)
    assert n >= 1
    goff = np.empty(GRID.t * GRID.h * GRID.w // (CUBE.t * CUBE.h * CUBE.w) + 1, dtype=np.int32)
    gidx = np.empty(n, dtype=np.int32)
    assert f(goff.ctypes.data, gidx.ctypes.data, n - 1, GRID, CUBE, GP, 4.0) == E_VALUE
    assert f(goff.ctypes.data, gidx.ctypes.data, n, GRID, CUBE, GP, 4.0) == n


def test_subset_attention_validation(lib):
    fn = lib.atlas_hier_attn_subset
    G1 = 1 << 30

    def call(goff=Q + 8 * G1, gidx=Q + 9 * G1, n=4, od=R, gp=GP, hd=64):
        return fn(od, R + G1, P, P + G1, P + 2 * G1, Q, Q + G1, Q + 2 * G1, goff, gidx, n,
                  GRID, CUBE, gp, 2, hd, 0.0, BF16, None)

    assert call(goff=None) == E_NULL
    assert call(gidx=None) == E_NULL
    assert call(n=-1) == E_VALUE
    assert call(goff=Q + 8 * G1 + 2) == E_ALIGN
    assert call(goff=R + 64) == E_ALIAS          # offsets inside o_detail
    assert call(gp=Dim3(1, 0, 1)) == E_SHAPE
    assert call(hd=96) == E_UNSUP


def test_subset_fwd_lse_validation(lib):
    fn = lib.atlas_hier_attn_subset_fwd
    G1 = 1 << 30

    def call(goff=Q + 8 * G1, gidx=Q + 9 * G1, n=4, ld=R + 2 * G1, lg=R + 3 * G1, od=R):
        return fn(od, R + G1, ld, lg, P, P + G1, P + 2 * G1, Q, Q + G1, Q + 2 * G1, goff, gidx, n,
                  GRID, CUBE, GP, 2, 64, 0.0, BF16, None)

    assert call(goff=None) == E_NULL
    assert call(n=-1) == E_VALUE
    assert call(gidx=Q + 9 * G1 + 1) == E_ALIGN
    assert call(gidx=R + 128) == E_ALIAS         # indices inside o_detail
    assert call(ld=None) == E_NULL
    assert call(ld=R + 64) == E_ALIAS            # lse inside o_detail


def test_subset_bwd_validation(lib):
    fn = lib.atlas_hier_attn_subset_bwd
    N, G, heads, hd = 256, 32, 2, 64
    need = lib.atlas_hier_attn_subset_bwd_workspace_bytes(GRID, CUBE, GP, heads, hd)
    # D rows rounded up to 256 bytes, then fp32 accumulators for dk and dv of the global keys
    assert need == (4 * heads * (N + G) + 255) // 256 * 256 + 2 * 4 * G * heads * hd
    assert lib.atlas_hier_attn_subset_bwd_workspace_bytes(GRID, Dim3(3, 4, 4), GP, heads, hd) == -1
    G1 = 1 << 30
    base = {"dqd": R, "dkd": R + G1, "dvd": R + 2 * G1, "dqg": R + 3 * G1, "dkg": R + 4 * G1,
            "dvg": R + 5 * G1, "qd": P, "kd": P + G1, "vd": P + 2 * G1, "qg": P + 3 * G1,
            "kg": P + 4 * G1, "vg": P + 5 * G1, "od": Q, "og": Q + G1, "dod": Q + 2 * G1,
            "dog": Q + 3 * G1, "ld": Q + 4 * G1, "lg": Q + 5 * G1, "goff": Q + 6 * G1,
            "gidx": Q + 7 * G1, "ws": Q + 8 * G1}
    order = ("dqd", "dkd", "dvd", "dqg", "dkg", "dvg", "qd", "kd", "vd", "qg", "kg", "vg", "od",
             "og", "dod", "dog", "ld", "lg", "goff", "gidx")

    def call(n=4, ws_bytes=need, scale=0.0, **kw):
        p = dict(base)
        p.update(kw)
        return fn(*(p[k] for k in order), n, p["ws"], ws_bytes, GRID, CUBE, GP, heads, hd, scale,
                  BF16, None)

    assert call(goff=None) == E_NULL
    assert call(gidx=None) == E_NULL
    assert call(n=-1) == E_VALUE
    assert call(goff=Q + 6 * G1 + 2) == E_ALIGN
    assert call(ws_bytes=need - 4) == E_VALUE     # the plain backward's size is not enough
    assert call(ws_bytes=4 * heads * (N + G)) == E_VALUE
    assert call(goff=R + 4 * G1 + 64) == E_ALIAS  # offsets inside dk_g
    assert call(gidx=R + 1 * G1 + 64) == E_ALIAS  # indices inside dk_d
    assert call(ws=R + 5 * G1 + 16) == E_ALIAS    # workspace inside dv_g
    assert call(scale=float("inf")) == E_VALUE


def test_host_checks_are_thread_safe(lib):
    """Eight host threads call the argument checks and the FLOP helper at once
    (ctypes releases the GIL around each call): every call gets its own
    status, and no thread sees a HIP error."""
    import threading
    want = float(lib.atlas_hier_attn_useful_flops(GRID, CUBE, GP, 2, 64))
    bad_cube = Dim3(3, 4, 4)               # 3 does not divide 4
    errors = []

    def worker(k):
        try:
            for i in range(2000):
                if (i + k) % 3 == 0:
                    rc = lib.atlas_cube_reorder(None, None, GRID, CUBE, 2, 64, BF16, None)
                    assert rc == E_NULL, rc
                elif (i + k) % 3 == 1:
                    rc = lib.atlas_cube_reorder(P, Q, GRID, bad_cube, 2, 64, BF16, None)
                    assert rc == E_SHAPE, rc
                else:
                    assert float(lib.atlas_hier_attn_useful_flops(GRID, CUBE, GP, 2, 64)) == want
                assert lib.atlas_last_hip_error() == 0
        except AssertionError as e:          # pragma: no cover - reported below
            errors.append((k, e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
