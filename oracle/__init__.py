"""fp64 CPU oracle for the hierarchical locality-preserving attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The HIP library never imports,
links or calls anything here, and nothing here touches the GPU.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over output rows); this
module only marshals numpy arrays into it.  Definitions follow
"Technische Samenvatting: AtlasVid" (Methodologie 1, Fase 1 and Fase 2;
Methodologie 2, Asymmetrische Hierarchische Attention and Positie-uitlijning)
and the English abstract of "AtlasVid: Efficient Ultra-High-Resolution Long
Video Generation via Decoupled Global-Local Modeling".

Boundary tensors are numpy arrays shaped ``[tokens, heads, D]``:
``uint16`` arrays hold raw bf16 bit patterns, ``float32`` and ``float64``
arrays hold themselves.  Every function upcasts the exact stored values to
fp64.

Parity pins (tests/test_oracle_pins.py): the permutation is checked against a
brute-force cube enumeration and round trips; RoPE against a complex-number
formulation, norm preservation, the relative-position identity and position
zero; attention against a dense masked softmax over the concatenation
[X_global; X_detail], single-cube full attention, log-sum-exp merging and
closed-form special cases; the backward against central finite differences of
the forward, automatic differentiation of the dense masked softmax and the
sum rules of softmax gradients.  The choices the pages leave open (cube
enumeration order, the head_dim split and frequency ladder of RoPE, the exact
global coordinates) are parity unpinned by the pages: only the agreement of
two independent implementations pins them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16, F32, F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.orc_round_bf16.argtypes = [dbl]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_round_bf16_array.argtypes = [vp, vp, i64]
    lib.orc_round_bf16_array.restype = None
    lib.orc_cube_src.argtypes = [i64] * 7
    lib.orc_cube_src.restype = i64
    lib.orc_cube_dst.argtypes = [i64] * 7
    lib.orc_cube_dst.restype = i64
    lib.orc_cube_perm.argtypes = [vp] + [i64] * 6
    lib.orc_cube_perm.restype = None
    for name in ("orc_cube_reorder", "orc_cube_unorder"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, i64] + [i64] * 6
        f.restype = None
    lib.orc_pos_detail.argtypes = [vp, i64] + [i64] * 6
    lib.orc_pos_detail.restype = None
    lib.orc_pos_global.argtypes = [vp, i64, i64, i64, i64, i64, i64, dbl]
    lib.orc_pos_global.restype = None
    lib.orc_rope_vec.argtypes = [vp, i32, vp, dbl]
    lib.orc_rope_vec.restype = None
    lib.orc_rope_rows.argtypes = [vp, vp, i64, i32, i32, dbl]
    lib.orc_rope_rows.restype = None
    lib.orc_hier_attn.argtypes = ([vp] * 8 + [i32, i64, i64, i64, i32, i32, dbl]
                                  + [vp, vp, vp, i64, vp, vp])
    lib.orc_hier_attn.restype = None
    lib.orc_pipeline_rows.argtypes = ([vp] * 7 + [i32] + [i64] * 9
                                      + [dbl, dbl, i32, i32, dbl] + [vp, vp, vp, i64])
    lib.orc_pipeline_rows.restype = None
    lib.orc_aligned_subset.argtypes = [vp, vp] + [i64] * 9 + [dbl]
    lib.orc_aligned_subset.restype = i64
    lib.orc_hier_attn_bwd.argtypes = [vp] * 18 + [i32, i64, i64, i64, i32, i32, dbl, vp, vp]
    lib.orc_hier_attn_bwd.restype = None
    lib.orc_hier_attn_bwd_rows.argtypes = ([vp] * 11 + [i32, i64, i64, i64, i32, i32, dbl]
                                           + [vp, vp, vp, i64])
    lib.orc_hier_attn_bwd_rows.restype = None
    lib.orc_hier_attn_bwd_window.argtypes = [vp] * 8 + [i32, i64, i64, i32, i32, dbl, i32, i64]
    lib.orc_hier_attn_bwd_window.restype = None
    # dk, dv, qd, kd, vd, dod, qg, kg, vg, dog | dtype, N, V, G, heads, D, scale, head, key, nsel
    lib.orc_hier_attn_bwd_gkeys.argtypes = [vp] * 10 + [i32, i64, i64, i64, i32, i32, dbl, i32, vp, i64]
    lib.orc_hier_attn_bwd_gkeys.restype = None
    # the same loops summing the squares of the terms (error scales of the tests)
    for name in ("orc_hier_attn_bwd", "orc_hier_attn_bwd_rows", "orc_hier_attn_bwd_window",
                 "orc_hier_attn_bwd_gkeys"):
        f = getattr(lib, name + "_rss")
        f.argtypes = getattr(lib, name).argtypes
        f.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported boundary dtype {a.dtype}")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


# ---------------------------------------------------------------- bf16 helpers

def round_bf16(x) -> np.ndarray:
    """Exact fp64 -> bf16 round-to-nearest-even, as raw uint16 bit patterns."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_round_bf16_array(_ptr(out), _ptr(x), x.size)
    return out


def to_f64(a: np.ndarray) -> np.ndarray:
    """Upcast a boundary array (bf16 bits / fp32 / fp64) to fp64 exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- O1 / O4

def cube_src(p: int, grid, cube) -> int:
    return int(_load().orc_cube_src(p, *grid, *cube))


def cube_dst(r: int, grid, cube) -> int:
    return int(_load().orc_cube_dst(r, *grid, *cube))


def cube_perm(grid, cube) -> np.ndarray:
    """pi as an int64 array: cube-order position p -> raster index pi[p]."""
    T, H, W = grid
    pi = np.empty(T * H * W, dtype=np.int64)
    _load().orc_cube_perm(_ptr(pi), *grid, *cube)
    return pi


def cube_reorder(x: np.ndarray, grid, cube) -> np.ndarray:
    """Y[p] = X[pi(p)] for X of shape [T*H*W, ...] (any dtype; bytes move)."""
    x = np.ascontiguousarray(x)
    y = np.empty_like(x)
    rb = x.nbytes // x.shape[0]
    _load().orc_cube_reorder(_ptr(y), _ptr(x), rb, *grid, *cube)
    return y


def cube_unorder(y: np.ndarray, grid, cube) -> np.ndarray:
    """X[pi(p)] = Y[p]."""
    y = np.ascontiguousarray(y)
    x = np.empty_like(y)
    rb = y.nbytes // y.shape[0]
    _load().orc_cube_unorder(_ptr(x), _ptr(y), rb, *grid, *cube)
    return x


# ---------------------------------------------------------------- O2

def pos_detail(p_rows, grid, cube) -> np.ndarray:
    """[n, 3] RoPE coordinates of detail tokens at cube-order positions."""
    lib = _load()
    p_rows = np.asarray(p_rows, dtype=np.int64).reshape(-1)
    out = np.empty((p_rows.size, 3), dtype=np.float64)
    for i, p in enumerate(p_rows):
        lib.orc_pos_detail(_ptr(out[i]), int(p), *grid, *cube)
    return out


def pos_global(r_rows, grid, gproxy, r_t) -> np.ndarray:
    """[n, 3] RoPE coordinates of global tokens at proxy raster positions."""
    lib = _load()
    r_rows = np.asarray(r_rows, dtype=np.int64).reshape(-1)
    _, H, W = grid
    out = np.empty((r_rows.size, 3), dtype=np.float64)
    for i, r in enumerate(r_rows):
        lib.orc_pos_global(_ptr(out[i]), int(r), H, W, *gproxy, float(r_t))
    return out


def rope_rows(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotate rows x [n, heads, D] (any boundary dtype) to coordinates pos [n, 3].

    Returns fp64 (no rounding)."""
    xf = np.ascontiguousarray(to_f64(x))
    n, heads, D = xf.shape
    pos = np.ascontiguousarray(pos, dtype=np.float64).reshape(n, 3)
    _load().orc_rope_rows(_ptr(xf), _ptr(pos), n, heads, D, float(theta))
    return xf


def rope_detail(x: np.ndarray, p_rows, grid, cube, theta: float = 10000.0) -> np.ndarray:
    return rope_rows(x, pos_detail(p_rows, grid, cube), theta)


def rope_global(x: np.ndarray, r_rows, grid, gproxy, r_t, theta: float = 10000.0) -> np.ndarray:
    return rope_rows(x, pos_global(r_rows, grid, gproxy, r_t), theta)


# ---------------------------------------------------------------- O3

def _selection(N, G, heads, sel):
    if sel is None:
        rows = np.concatenate([np.repeat(np.arange(N), heads), np.repeat(np.arange(G), heads)])
        hds = np.concatenate([np.tile(np.arange(heads), N), np.tile(np.arange(heads), G)])
        isg = np.concatenate([np.zeros(N * heads), np.ones(G * heads)])
    else:
        rows, hds, isg = sel
    return (np.ascontiguousarray(rows, dtype=np.int64), np.ascontiguousarray(hds, dtype=np.int32),
            np.ascontiguousarray(isg, dtype=np.int8))


def hier_attn(qd, kd, vd, qg, kg, vg, V: int, scale: float | None = None,
              sel=None, return_lse: bool = False, subset=None):
    """Asymmetric hierarchical attention in fp64.

    qd/kd/vd: [N, heads, D] detail tensors in cube order; qg/kg/vg: [G, heads, D]
    (or None when G = 0).  ``sel`` = (rows, heads, is_global) arrays selects
    outputs; None computes everything and returns (o_detail [N,heads,D],
    o_global [G,heads,D] or None).  With ``sel`` returns [nsel, D].
    ``return_lse`` adds the natural-log softmax denominator of every selected
    row (with ``sel``: [nsel]; without: [heads, N] and [heads, G] or None).
    ``subset`` = (goff [C+1], gidx) restricts the global keys of a detail query
    in window c to rows gidx[goff[c]:goff[c+1]] (global queries unchanged)."""
    lib = _load()
    qd, kd, vd = _c(qd), _c(kd), _c(vd)
    qg, kg, vg = _c(qg), _c(kg), _c(vg)
    dt = _dtype_code(qd)
    N, heads, D = qd.shape
    G = 0 if qg is None else qg.shape[0]
    for a in (kd, vd) + ((qg, kg, vg) if G else ()):
        if _dtype_code(a) != dt:
            raise TypeError("all inputs must share one dtype")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    full = sel is None
    rows, hds, isg = _selection(N, G, heads, sel)
    out = np.empty((rows.size, D), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    goff = gidx = None
    if subset is not None:
        goff = np.ascontiguousarray(subset[0], dtype=np.int64)
        gidx = np.ascontiguousarray(subset[1], dtype=np.int32)
        if goff.size != N // V + 1 or goff[-1] > gidx.size:
            raise ValueError("subset: goff must have C+1 entries and index gidx")
        if gidx.size == 0:
            gidx = np.zeros(1, dtype=np.int32)
    lib.orc_hier_attn(_ptr(out), _ptr(lse), _ptr(qd), _ptr(kd), _ptr(vd), _ptr(qg), _ptr(kg),
                      _ptr(vg), dt, N, V, G, heads, D, float(scale),
                      _ptr(rows), _ptr(hds), _ptr(isg), rows.size, _ptr(goff), _ptr(gidx))
    if not full:
        return (out, lse) if return_lse else out
    od = out[: N * heads].reshape(N, heads, D)
    og = out[N * heads:].reshape(G, heads, D) if G else None
    if not return_lse:
        return od, og
    ld = np.ascontiguousarray(lse[: N * heads].reshape(N, heads).T)
    lg = np.ascontiguousarray(lse[N * heads:].reshape(G, heads).T) if G else None
    return od, og, ld, lg


def aligned_subset(grid, cube, gproxy, r_t):
    """Co-located global subset: (goff int64 [C+1], gidx int32) with the proxy
    tokens whose aligned position lies in each cube's box."""
    lib = _load()
    T, H, W = grid
    ct, ch, cw = cube
    C = (T // ct) * (H // ch) * (W // cw)
    G = gproxy[0] * gproxy[1] * gproxy[2]
    goff = np.empty(C + 1, dtype=np.int64)
    gidx = np.empty(max(G, 1), dtype=np.int32)
    n = lib.orc_aligned_subset(_ptr(goff), _ptr(gidx), *grid, *cube, *gproxy, float(r_t))
    return goff, gidx[:n].copy()


# ---------------------------------------------------------------- O3 backward

def _bwd_inputs(qd, kd, vd, dod, qg, kg, vg, dog):
    qd, kd, vd, dod = _c(qd), _c(kd), _c(vd), _c(dod)
    qg, kg, vg, dog = _c(qg), _c(kg), _c(vg), _c(dog)
    dt = _dtype_code(qd)
    G = 0 if qg is None else qg.shape[0]
    for a in (kd, vd, dod) + ((qg, kg, vg, dog) if G else ()):
        if _dtype_code(a) != dt:
            raise TypeError("all inputs must share one dtype")
    return (qd, kd, vd, dod, qg, kg, vg, dog), dt, G


def hier_attn_bwd(qd, kd, vd, dod, qg, kg, vg, dog, V: int, scale: float | None = None,
                  subset=None, rss: bool = False):
    """Gradients of the asymmetric attention in fp64, every row.

    ``subset`` = (goff [C+1], gidx) restricts window c's global keys to rows
    gidx[goff[c]:goff[c+1]] (indices in [0, G)), as in hier_attn.
    Returns a dict: dq_d, dk_d, dv_d [N, heads, D]; dq_g, dk_g, dv_g [G, heads, D]
    (None when G = 0); lse_d, delta_d [heads, N]; lse_g, delta_g [heads, G].
    ``rss=True`` returns, in place of each gradient element, the root-sum-square
    of the terms that sum to it (scale dS_ij k_j, scale dS_ij q_i, P_ij dO_i):
    the scale of independent rounding errors of those terms."""
    lib = _load()
    (qd, kd, vd, dod, qg, kg, vg, dog), dt, G = _bwd_inputs(qd, kd, vd, dod, qg, kg, vg, dog)
    N, heads, D = qd.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    goff = gidx = None
    if subset is not None:
        goff = np.ascontiguousarray(subset[0], dtype=np.int64)
        gidx = np.ascontiguousarray(subset[1], dtype=np.int32)
        if goff.size != N // V + 1 or goff[0] != 0 or np.any(np.diff(goff) < 0) or goff[-1] > gidx.size:
            raise ValueError("goff must be C + 1 nondecreasing offsets into gidx")
        if gidx.size and (gidx.min() < 0 or gidx.max() >= G):
            raise ValueError("subset index out of range")
    shp_d, shp_g = (N, heads, D), (max(G, 1), heads, D)
    r = {k: np.empty(shp_d) for k in ("dq_d", "dk_d", "dv_d")}
    r.update({k: np.empty(shp_g) for k in ("dq_g", "dk_g", "dv_g")})
    r.update(lse_d=np.empty((heads, N)), delta_d=np.empty((heads, N)),
             lse_g=np.empty((heads, max(G, 1))), delta_g=np.empty((heads, max(G, 1))))
    fn = lib.orc_hier_attn_bwd_rss if rss else lib.orc_hier_attn_bwd
    fn(_ptr(r["dq_d"]), _ptr(r["dk_d"]), _ptr(r["dv_d"]),
       _ptr(r["dq_g"]), _ptr(r["dk_g"]), _ptr(r["dv_g"]),
       _ptr(r["lse_d"]), _ptr(r["lse_g"]), _ptr(r["delta_d"]), _ptr(r["delta_g"]),
       _ptr(qd), _ptr(kd), _ptr(vd), _ptr(dod), _ptr(qg), _ptr(kg), _ptr(vg),
       _ptr(dog), dt, N, V, G, heads, D, float(scale),
       None if goff is None else _ptr(goff), None if gidx is None else _ptr(gidx))
    if G == 0:
        for k in ("dq_g", "dk_g", "dv_g", "lse_g", "delta_g"):
            r[k] = None
    return r


def hier_attn_bwd_rows(qd, kd, vd, dod, qg, kg, vg, dog, V: int, sel, scale: float | None = None,
                       rss: bool = False):
    """dq [nsel, D], lse [nsel] and delta [nsel] of selected query rows
    ``sel`` = (rows, heads, is_global); ``rss=True``: the root-sum-square of
    dq's terms in place of dq (see hier_attn_bwd)."""
    lib = _load()
    (qd, kd, vd, dod, qg, kg, vg, dog), dt, G = _bwd_inputs(qd, kd, vd, dod, qg, kg, vg, dog)
    N, heads, D = qd.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows, hds, isg = _selection(N, G, heads, sel)
    dq = np.empty((rows.size, D))
    lse = np.empty(rows.size)
    dl = np.empty(rows.size)
    fn = lib.orc_hier_attn_bwd_rows_rss if rss else lib.orc_hier_attn_bwd_rows
    fn(_ptr(dq), _ptr(lse), _ptr(dl), _ptr(qd), _ptr(kd), _ptr(vd),
       _ptr(dod), _ptr(qg), _ptr(kg), _ptr(vg), _ptr(dog), dt, N, V, G,
       heads, D, float(scale), _ptr(rows), _ptr(hds), _ptr(isg), rows.size)
    return dq, lse, dl


def hier_attn_bwd_window(qd, kd, vd, dod, kg, vg, V: int, head: int, c: int,
                         scale: float | None = None, rss: bool = False):
    """dk, dv [V, D] of the detail keys of window c for one head (``rss=True``:
    the root-sum-square of their terms, see hier_attn_bwd)."""
    lib = _load()
    qd, kd, vd, dod, kg, vg = _c(qd), _c(kd), _c(vd), _c(dod), _c(kg), _c(vg)
    dt = _dtype_code(qd)
    N, heads, D = qd.shape
    G = 0 if kg is None else kg.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dk = np.empty((V, D))
    dv = np.empty((V, D))
    fn = lib.orc_hier_attn_bwd_window_rss if rss else lib.orc_hier_attn_bwd_window
    fn(_ptr(dk), _ptr(dv), _ptr(qd), _ptr(kd), _ptr(vd), _ptr(dod),
       _ptr(kg), _ptr(vg), dt, V, G, heads, D, float(scale), head, c)
    return dk, dv


def hier_attn_bwd_gkeys(qd, kd, vd, dod, qg, kg, vg, dog, V: int, head: int, keys,
                        scale: float | None = None, rss: bool = False):
    """dk, dv [len(keys), D] of the selected global keys of one head: the sum
    over every detail and global query (each sees every global key);
    ``rss=True``: the root-sum-square of their terms (see hier_attn_bwd)."""
    lib = _load()
    qd, kd, vd, dod = _c(qd), _c(kd), _c(vd), _c(dod)
    qg, kg, vg, dog = _c(qg), _c(kg), _c(vg), _c(dog)
    dt = _dtype_code(qd)
    N, heads, D = qd.shape
    G = kg.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    if keys.size and (keys.min() < 0 or keys.max() >= G):
        raise ValueError("global key index out of range")
    dk = np.empty((keys.size, D))
    dv = np.empty((keys.size, D))
    fn = lib.orc_hier_attn_bwd_gkeys_rss if rss else lib.orc_hier_attn_bwd_gkeys
    fn(_ptr(dk), _ptr(dv), _ptr(qd), _ptr(kd), _ptr(vd), _ptr(dod),
       _ptr(qg), _ptr(kg), _ptr(vg), _ptr(dog), dt, N, V, G, heads, D,
       float(scale), int(head), _ptr(keys), keys.size)
    return dk, dv


# ---------------------------------------------------------------- end to end

def pipeline_rows(qd, kd, vd, qg, kg, vg, grid, cube, gproxy, r_t,
                  theta: float = 10000.0, scale: float | None = None, sel=None):
    """reorder -> RoPE -> attention -> unorder for selected raster output rows.

    Inputs are raw raster-order tensors.  Rotated q/k are rounded to the
    boundary dtype before attention, as they are stored between the calls.
    ``sel`` = (rows, heads, is_global); None computes every row."""
    lib = _load()
    qd, kd, vd = _c(qd), _c(kd), _c(vd)
    qg, kg, vg = _c(qg), _c(kg), _c(vg)
    dt = _dtype_code(qd)
    N, heads, D = qd.shape
    G = 0 if qg is None else qg.shape[0]
    if G == 0:
        gproxy = (0, 0, 0)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    full = sel is None
    if full:
        rows = np.concatenate([np.repeat(np.arange(N), heads), np.repeat(np.arange(G), heads)])
        hds = np.concatenate([np.tile(np.arange(heads), N), np.tile(np.arange(heads), G)])
        isg = np.concatenate([np.zeros(N * heads), np.ones(G * heads)])
    else:
        rows, hds, isg = sel
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    hds = np.ascontiguousarray(hds, dtype=np.int32)
    isg = np.ascontiguousarray(isg, dtype=np.int8)
    out = np.empty((rows.size, D), dtype=np.float64)
    lib.orc_pipeline_rows(_ptr(out), _ptr(qd), _ptr(kd), _ptr(vd), _ptr(qg), _ptr(kg), _ptr(vg),
                          dt, *grid, *cube, *gproxy, float(r_t), float(theta), heads, D,
                          float(scale), _ptr(rows), _ptr(hds), _ptr(isg), rows.size)
    if not full:
        return out
    od = out[: N * heads].reshape(N, heads, D)
    og = out[N * heads:].reshape(G, heads, D) if G else None
    return od, og
