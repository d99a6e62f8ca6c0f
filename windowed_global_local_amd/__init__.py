"""Hierarchical locality-preserving attention for MI355X (gfx950).

Thin Python binding of the C ABI in ``include/atlas.h``; the functions keep
the C names.  Tensors are torch tensors on the GPU, shaped
``[tokens, heads, head_dim]``, contiguous, bfloat16 or float32; heads,
head_dim and dtype are read from the tensors.  ``stream`` defaults to torch's
current stream.  A nonzero status raises :class:`AtlasError`.

The four steps ("Technische Samenvatting: AtlasVid", Methodologie 1 Fase 1
and Fase 2, Methodologie 2):
  atlas_cube_reorder  raster -> cube order (tokens of one cube contiguous)
  atlas_rope3d        3D RoPE, proxy time scaled by r_t, proxy space aligned
  atlas_hier_attn     detail -> own cube + all global; global -> global only
  atlas_cube_unorder  cube order -> raster
and the same path with its layout passes fused:
  atlas_cube_reorder_rope3d  reorder + RoPE in one pass
  atlas_hier_attn_raster     attention writing the detail output in raster order
the mask variant with a per-window global subset (cube order):
  atlas_aligned_subset       host: the co-located global tokens of every cube
  atlas_hier_attn_subset     attention where window c sees only its listed global keys
and the backward pass of the attention (cube order):
  atlas_hier_attn_fwd        attention that also writes the log-sum-exp per query
  atlas_hier_attn_bwd        dq, dk, dv from q, k, v, o, dO and the log-sum-exp
  atlas_hier_attn_subset_fwd / atlas_hier_attn_subset_bwd  the same for the subset mask
Token row counts are checked against the grid and the proxy grid, and the
window offsets against the number of windows, before any launch.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    ATLAS_BF16,
    ATLAS_F32,
    EXPORTS,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    AtlasError,
    Dim3,
    check,
    dim3,
    load,
)

__all__ = [
    "atlas_cube_reorder", "atlas_cube_unorder", "atlas_rope3d", "atlas_cube_reorder_rope3d",
    "atlas_hier_attn", "atlas_hier_attn_raster", "atlas_hier_attn_subset", "atlas_aligned_subset",
    "atlas_hier_attn_fwd", "atlas_hier_attn_bwd", "atlas_hier_attn_bwd_workspace_bytes",
    "atlas_hier_attn_bwd_noalloc",
    "atlas_hier_attn_subset_fwd", "atlas_hier_attn_subset_bwd",
    "atlas_hier_attn_subset_bwd_workspace_bytes", "atlas_hier_attn_useful_flops", "atlas_version",
    "AtlasError", "Dim3", "load",
]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATLAS_BF16
    if t.dtype == torch.float32:
        return ATLAS_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_tensor(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != 3:
        raise ValueError(f"{name} must be [tokens, heads, head_dim]")


def _check_buffer(t, name):
    """A GPU buffer of any shape (log-sum-exp arrays, workspace)."""
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _volume(d) -> int:
    d = dim3(d)
    return int(d.t) * int(d.h) * int(d.w)


def _check_rows(n, what, *named):
    """Every tensor given has n token rows: the kernels read or write n rows of
    each, so a shorter tensor would be overrun on the GPU."""
    for name, t in named:
        if t is not None and t.shape[0] != n:
            raise ValueError(f"{name} has {t.shape[0]} token rows; {what} has {n}")


def _check_lse(t, name, heads, rows):
    if t is not None and tuple(t.shape) != (heads, rows):
        raise ValueError(f"{name} must be [heads, {rows}] = [{heads}, {rows}]")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _layout(ref):
    return ref.shape[1], ref.shape[2], _dtype_code(ref)


def atlas_cube_reorder(dst, src, grid, cube, stream=None):
    """dst[p] = src[pi(p)]: raster-order src -> cube-order dst."""
    _check_tensor(dst, "dst")
    _check_tensor(src, "src")
    heads, hd, dt = _layout(src)
    if dst.shape != src.shape or dst.dtype != src.dtype:
        raise ValueError("dst and src must have the same shape and dtype")
    _check_rows(_volume(grid), "the grid", ("dst", dst), ("src", src))
    check(load().atlas_cube_reorder(_ptr(dst), _ptr(src), dim3(grid), dim3(cube), heads, hd, dt,
                                    _stream(stream)), "atlas_cube_reorder")
    return dst


def atlas_cube_unorder(dst, src, grid, cube, stream=None):
    """dst[pi(p)] = src[p]: cube-order src -> raster-order dst."""
    _check_tensor(dst, "dst")
    _check_tensor(src, "src")
    heads, hd, dt = _layout(src)
    if dst.shape != src.shape or dst.dtype != src.dtype:
        raise ValueError("dst and src must have the same shape and dtype")
    _check_rows(_volume(grid), "the grid", ("dst", dst), ("src", src))
    check(load().atlas_cube_unorder(_ptr(dst), _ptr(src), dim3(grid), dim3(cube), heads, hd, dt,
                                    _stream(stream)), "atlas_cube_unorder")
    return dst


def atlas_rope3d(x_detail, x_global, grid, cube, gproxy, r_t, theta=10000.0, stream=None):
    """In-place 3D RoPE of a detail tensor (cube order) and/or a global tensor."""
    _check_tensor(x_detail, "x_detail")
    _check_tensor(x_global, "x_global")
    ref = x_detail if x_detail is not None else x_global
    if ref is None:
        raise ValueError("x_detail and x_global are both None")
    heads, hd, dt = _layout(ref)
    if x_detail is not None and x_global is not None:
        if x_detail.shape[1:] != x_global.shape[1:] or x_detail.dtype != x_global.dtype:
            raise ValueError("x_detail and x_global must share heads, head_dim and dtype")
    _check_rows(_volume(grid), "the grid", ("x_detail", x_detail))
    _check_rows(_volume(gproxy), "the proxy grid", ("x_global", x_global))
    check(load().atlas_rope3d(_ptr(x_detail), _ptr(x_global), dim3(grid), dim3(cube),
                              dim3(gproxy), float(r_t), float(theta), heads, hd, dt,
                              _stream(stream)), "atlas_rope3d")


def atlas_cube_reorder_rope3d(x_detail, x_raster, x_global, grid, cube, gproxy, r_t, theta=10000.0,
                              stream=None):
    """x_detail = RoPE(cube reorder of x_raster); x_global rotated in place."""
    _check_tensor(x_detail, "x_detail")
    _check_tensor(x_raster, "x_raster")
    _check_tensor(x_global, "x_global")
    ref = x_raster if x_raster is not None else x_global
    if ref is None:
        raise ValueError("x_raster and x_global are both None")
    heads, hd, dt = _layout(ref)
    for t in (x_detail, x_global):
        if t is not None and (t.shape[1:] != ref.shape[1:] or t.dtype != ref.dtype):
            raise ValueError("all tensors must share heads, head_dim and dtype")
    if x_detail is not None and x_raster is not None and x_detail.shape != x_raster.shape:
        raise ValueError("x_detail and x_raster must have the same shape")
    _check_rows(_volume(grid), "the grid", ("x_detail", x_detail), ("x_raster", x_raster))
    _check_rows(_volume(gproxy), "the proxy grid", ("x_global", x_global))
    check(load().atlas_cube_reorder_rope3d(_ptr(x_detail), _ptr(x_raster), _ptr(x_global), dim3(grid),
                                           dim3(cube), dim3(gproxy), float(r_t), float(theta), heads,
                                           hd, dt, _stream(stream)), "atlas_cube_reorder_rope3d")
    return x_detail


def _attn(fn, name, o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
          softmax_scale, stream):
    for t, n in ((o_detail, "o_detail"), (o_global, "o_global"), (q_d, "q_d"), (k_d, "k_d"),
                 (v_d, "v_d"), (q_g, "q_g"), (k_g, "k_g"), (v_g, "v_g")):
        _check_tensor(t, n)
    heads, hd, dt = _layout(q_d)
    for t in (o_detail, o_global, k_d, v_d, q_g, k_g, v_g):
        if t is not None and (t.shape[1:] != q_d.shape[1:] or t.dtype != q_d.dtype):
            raise ValueError("all tensors must share heads, head_dim and dtype")
    _check_rows(_volume(grid), "the grid", ("o_detail", o_detail), ("q_d", q_d), ("k_d", k_d),
                ("v_d", v_d))
    _check_rows(_volume(gproxy), "the proxy grid", ("o_global", o_global), ("q_g", q_g),
                ("k_g", k_g), ("v_g", v_g))
    check(fn(_ptr(o_detail), _ptr(o_global), _ptr(q_d), _ptr(k_d), _ptr(v_d), _ptr(q_g), _ptr(k_g),
             _ptr(v_g), dim3(grid), dim3(cube), dim3(gproxy), heads, hd, float(softmax_scale), dt,
             _stream(stream)), name)


def atlas_hier_attn(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                    softmax_scale=0.0, stream=None):
    """Asymmetric hierarchical attention; detail tensors in cube order."""
    _attn(load().atlas_hier_attn, "atlas_hier_attn", o_detail, o_global, q_d, k_d, v_d, q_g, k_g,
          v_g, grid, cube, gproxy, softmax_scale, stream)


def atlas_hier_attn_raster(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                           softmax_scale=0.0, stream=None):
    """As atlas_hier_attn, with o_detail written in raster order."""
    _attn(load().atlas_hier_attn_raster, "atlas_hier_attn_raster", o_detail, o_global, q_d, k_d,
          v_d, q_g, k_g, v_g, grid, cube, gproxy, softmax_scale, stream)


def atlas_aligned_subset(grid, cube, gproxy, r_t):
    """Co-located global subset on the host: (win_goff int32 [C+1], win_gidx int32)."""
    import numpy as np
    lib = load()
    n = int(lib.atlas_aligned_subset(None, None, 0, dim3(grid), dim3(cube), dim3(gproxy), float(r_t)))
    if n < 0:
        check(n, "atlas_aligned_subset")
    C = (grid[0] // cube[0]) * (grid[1] // cube[1]) * (grid[2] // cube[2])
    goff = np.empty(C + 1, dtype=np.int32)
    gidx = np.empty(max(n, 1), dtype=np.int32)
    r = int(lib.atlas_aligned_subset(goff.ctypes.data, gidx.ctypes.data, gidx.size, dim3(grid),
                                     dim3(cube), dim3(gproxy), float(r_t)))
    if r < 0:
        check(r, "atlas_aligned_subset")
    return goff, gidx[:n]


def atlas_hier_attn_subset(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, win_goff, win_gidx,
                           grid, cube, gproxy, softmax_scale=0.0, stream=None):
    """atlas_hier_attn where window c sees only global rows
    win_gidx[win_goff[c]:win_goff[c+1]]; the lists are int32 GPU tensors."""
    n_gidx = _check_lists(win_goff, win_gidx, grid, cube)

    def fn(od, og, qd, kd, vd, qg, kg, vg, *rest):
        return load().atlas_hier_attn_subset(od, og, qd, kd, vd, qg, kg, vg, _ptr(win_goff),
                                             _ptr(win_gidx), n_gidx, *rest)

    _attn(fn, "atlas_hier_attn_subset", o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid,
          cube, gproxy, softmax_scale, stream)


def atlas_hier_attn_fwd(o_detail, o_global, lse_detail, lse_global, q_d, k_d, v_d, q_g, k_g, v_g,
                        grid, cube, gproxy, softmax_scale=0.0, stream=None):
    """atlas_hier_attn (cube order) that also writes lse_detail [heads, N] and
    lse_global [heads, G] (float32), the natural-log softmax denominators."""
    torch = _torch()
    for t, n in ((lse_detail, "lse_detail"), (lse_global, "lse_global")):
        _check_buffer(t, n)
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    heads = q_d.shape[1]
    if lse_detail.shape != (heads, q_d.shape[0]):
        raise ValueError("lse_detail must be [heads, N]")
    if q_g is not None and (lse_global is None or lse_global.shape != (heads, q_g.shape[0])):
        raise ValueError("lse_global must be [heads, G]")

    def fn(od, og, qd, kd, vd, qg, kg, vg, *rest):
        return load().atlas_hier_attn_fwd(od, og, _ptr(lse_detail), _ptr(lse_global), qd, kd, vd,
                                          qg, kg, vg, *rest)

    _attn(fn, "atlas_hier_attn_fwd", o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube,
          gproxy, softmax_scale, stream)


def _check_bwd_rows(grid, gproxy, heads, dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g,
                    v_g, o_d, o_g, do_d, do_g, lse_detail, lse_global):
    N, G = _volume(grid), _volume(gproxy)
    _check_rows(N, "the grid", ("dq_d", dq_d), ("dk_d", dk_d), ("dv_d", dv_d), ("q_d", q_d),
                ("k_d", k_d), ("v_d", v_d), ("o_d", o_d), ("do_d", do_d))
    _check_rows(G, "the proxy grid", ("dq_g", dq_g), ("dk_g", dk_g), ("dv_g", dv_g), ("q_g", q_g),
                ("k_g", k_g), ("v_g", v_g), ("o_g", o_g), ("do_g", do_g))
    _check_lse(lse_detail, "lse_detail", heads, N)
    if G > 0:
        _check_lse(lse_global, "lse_global", heads, G)


def atlas_hier_attn_bwd_workspace_bytes(grid, cube, gproxy, heads, head_dim) -> int:
    return int(load().atlas_hier_attn_bwd_workspace_bytes(dim3(grid), dim3(cube), dim3(gproxy),
                                                          int(heads), int(head_dim)))


def atlas_hier_attn_bwd(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g, v_g,
                        o_d, o_g, do_d, do_g, lse_detail, lse_global, workspace, grid, cube, gproxy,
                        softmax_scale=0.0, stream=None):
    """Gradients of the asymmetric attention (detail tensors in cube order).

    ``workspace`` is a GPU tensor of at least atlas_hier_attn_bwd_workspace_bytes
    bytes (any dtype)."""
    torch = _torch()
    named = (("dq_d", dq_d), ("dk_d", dk_d), ("dv_d", dv_d), ("dq_g", dq_g), ("dk_g", dk_g),
             ("dv_g", dv_g), ("q_d", q_d), ("k_d", k_d), ("v_d", v_d), ("q_g", q_g), ("k_g", k_g),
             ("v_g", v_g), ("o_d", o_d), ("o_g", o_g), ("do_d", do_d), ("do_g", do_g))
    for n, t in named:
        _check_tensor(t, n)
        if t is not None and (t.shape[1:] != q_d.shape[1:] or t.dtype != q_d.dtype):
            raise ValueError("all tensors must share heads, head_dim and dtype")
    for n, t in (("lse_detail", lse_detail), ("lse_global", lse_global)):
        _check_buffer(t, n)
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    _check_buffer(workspace, "workspace")
    heads, hd, dt = _layout(q_d)
    _check_bwd_rows(grid, gproxy, heads, dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g,
                    v_g, o_d, o_g, do_d, do_g, lse_detail, lse_global)
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load()
    check(lib.atlas_hier_attn_bwd(
        _ptr(dq_d), _ptr(dk_d), _ptr(dv_d), _ptr(dq_g), _ptr(dk_g), _ptr(dv_g),
        _ptr(q_d), _ptr(k_d), _ptr(v_d), _ptr(q_g), _ptr(k_g), _ptr(v_g),
        _ptr(o_d), _ptr(o_g), _ptr(do_d), _ptr(do_g), _ptr(lse_detail), _ptr(lse_global),
        _ptr(workspace), ws_bytes, dim3(grid), dim3(cube), dim3(gproxy), heads, hd,
        float(softmax_scale), dt, _stream(stream)), "atlas_hier_attn_bwd")


def atlas_hier_attn_bwd_noalloc(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g, v_g,
                                o_d, o_g, do_d, do_g, lse_detail, lse_global, grid, cube, gproxy,
                                softmax_scale=0.0, stream=None):
    """atlas_hier_attn_bwd without a workspace argument: the library's fixed
    device array (NOALLOC_SCRATCH_BYTES) serves as workspace, so the call
    allocates nothing.  Calls overlapping on one GPU race on that array."""
    torch = _torch()
    named = (("dq_d", dq_d), ("dk_d", dk_d), ("dv_d", dv_d), ("dq_g", dq_g), ("dk_g", dk_g),
             ("dv_g", dv_g), ("q_d", q_d), ("k_d", k_d), ("v_d", v_d), ("q_g", q_g), ("k_g", k_g),
             ("v_g", v_g), ("o_d", o_d), ("o_g", o_g), ("do_d", do_d), ("do_g", do_g))
    for n, t in named:
        _check_tensor(t, n)
        if t is not None and (t.shape[1:] != q_d.shape[1:] or t.dtype != q_d.dtype):
            raise ValueError("all tensors must share heads, head_dim and dtype")
    for n, t in (("lse_detail", lse_detail), ("lse_global", lse_global)):
        _check_buffer(t, n)
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    heads, hd, dt = _layout(q_d)
    _check_bwd_rows(grid, gproxy, heads, dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g,
                    v_g, o_d, o_g, do_d, do_g, lse_detail, lse_global)
    lib = load()
    check(lib.atlas_hier_attn_bwd_noalloc(
        _ptr(dq_d), _ptr(dk_d), _ptr(dv_d), _ptr(dq_g), _ptr(dk_g), _ptr(dv_g),
        _ptr(q_d), _ptr(k_d), _ptr(v_d), _ptr(q_g), _ptr(k_g), _ptr(v_g),
        _ptr(o_d), _ptr(o_g), _ptr(do_d), _ptr(do_g), _ptr(lse_detail), _ptr(lse_global),
        dim3(grid), dim3(cube), dim3(gproxy), heads, hd, float(softmax_scale), dt, _stream(stream)),
        "atlas_hier_attn_bwd_noalloc")


def _check_lists(win_goff, win_gidx, grid, cube):
    """int32 GPU lists; win_goff holds C + 1 offsets (the kernels read
    win_goff[c] and win_goff[c + 1] of every window c)."""
    torch = _torch()
    for t, n in ((win_goff, "win_goff"), (win_gidx, "win_gidx")):
        _check_buffer(t, n)
        if t is not None and t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    N, V = _volume(grid), _volume(cube)
    if win_goff is not None and V > 0 and N % V == 0 and win_goff.numel() != N // V + 1:
        raise ValueError(f"win_goff must hold C + 1 = {N // V + 1} offsets")
    return 0 if win_gidx is None else win_gidx.numel()


def atlas_hier_attn_subset_fwd(o_detail, o_global, lse_detail, lse_global, q_d, k_d, v_d, q_g, k_g,
                               v_g, win_goff, win_gidx, grid, cube, gproxy, softmax_scale=0.0,
                               stream=None):
    """atlas_hier_attn_subset that also writes lse_detail [heads, N] and
    lse_global [heads, G] (float32)."""
    torch = _torch()
    n_gidx = _check_lists(win_goff, win_gidx, grid, cube)
    for t, n in ((lse_detail, "lse_detail"), (lse_global, "lse_global")):
        _check_buffer(t, n)
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    heads = q_d.shape[1]
    if lse_detail.shape != (heads, q_d.shape[0]):
        raise ValueError("lse_detail must be [heads, N]")
    if q_g is not None and (lse_global is None or lse_global.shape != (heads, q_g.shape[0])):
        raise ValueError("lse_global must be [heads, G]")

    def fn(od, og, qd, kd, vd, qg, kg, vg, *rest):
        return load().atlas_hier_attn_subset_fwd(od, og, _ptr(lse_detail), _ptr(lse_global), qd, kd,
                                                 vd, qg, kg, vg, _ptr(win_goff), _ptr(win_gidx),
                                                 n_gidx, *rest)

    _attn(fn, "atlas_hier_attn_subset_fwd", o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid,
          cube, gproxy, softmax_scale, stream)


def atlas_hier_attn_subset_bwd_workspace_bytes(grid, cube, gproxy, heads, head_dim) -> int:
    return int(load().atlas_hier_attn_subset_bwd_workspace_bytes(dim3(grid), dim3(cube),
                                                                 dim3(gproxy), int(heads),
                                                                 int(head_dim)))


def atlas_hier_attn_subset_bwd(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g, v_g,
                               o_d, o_g, do_d, do_g, lse_detail, lse_global, win_goff, win_gidx,
                               workspace, grid, cube, gproxy, softmax_scale=0.0, stream=None):
    """Gradients of atlas_hier_attn_subset; ``workspace`` holds at least
    atlas_hier_attn_subset_bwd_workspace_bytes bytes."""
    torch = _torch()
    n_gidx = _check_lists(win_goff, win_gidx, grid, cube)
    named = (("dq_d", dq_d), ("dk_d", dk_d), ("dv_d", dv_d), ("dq_g", dq_g), ("dk_g", dk_g),
             ("dv_g", dv_g), ("q_d", q_d), ("k_d", k_d), ("v_d", v_d), ("q_g", q_g), ("k_g", k_g),
             ("v_g", v_g), ("o_d", o_d), ("o_g", o_g), ("do_d", do_d), ("do_g", do_g))
    for n, t in named:
        _check_tensor(t, n)
        if t is not None and (t.shape[1:] != q_d.shape[1:] or t.dtype != q_d.dtype):
            raise ValueError("all tensors must share heads, head_dim and dtype")
    for n, t in (("lse_detail", lse_detail), ("lse_global", lse_global)):
        _check_buffer(t, n)
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    _check_buffer(workspace, "workspace")
    heads, hd, dt = _layout(q_d)
    _check_bwd_rows(grid, gproxy, heads, dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g,
                    v_g, o_d, o_g, do_d, do_g, lse_detail, lse_global)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(load().atlas_hier_attn_subset_bwd(
        _ptr(dq_d), _ptr(dk_d), _ptr(dv_d), _ptr(dq_g), _ptr(dk_g), _ptr(dv_g),
        _ptr(q_d), _ptr(k_d), _ptr(v_d), _ptr(q_g), _ptr(k_g), _ptr(v_g),
        _ptr(o_d), _ptr(o_g), _ptr(do_d), _ptr(do_g), _ptr(lse_detail), _ptr(lse_global),
        _ptr(win_goff), _ptr(win_gidx), n_gidx, _ptr(workspace), ws_bytes, dim3(grid), dim3(cube),
        dim3(gproxy), heads, hd, float(softmax_scale), dt, _stream(stream)),
        "atlas_hier_attn_subset_bwd")


def atlas_hier_attn_useful_flops(grid, cube, gproxy, heads, head_dim) -> float:
    return float(load().atlas_hier_attn_useful_flops(dim3(grid), dim3(cube), dim3(gproxy),
                                                     int(heads), int(head_dim)))


def atlas_version() -> int:
    return int(load().atlas_version())
