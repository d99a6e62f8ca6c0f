"""ctypes binding of libatlas.so (include/atlas.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libatlas.so.  PyTorch supplies device memory and the current HIP stream.
There is no fallback: if the library is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libatlas.so")

ATLAS_BF16, ATLAS_F32 = 0, 1
ATLAS_OK = 0
STATUS = {
    0: "ATLAS_OK", -1: "ATLAS_ERR_NULL", -2: "ATLAS_ERR_SHAPE", -3: "ATLAS_ERR_DTYPE",
    -4: "ATLAS_ERR_UNSUPPORTED", -5: "ATLAS_ERR_ALIGN", -6: "ATLAS_ERR_ALIAS",
    -7: "ATLAS_ERR_HIP", -8: "ATLAS_ERR_VALUE", -9: "ATLAS_ERR_SCRATCH",
}
# bytes of the fixed device array behind atlas_hier_attn_bwd_noalloc
NOALLOC_SCRATCH_BYTES = 128 << 20
# every symbol include/atlas.h declares
EXPORTS = ("atlas_cube_reorder", "atlas_cube_unorder", "atlas_rope3d", "atlas_cube_reorder_rope3d",
           "atlas_hier_attn", "atlas_hier_attn_raster", "atlas_hier_attn_subset",
           "atlas_aligned_subset", "atlas_hier_attn_fwd",
           "atlas_hier_attn_bwd_workspace_bytes", "atlas_hier_attn_bwd", "atlas_hier_attn_bwd_noalloc",
           "atlas_hier_attn_subset_fwd",
           "atlas_hier_attn_subset_bwd_workspace_bytes", "atlas_hier_attn_subset_bwd",
           "atlas_hier_attn_useful_flops",
           "atlas_status_string", "atlas_last_hip_error", "atlas_version")


class Dim3(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]

    def __repr__(self):
        return f"Dim3({self.t}, {self.h}, {self.w})"


def dim3(x) -> Dim3:
    if isinstance(x, Dim3):
        return x
    t, h, w = (int(v) for v in x)
    return Dim3(t, h, w)


class AtlasError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.name = STATUS.get(code, str(code))
        msg = load().atlas_status_string(code).decode()
        if code == -7:
            msg += f" (hipError {load().atlas_last_hip_error()})"
        super().__init__(f"{where}: {self.name}: {msg}")


_lib = None


def load():
    """Load libatlas.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python windowed_global_local_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    copy_sig = [vp, vp, Dim3, Dim3, i32, i32, i32, vp]
    lib.atlas_cube_reorder.argtypes = copy_sig
    lib.atlas_cube_reorder.restype = ctypes.c_int
    lib.atlas_cube_unorder.argtypes = copy_sig
    lib.atlas_cube_unorder.restype = ctypes.c_int
    lib.atlas_rope3d.argtypes = [vp, vp, Dim3, Dim3, Dim3, f32, f32, i32, i32, i32, vp]
    lib.atlas_rope3d.restype = ctypes.c_int
    lib.atlas_cube_reorder_rope3d.argtypes = [vp, vp, vp, Dim3, Dim3, Dim3, f32, f32, i32, i32, i32, vp]
    lib.atlas_cube_reorder_rope3d.restype = ctypes.c_int
    lib.atlas_hier_attn.argtypes = [vp] * 8 + [Dim3, Dim3, Dim3, i32, i32, f32, i32, vp]
    lib.atlas_hier_attn.restype = ctypes.c_int
    lib.atlas_hier_attn_raster.argtypes = [vp] * 8 + [Dim3, Dim3, Dim3, i32, i32, f32, i32, vp]
    lib.atlas_hier_attn_raster.restype = ctypes.c_int
    lib.atlas_hier_attn_subset.argtypes = [vp] * 10 + [ctypes.c_int64, Dim3, Dim3, Dim3, i32, i32,
                                                       f32, i32, vp]
    lib.atlas_hier_attn_subset.restype = ctypes.c_int
    lib.atlas_aligned_subset.argtypes = [vp, vp, ctypes.c_int64, Dim3, Dim3, Dim3, f32]
    lib.atlas_aligned_subset.restype = ctypes.c_int64
    lib.atlas_hier_attn_fwd.argtypes = [vp] * 10 + [Dim3, Dim3, Dim3, i32, i32, f32, i32, vp]
    lib.atlas_hier_attn_fwd.restype = ctypes.c_int
    lib.atlas_hier_attn_bwd_workspace_bytes.argtypes = [Dim3, Dim3, Dim3, i32, i32]
    lib.atlas_hier_attn_bwd_workspace_bytes.restype = ctypes.c_int64
    lib.atlas_hier_attn_bwd.argtypes = ([vp] * 19 + [ctypes.c_int64]
                                        + [Dim3, Dim3, Dim3, i32, i32, f32, i32, vp])
    lib.atlas_hier_attn_bwd.restype = ctypes.c_int
    lib.atlas_hier_attn_bwd_noalloc.argtypes = [vp] * 18 + [Dim3, Dim3, Dim3, i32, i32, f32, i32, vp]
    lib.atlas_hier_attn_bwd_noalloc.restype = ctypes.c_int
    lib.atlas_hier_attn_subset_fwd.argtypes = [vp] * 12 + [ctypes.c_int64, Dim3, Dim3, Dim3, i32, i32,
                                                           f32, i32, vp]
    lib.atlas_hier_attn_subset_fwd.restype = ctypes.c_int
    lib.atlas_hier_attn_subset_bwd_workspace_bytes.argtypes = [Dim3, Dim3, Dim3, i32, i32]
    lib.atlas_hier_attn_subset_bwd_workspace_bytes.restype = ctypes.c_int64
    # 18 tensors, goff, gidx | n_gidx | workspace | bytes | dims ...
    lib.atlas_hier_attn_subset_bwd.argtypes = ([vp] * 20 + [ctypes.c_int64, vp, ctypes.c_int64]
                                               + [Dim3, Dim3, Dim3, i32, i32, f32, i32, vp])
    lib.atlas_hier_attn_subset_bwd.restype = ctypes.c_int
    lib.atlas_hier_attn_useful_flops.argtypes = [Dim3, Dim3, Dim3, i32, i32]
    lib.atlas_hier_attn_useful_flops.restype = ctypes.c_double
    lib.atlas_status_string.argtypes = [ctypes.c_int]
    lib.atlas_status_string.restype = ctypes.c_char_p
    lib.atlas_last_hip_error.argtypes = []
    lib.atlas_last_hip_error.restype = ctypes.c_int
    lib.atlas_version.argtypes = []
    lib.atlas_version.restype = ctypes.c_int
    _lib = lib
    return lib


def check(code: int, where: str) -> None:
    if code != ATLAS_OK:
        raise AtlasError(code, where)
