"""The six workloads of the hierarchical attention path, plus a helper for
small custom shapes used by the tests.

Shapes follow the latent grids the AtlasVid summary pages talk about
(720P training resolution, 1080P, 4K, a longer 4K clip, and 8K), with the detail
grid (T, H, W), the cube (ct, ch, cw), the global proxy grid (Tg, Hg, Wg), the
temporal RoPE scale r_t, heads and head_dim.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    grid: tuple          # detail grid (T, H, W)
    cube: tuple          # cube (ct, ch, cw)
    gproxy: tuple        # global proxy grid (Tg, Hg, Wg); (0, 0, 0) = no global tokens
    r_t: float           # temporal RoPE scale of the global proxy
    heads: int
    head_dim: int
    dtype: str           # "f32" or "bf16"
    outliers: bool = False   # 1% of q/k token rows scaled by 8
    theta: float = 10000.0
    seed: int = 0

    @property
    def N(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def V(self) -> int:
        ct, ch, cw = self.cube
        return ct * ch * cw

    @property
    def C(self) -> int:
        return self.N // self.V

    @property
    def G(self) -> int:
        Tg, Hg, Wg = self.gproxy
        return Tg * Hg * Wg

    @property
    def row_elems(self) -> int:
        return self.heads * self.head_dim

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "grid": list(self.grid), "cube": list(self.cube), "gproxy": list(self.gproxy),
            "r_t": self.r_t, "heads": self.heads, "head_dim": self.head_dim,
            "N": self.N, "V": self.V, "G": self.G, "dtype": self.dtype,
            "outlier_rows": "1% of q/k rows x8" if self.outliers else "none",
        }


CONFIGS = [
    Config("tiny-4x8x8", (4, 8, 8), (2, 4, 4), (2, 4, 4), 4.0, 2, 64, "f32"),
    Config("720p-latent", (21, 45, 80), (3, 15, 16), (6, 23, 40), 4.0, 40, 128, "bf16"),
    Config("1080p-latent", (21, 68, 120), (3, 17, 24), (21, 30, 52), 4.0, 40, 128, "bf16"),
    Config("4k-latent", (21, 136, 240), (3, 17, 24), (21, 30, 52), 4.0, 40, 128, "bf16",
           outliers=True),
    Config("long-4k-latent", (42, 136, 240), (3, 17, 24), (21, 30, 52), 8.0, 40, 128, "bf16"),
    # 8K, 29 frames: the 4K latent scaling (frames 1 + 28/4 = 8; 4320 x 7680 / 16 = 270 x 480).
    # The pages give no cube or proxy for 8K: a 4 x 10 x 32 cube (V = 1280, near the 4K
    # cube's 1224, dividing the grid, and a whole number of 256-query attention blocks)
    # and the 4K proxy's 30 x 52 over the 8 frames, r_t = 4.
    Config("8k-latent", (8, 270, 480), (4, 10, 32), (8, 30, 52), 4.0, 40, 128, "bf16"),
]


def by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def custom(name, grid, cube, gproxy, r_t=4.0, heads=2, head_dim=128, dtype="bf16",
           outliers=False, seed=0) -> Config:
    return Config(name, tuple(grid), tuple(cube), tuple(gproxy), float(r_t), heads, head_dim,
                  dtype, outliers, 10000.0, seed)
