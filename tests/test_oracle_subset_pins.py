"""Pins of the oracle's mask variants (CPU only).

"Technische Samenvatting: AtlasVid", Methodologie 2 (Asymmetrische
Hierarchische Attention) lets a detail query see "aligned" global tokens;
Positie-uitlijning maps proxy token (tg, hg, wg) to (r_t*tg, (H/Hg)*hg,
(W/Wg)*wg).  The co-located reading gives each cube the proxy tokens whose
mapped position lies in its box.  Pins:
  * the subset attention with every window's list = all global keys is the
    plain attention, and with arbitrary lists it is the dense masked softmax
    whose mask lets window c see exactly its listed global columns;
  * the co-located lists: hand-worked small grids, and r_t = 1 with proxy grid
    = detail grid, where every proxy token sits on a detail token and cube c's
    list is the raster indices of its own tokens (the cube permutation, pinned
    separately);
  * Experimentele Resultaten (Ablatiestudies) compares against naive block
    attention: windows of V consecutive raster tokens, which is the same
    attention run on raster-order tensors, checked here against a dense
    block-diagonal mask.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from workload import custom, gen_inputs


def dense_subset_attention(qd, kd, vd, qg, kg, vg, V, goff, gidx, scale):
    """Dense masked softmax over [X_global; X_detail] with the subset mask."""
    N, heads, D = qd.shape
    G = qg.shape[0]
    Q, K, Vv = (np.concatenate([a, b], 0) for a, b in ((qg, qd), (kg, kd), (vg, vd)))
    L = G + N
    allow = np.zeros((L, L), dtype=bool)
    allow[:G, :G] = True
    for c in range(N // V):
        rows = slice(G + c * V, G + (c + 1) * V)
        allow[rows, G + c * V:G + (c + 1) * V] = True
        cols = np.asarray(gidx[goff[c]:goff[c + 1]], dtype=np.int64)
        allow[rows, cols] = True
    out = np.empty_like(Q)
    for h in range(heads):
        s = (Q[:, h] @ K[:, h].T) * scale
        s = np.where(allow, s, -np.inf)
        s = s - s.max(1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(1, keepdims=True)
        out[:, h] = p @ Vv[:, h]
    return out[G:], out[:G]


def _f64(cfg):
    return {k: (None if v is None else oracle.to_f64(v)) for k, v in gen_inputs(cfg).items()}


def test_subset_all_global_equals_plain_attention():
    cfg = custom("s1", (2, 6, 8), (2, 3, 4), (1, 3, 5), heads=2, head_dim=64, dtype="f32")
    x = _f64(cfg)
    goff = np.arange(cfg.C + 1, dtype=np.int64) * cfg.G
    gidx = np.tile(np.arange(cfg.G, dtype=np.int32), cfg.C)
    a = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V)
    b = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V,
                         subset=(goff, gidx))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("seed", [0, 1])
def test_subset_matches_dense_masked_softmax(seed):
    cfg = custom("s2", (2, 6, 8), (2, 3, 4), (1, 3, 5), heads=2, head_dim=64, dtype="f32")
    x = _f64(cfg)
    rng = np.random.default_rng(seed)
    lists = [np.sort(rng.choice(cfg.G, size=int(rng.integers(0, cfg.G + 1)), replace=False))
             for _ in range(cfg.C)]
    lists[0] = np.zeros(0, dtype=np.int64)          # one window with no global keys
    goff = np.concatenate([[0], np.cumsum([len(l) for l in lists])]).astype(np.int64)
    gidx = np.concatenate(lists).astype(np.int32)
    od, og = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V,
                              subset=(goff, gidx))
    wd, wg = dense_subset_attention(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                                    cfg.V, goff, gidx, 1 / math.sqrt(cfg.head_dim))
    np.testing.assert_allclose(od, wd, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(og, wg, rtol=1e-11, atol=1e-12)


def test_aligned_subset_hand_worked():
    # grid 4x4x4, cube 2x2x2, proxy 2x2x2, r_t = 2: proxy g = (tg, hg, wg) maps to
    # (2tg, 2hg, 2wg), the corner of cube (tg, hg, wg), whose raster number is g
    goff, gidx = oracle.aligned_subset((4, 4, 4), (2, 2, 2), (2, 2, 2), 2.0)
    np.testing.assert_array_equal(goff, np.arange(9))
    np.testing.assert_array_equal(gidx, np.arange(8))
    # proxy 1x1x1: one token at the origin, in cube 0 only
    goff, gidx = oracle.aligned_subset((4, 4, 4), (2, 2, 2), (1, 1, 1), 4.0)
    np.testing.assert_array_equal(goff, [0] + [1] * 8)
    np.testing.assert_array_equal(gidx, [0])
    # r_t = 4 with ct = 2: proxy frames at t = 0 and 4; 4 >= T = 4 lies outside
    goff, gidx = oracle.aligned_subset((4, 4, 4), (2, 2, 2), (2, 2, 2), 4.0)
    np.testing.assert_array_equal(np.diff(goff), [1, 1, 1, 1, 0, 0, 0, 0])
    np.testing.assert_array_equal(gidx, [0, 1, 2, 3])
    # fractional spatial ratios: W/Wg = 6/4 puts wg = 0,1,2,3 at 0, 1.5, 3, 4.5;
    # cubes of width 3 take {0, 1.5} and {3, 4.5}
    goff, gidx = oracle.aligned_subset((1, 1, 6), (1, 1, 3), (1, 1, 4), 1.0)
    np.testing.assert_array_equal(goff, [0, 2, 4])
    np.testing.assert_array_equal(gidx, [0, 1, 2, 3])


@pytest.mark.parametrize("grid,cube", [((4, 6, 8), (2, 3, 4)), ((3, 4, 10), (1, 2, 5)),
                                       ((2, 2, 2), (2, 2, 2))])
def test_aligned_subset_identity_proxy_is_cube_membership(grid, cube):
    goff, gidx = oracle.aligned_subset(grid, cube, grid, 1.0)
    pi = oracle.cube_perm(grid, cube)
    V = cube[0] * cube[1] * cube[2]
    C = pi.size // V
    np.testing.assert_array_equal(goff, np.arange(C + 1) * V)
    for c in range(C):
        np.testing.assert_array_equal(gidx[goff[c]:goff[c + 1]], np.sort(pi[c * V:(c + 1) * V]))


def test_aligned_subset_partition():
    for grid, cube, gp, rt in (((21, 45, 80), (3, 15, 16), (6, 23, 40), 4.0),
                               ((21, 136, 240), (3, 17, 24), (21, 30, 52), 4.0)):
        goff, gidx = oracle.aligned_subset(grid, cube, gp, rt)
        assert np.all(np.diff(goff) >= 0)
        assert np.unique(gidx).size == gidx.size            # at most one cube per token
        tg = gidx // (gp[1] * gp[2])
        assert np.all(rt * tg < grid[0])                   # only tokens inside the clip
        # every token whose frame maps inside the clip is listed
        assert gidx.size == int(np.sum(rt * np.arange(gp[0]) < grid[0])) * gp[1] * gp[2]


def test_block_attention_is_raster_windows():
    """Naive block attention (windows of V consecutive raster tokens) is the
    attention of raster-order tensors: a block-diagonal dense mask."""
    cfg = custom("blk", (2, 4, 6), (1, 2, 6), (0, 0, 0), heads=2, head_dim=64, dtype="f32")
    x = _f64(cfg)
    od, _ = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], None, None, None, cfg.V)
    N, V = cfg.N, cfg.V
    for h in range(cfg.heads):
        s = x["q_d"][:, h] @ x["k_d"][:, h].T / math.sqrt(cfg.head_dim)
        blk = np.arange(N) // V
        s = np.where(blk[:, None] == blk[None, :], s, -np.inf)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(od[:, h], p @ x["v_d"][:, h], rtol=1e-12, atol=1e-13)
    # cube (1, ch, W) makes the permutation the identity: raster blocks are cubes
    np.testing.assert_array_equal(oracle.cube_perm(cfg.grid, cfg.cube), np.arange(N))
