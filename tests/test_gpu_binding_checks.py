"""The Python binding rejects tensors whose token rows do not match the grid
or the proxy grid, window offset arrays without C + 1 entries and
log-sum-exp arrays of the wrong shape, before any launch (the C ABI sees
only pointers, so these sizes are the binding's to check)."""
import pytest

from workload import custom

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import windowed_global_local_amd as atlas
    atlas.load()


CFG = custom("checks", (2, 4, 8), (1, 2, 4), (1, 2, 4), heads=2, head_dim=64)


def _t(rows):
    return torch.zeros(rows, CFG.heads, CFG.head_dim, dtype=torch.bfloat16, device="cuda")


def test_row_counts_and_lists():
    import windowed_global_local_amd as A
    g, c, gp = CFG.grid, CFG.cube, CFG.gproxy
    N, G, C = CFG.N, CFG.G, CFG.C
    d, gl, short = _t(N), _t(G), _t(N - 1)
    with pytest.raises(ValueError, match="token rows"):
        A.atlas_cube_reorder(short, short, g, c)
    with pytest.raises(ValueError, match="token rows"):
        A.atlas_rope3d(d, _t(G + 1), g, c, gp, CFG.r_t)
    with pytest.raises(ValueError, match="token rows"):
        A.atlas_cube_reorder_rope3d(short, short, gl, g, c, gp, CFG.r_t)
    with pytest.raises(ValueError, match="token rows"):
        A.atlas_hier_attn(d, gl, d, short, d, gl, gl, gl, g, c, gp)
    with pytest.raises(ValueError, match="token rows"):
        A.atlas_hier_attn_raster(d, gl, d, d, d, gl, gl, _t(G - 1), g, c, gp)
    goff = torch.zeros(C, dtype=torch.int32, device="cuda")              # one short
    gidx = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="C \\+ 1"):
        A.atlas_hier_attn_subset(d, gl, d, d, d, gl, gl, gl, goff, gidx, g, c, gp)
    lse_d = torch.zeros(CFG.heads, N, dtype=torch.float32, device="cuda")
    lse_g = torch.zeros(CFG.heads, G, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="C \\+ 1"):
        A.atlas_hier_attn_subset_fwd(d, gl, lse_d, lse_g, d, d, d, gl, gl, gl, goff, gidx, g, c, gp)
    ws = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    bad_lse = torch.zeros(CFG.heads, G + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="lse_global"):
        A.atlas_hier_attn_bwd(d, d, d, gl, gl, gl, d, d, d, gl, gl, gl, d, gl, d, gl, lse_d, bad_lse,
                              ws, g, c, gp)
    with pytest.raises(ValueError, match="token rows"):
        A.atlas_hier_attn_bwd(d, d, d, gl, gl, gl, d, d, d, gl, gl, gl, short, gl, d, gl, lse_d, lse_g,
                              ws, g, c, gp)
    with pytest.raises(ValueError, match="C \\+ 1"):
        A.atlas_hier_attn_subset_bwd(d, d, d, gl, gl, gl, d, d, d, gl, gl, gl, d, gl, d, gl, lse_d,
                                     lse_g, goff, gidx, ws, g, c, gp)
