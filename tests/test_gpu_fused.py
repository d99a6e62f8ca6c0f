"""GPU tests of the fused layout passes (the cube reorder fused into the RoPE
pass, the cube unorder fused into the attention epilogue).  Each fused call
must give the same bits as the separate calls it replaces, and the fused
pipeline must match the fp64 oracle to the attention tolerance.
"""
import numpy as np
import pytest

import oracle
from workload import CONFIGS, custom, gen_inputs

from ._gpu import assert_attn_close, assert_rope_close, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import windowed_global_local_amd as atlas
    atlas.load()


def atlas():
    import windowed_global_local_amd as m
    return m


FUSED_CASES = [
    CONFIGS[0],
    custom("fused-bf16-frac", (6, 10, 12), (2, 5, 4), (2, 3, 5), r_t=4.0, heads=3, head_dim=128),
    custom("fused-bf16-d64", (4, 8, 8), (2, 4, 4), (4, 3, 3), r_t=8.0, heads=2, head_dim=64),
    custom("fused-f32-d128", (2, 6, 4), (1, 3, 2), (1, 2, 2), r_t=4.0, heads=2, head_dim=128, dtype="f32"),
    custom("fused-ragged-v300-g77", (2, 10, 30), (1, 10, 30), (1, 7, 11), heads=3, head_dim=128),
    custom("fused-no-global", (2, 10, 20), (2, 5, 20), (0, 0, 0), heads=2, head_dim=128),
    custom("fused-v286", (4, 22, 26), (2, 11, 13), (2, 5, 6), r_t=4.0, heads=2, head_dim=128),
]


@pytest.mark.parametrize("cfg", FUSED_CASES, ids=lambda c: c.name)
def test_reorder_rope_fused_equals_separate(cfg):
    say("reorder+rope", cfg.name)
    ins = gen_inputs(cfg)
    A = atlas()
    x = dev(ins["k_d"])
    xg1 = dev(ins["k_g"]) if cfg.G else None
    xg2 = dev(ins["k_g"]) if cfg.G else None
    # separate: reorder, then rotate in cube order
    a = torch.empty_like(x)
    A.atlas_cube_reorder(a, x, cfg.grid, cfg.cube)
    A.atlas_rope3d(a, xg1, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    # fused
    b = torch.empty_like(x)
    A.atlas_cube_reorder_rope3d(b, x, xg2, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if cfg.G:
        assert torch.equal(xg1, xg2)
    # the raster input is left unchanged
    np.testing.assert_array_equal(host(x), ins["k_d"])
    # and against the oracle
    want = oracle.rope_detail(oracle.cube_reorder(ins["k_d"], cfg.grid, cfg.cube), np.arange(cfg.N),
                              cfg.grid, cfg.cube, cfg.theta)
    assert_rope_close(host(b), want, f"{cfg.name} fused detail")


def test_reorder_rope_fused_argument_errors():
    cfg = FUSED_CASES[1]
    A = atlas()
    x = torch.zeros(cfg.N, cfg.heads, cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AtlasError) as e:      # output aliases its raster input
        A.atlas_cube_reorder_rope3d(x, x, None, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t)
    assert e.value.name == "ATLAS_ERR_ALIAS"
    # output without an input: the C entry point itself refuses it
    lib = A.load()
    rc = lib.atlas_cube_reorder_rope3d(x.data_ptr(), None, None, A.dim3(cfg.grid), A.dim3(cfg.cube),
                                       A.dim3(cfg.gproxy), float(cfg.r_t), 10000.0, cfg.heads,
                                       cfg.head_dim, 0, None)
    assert rc == -1     # ATLAS_ERR_NULL
    # the Python wrapper refuses it before the call
    with pytest.raises(ValueError):
        A.atlas_cube_reorder_rope3d(x, None, None, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t)


@pytest.mark.parametrize("cfg", FUSED_CASES, ids=lambda c: c.name)
def test_attention_raster_equals_unorder(cfg):
    say("attn raster", cfg.name)
    ins = gen_inputs(cfg)
    A = atlas()
    x = {k: dev(v) for k, v in ins.items()}
    qc, kc, vc = (torch.empty_like(x[n]) for n in ("q_d", "k_d", "v_d"))
    for dst, n in ((qc, "q_d"), (kc, "k_d"), (vc, "v_d")):
        A.atlas_cube_reorder(dst, x[n], cfg.grid, cfg.cube)
    oc = torch.empty_like(qc)
    og1 = torch.empty_like(x["q_g"]) if cfg.G else None
    A.atlas_hier_attn(oc, og1, qc, kc, vc, x["q_g"], x["k_g"], x["v_g"], cfg.grid, cfg.cube, cfg.gproxy)
    od = torch.empty_like(oc)
    A.atlas_cube_unorder(od, oc, cfg.grid, cfg.cube)
    orr = torch.empty_like(oc)
    og2 = torch.empty_like(x["q_g"]) if cfg.G else None
    A.atlas_hier_attn_raster(orr, og2, qc, kc, vc, x["q_g"], x["k_g"], x["v_g"], cfg.grid, cfg.cube,
                             cfg.gproxy)
    torch.cuda.synchronize()
    assert torch.equal(orr, od)
    if cfg.G:
        assert torch.equal(og1, og2)


@pytest.mark.parametrize("cfg", [
    CONFIGS[0],
    custom("fused-e2e-bf16", (6, 10, 12), (3, 5, 4), (2, 3, 5), r_t=4.0, heads=2, head_dim=128),
    custom("fused-e2e-d64-rt8", (4, 8, 8), (2, 4, 4), (4, 3, 3), r_t=8.0, heads=2, head_dim=64),
], ids=lambda c: c.name)
def test_fused_pipeline_end_to_end(cfg):
    """raster q,k,v -> fused reorder+RoPE (q, k), reorder v -> attention with the
    raster epilogue, against the oracle pipeline."""
    say("fused pipeline", cfg.name)
    ins = gen_inputs(cfg)
    A = atlas()
    x = {k: dev(v) for k, v in ins.items()}
    qc, kc, vc = (torch.empty_like(x[n]) for n in ("q_d", "k_d", "v_d"))
    qg = x["q_g"].clone() if cfg.G else None
    kg = x["k_g"].clone() if cfg.G else None
    A.atlas_cube_reorder_rope3d(qc, x["q_d"], qg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    A.atlas_cube_reorder_rope3d(kc, x["k_d"], kg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    A.atlas_cube_reorder(vc, x["v_d"], cfg.grid, cfg.cube)
    od = torch.empty_like(qc)
    og = torch.empty_like(qg) if cfg.G else None
    A.atlas_hier_attn_raster(od, og, qc, kc, vc, qg, kg, x["v_g"], cfg.grid, cfg.cube, cfg.gproxy)
    torch.cuda.synchronize()
    ref_d, ref_g = oracle.pipeline_rows(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                        ins["v_g"], cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    assert_attn_close(host(od), ref_d, f"{cfg.name} fused e2e detail (raster order)")
    if cfg.G:
        assert_attn_close(host(og), ref_g, f"{cfg.name} fused e2e global")
