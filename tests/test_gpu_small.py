"""GPU parity at sizes the oracle finishes in seconds: every call goes through
the C ABI (libatlas.so) and is compared element by element with the fp64
oracle on the same seeded inputs.  Shapes span several 64-key tiles, several
256-row query blocks, ragged tails, no global tokens, one cube covering the
whole volume, head_dim 64 and 128, fp32 and bf16, and q/k outlier rows.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from workload import CONFIGS, custom, gen_inputs
from workload.gen import bf16_bits_from_f32, f32_from_bf16_bits

from ._gpu import (assert_attn_close, assert_rope_close, dev, host, say)

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


TINY = CONFIGS[0]

ATTN_CASES = [
    TINY,
    custom("ragged-v300-g77", (2, 10, 30), (1, 10, 30), (1, 7, 11), heads=3, head_dim=128),
    custom("d64-v24-g135", (4, 6, 8), (2, 3, 4), (3, 5, 9), heads=2, head_dim=64),
    custom("no-global-v200", (2, 10, 20), (2, 5, 20), (0, 0, 0), heads=2, head_dim=128),
    custom("one-cube-full-attn", (2, 8, 33), (2, 8, 33), (0, 0, 0), heads=1, head_dim=128),
    custom("outliers-v1224-g260", (3, 17, 24), (3, 17, 24), (2, 10, 13), heads=2, head_dim=128,
           outliers=True),
    custom("f32-d128-v32-g6", (2, 4, 8), (1, 4, 8), (1, 2, 3), heads=2, head_dim=128, dtype="f32"),
    custom("v8-g600", (4, 4, 4), (1, 2, 4), (2, 15, 20), heads=2, head_dim=128),
    custom("d64-f32-v300", (2, 10, 30), (1, 10, 30), (1, 3, 3), heads=2, head_dim=64, dtype="f32"),
    custom("v1-g5", (2, 3, 4), (1, 1, 1), (1, 1, 5), heads=2, head_dim=128),
    # eight windows of V = 286 (a 30-row second query block: one partial wave)
    # and of V = 260 with no global keys (a 4-row second block)
    custom("v286-g60", (4, 22, 26), (2, 11, 13), (2, 5, 6), heads=2, head_dim=128),
    custom("v286-g260-outliers", (4, 22, 26), (2, 11, 13), (2, 10, 13), heads=2,
           head_dim=128, outliers=True),
    custom("d64-f32-v286", (4, 22, 26), (2, 11, 13), (2, 5, 6), heads=2, head_dim=64,
           dtype="f32"),
    custom("no-global-v260", (2, 13, 80), (1, 13, 20), (0, 0, 0), heads=2, head_dim=128),
]

COPY_CASES = [
    TINY,
    custom("bf16-h3", (3, 6, 10), (3, 2, 5), (0, 0, 0), heads=3, head_dim=128),
    custom("f32-d64-h5", (2, 4, 6), (1, 2, 3), (0, 0, 0), heads=5, head_dim=64, dtype="f32"),
    custom("identity", (2, 6, 8), (1, 3, 8), (0, 0, 0), heads=1, head_dim=64),
]

ROPE_CASES = [
    TINY,
    custom("bf16-frac-ratio", (6, 10, 12), (2, 5, 4), (2, 3, 5), r_t=4.0, heads=3, head_dim=128),
    custom("bf16-d64-rt8", (4, 8, 8), (2, 4, 4), (4, 3, 3), r_t=8.0, heads=2, head_dim=64),
    custom("f32-d128", (2, 6, 4), (1, 3, 2), (1, 2, 2), r_t=4.0, heads=2, head_dim=128, dtype="f32"),
    # a base other than 10000 and a fractional temporal scale
    dataclasses.replace(custom("bf16-theta500-rt2.5", (5, 6, 10), (5, 3, 5), (2, 3, 4), r_t=2.5,
                               heads=2, head_dim=128), theta=500.0),
]


def run_attn(cfg, x):
    od = torch.empty_like(x["q_d"])
    og = torch.empty_like(x["q_g"]) if cfg.G else None
    atlas().atlas_hier_attn(od, og, x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                            cfg.grid, cfg.cube, cfg.gproxy)
    torch.cuda.synchronize()
    return od, og


@pytest.mark.parametrize("cfg", ATTN_CASES, ids=lambda c: c.name)
def test_attention_parity(cfg):
    say("attention", cfg.name, cfg.describe())
    ins = gen_inputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    od, og = run_attn(cfg, x)
    ref_d, ref_g = oracle.hier_attn(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                    ins["v_g"], cfg.V)
    assert_attn_close(host(od), ref_d, f"{cfg.name} detail")
    if cfg.G:
        assert_attn_close(host(og), ref_g, f"{cfg.name} global")


@pytest.mark.parametrize("cfg", [
    custom("mask", (3, 8, 16), (3, 4, 8), (2, 5, 7), heads=2, head_dim=128),
    # eight windows of 286 keys, two query blocks each
    custom("mask-v286", (4, 22, 26), (2, 11, 13), (2, 5, 7), heads=2, head_dim=128),
], ids=lambda c: c.name)
def test_attention_deterministic_and_masks(cfg):
    say("mask invariants", cfg.describe())
    ins = gen_inputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    od, og = run_attn(cfg, x)
    od2, og2 = run_attn(cfg, x)
    assert torch.equal(od, od2) and torch.equal(og, og2), "not deterministic"
    V = cfg.V
    keep = slice(V, 2 * V)                       # cube 1 keeps its K/V
    kd, vd = x["k_d"].clone(), x["v_d"].clone()
    noise = torch.randn(kd.shape, generator=torch.Generator().manual_seed(3)).to(kd.dtype).cuda()
    kd = kd + noise
    vd = vd - noise
    kd[keep] = x["k_d"][keep]
    vd[keep] = x["v_d"][keep]
    y = dict(x, k_d=kd, v_d=vd)
    od3, og3 = run_attn(cfg, y)
    assert torch.equal(og3, og), "global outputs depend on detail K/V"
    assert torch.equal(od3[keep], od[keep]), "a cube's outputs depend on other cubes"
    assert not torch.equal(od3[:V], od[:V])


def logit_jump_inputs(cfg, seed=11):
    """q, k with base-2 logits a_i * h_j (plus noise), where a_i is a per-row
    scale in [-1.5, 1.5] and h_j a per-key height that steps up from one
    64-key tile of the key list [window | global] to the next."""
    rng = np.random.default_rng(seed)
    H, D, N, G = cfg.heads, cfg.head_dim, cfg.N, cfg.G
    u = rng.standard_normal((H, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    gamma = np.sqrt(np.sqrt(D) / np.log2(np.e))       # q.k / sqrt(D) * log2(e) = a h
    steps = np.array([0.0, 20.0, 45.0, 50.0, 100.0, 101.0, 190.0])
    h = np.repeat(steps, 64)[: N + G] + rng.uniform(-1.0, 0.0, N + G)
    a_d = rng.uniform(-1.5, 1.5, (N, H))
    a_g = rng.uniform(-1.5, 1.5, (G, H))

    def rows(scale):
        x = scale[:, :, None] * gamma * u[None] + 0.3 * rng.standard_normal((scale.shape[0], H, D))
        return bf16_bits_from_f32(x.astype(np.float32))

    ins = {"q_d": rows(a_d), "q_g": rows(a_g),
           "k_d": rows(np.repeat(h[:N, None], H, axis=1)), "k_g": rows(np.repeat(h[N:, None], H, axis=1)),
           "v_d": bf16_bits_from_f32(rng.standard_normal((N, H, D)).astype(np.float32)),
           "v_g": bf16_bits_from_f32(rng.standard_normal((G, H, D)).astype(np.float32))}
    return ins


def test_attention_logit_jumps_across_tiles():
    """The lazy rescale of the online softmax: from one key tile to the next
    the row max jumps by anything from 0 to about 190 (base-2 units), so some
    rows of a wave stay within the rescale headroom while others move the max,
    several times per row; every output checked against the fp64 oracle."""
    cfg = custom("logit-jumps", (1, 8, 32), (1, 8, 32), (1, 8, 24), heads=2, head_dim=128)
    ins = logit_jump_inputs(cfg)
    # the inputs do what they are for: per detail row, the largest base-2
    # logit of each 64-key tile (fp64 from the bf16 values), and its jumps
    q = f32_from_bf16_bits(ins["q_d"]).astype(np.float64)
    k = np.concatenate([f32_from_bf16_bits(ins["k_d"]), f32_from_bf16_bits(ins["k_g"])]).astype(np.float64)
    s2 = np.einsum("nhd,khd->hnk", q, k) / np.sqrt(cfg.head_dim) * np.log2(np.e)
    tmax = s2.reshape(cfg.heads, cfg.N, 7, 64).max(axis=3)
    jumps = np.diff(np.maximum.accumulate(tmax, axis=2), axis=2)
    assert (jumps > 64).any() and ((jumps > 4) & (jumps < 28)).any()
    assert (((jumps > 36).sum(axis=2)) >= 2).any()
    say("logit jumps", cfg.describe(), f"max jump {jumps.max():.1f}")
    x = {kk: dev(v) for kk, v in ins.items()}
    od, og = run_attn(cfg, x)
    ref_d, ref_g = oracle.hier_attn(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                    ins["v_g"], cfg.V)
    assert_attn_close(host(od), ref_d, "logit jumps detail")
    assert_attn_close(host(og), ref_g, "logit jumps global")


@pytest.mark.parametrize("cfg", COPY_CASES, ids=lambda c: c.name)
def test_reorder_unorder_bit_exact(cfg):
    say("reorder", cfg.name)
    ins = gen_inputs(cfg)
    src = ins["q_d"]
    x = dev(src)
    y = torch.empty_like(x)
    atlas().atlas_cube_reorder(y, x, cfg.grid, cfg.cube)
    z = torch.empty_like(x)
    atlas().atlas_cube_unorder(z, y, cfg.grid, cfg.cube)
    torch.cuda.synchronize()
    want = oracle.cube_reorder(src, cfg.grid, cfg.cube)
    np.testing.assert_array_equal(host(y), want)
    np.testing.assert_array_equal(host(z), src)
    np.testing.assert_array_equal(host(z), oracle.cube_unorder(want, cfg.grid, cfg.cube))


@pytest.mark.parametrize("cfg", ROPE_CASES, ids=lambda c: c.name)
def test_rope_parity(cfg):
    say("rope", cfg.name)
    ins = gen_inputs(cfg)
    qd = oracle.cube_reorder(ins["q_d"], cfg.grid, cfg.cube)        # detail in cube order
    xd, xg = dev(qd), dev(ins["q_g"])
    atlas().atlas_rope3d(xd, xg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    torch.cuda.synchronize()
    want_d = oracle.rope_detail(qd, np.arange(cfg.N), cfg.grid, cfg.cube, cfg.theta)
    want_g = oracle.rope_global(ins["q_g"], np.arange(cfg.G), cfg.grid, cfg.gproxy, cfg.r_t, cfg.theta)
    assert_rope_close(host(xd), want_d, f"{cfg.name} detail")
    assert_rope_close(host(xg), want_g, f"{cfg.name} global")
    # one side only
    xd2 = dev(qd)
    atlas().atlas_rope3d(xd2, None, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    xg2 = dev(ins["q_g"])
    atlas().atlas_rope3d(None, xg2, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    torch.cuda.synchronize()
    assert torch.equal(xd2, xd) and torch.equal(xg2, xg)


def test_rope_commutes_with_reorder_on_gpu():
    cfg = ROPE_CASES[1]
    ins = gen_inputs(cfg)
    x = dev(ins["k_d"])
    # path 1: reorder, then rotate in cube order
    a = torch.empty_like(x)
    atlas().atlas_cube_reorder(a, x, cfg.grid, cfg.cube)
    atlas().atlas_rope3d(a, None, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t)
    # path 2: rotate in raster order (cube = grid is the identity order), then reorder
    b0 = x.clone()
    atlas().atlas_rope3d(b0, None, cfg.grid, cfg.grid, cfg.gproxy, cfg.r_t)
    b = torch.empty_like(x)
    atlas().atlas_cube_reorder(b, b0, cfg.grid, cfg.cube)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def run_pipeline(cfg, x):
    """reorder q,k,v -> rope q,k -> attention -> unorder o (all on the GPU)."""
    A = atlas()
    qc, kc, vc = (torch.empty_like(x[n]) for n in ("q_d", "k_d", "v_d"))
    A.atlas_cube_reorder(qc, x["q_d"], cfg.grid, cfg.cube)
    A.atlas_cube_reorder(kc, x["k_d"], cfg.grid, cfg.cube)
    A.atlas_cube_reorder(vc, x["v_d"], cfg.grid, cfg.cube)
    qg = x["q_g"].clone() if cfg.G else None
    kg = x["k_g"].clone() if cfg.G else None
    A.atlas_rope3d(qc, qg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    A.atlas_rope3d(kc, kg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    oc = torch.empty_like(qc)
    og = torch.empty_like(qg) if cfg.G else None
    A.atlas_hier_attn(oc, og, qc, kc, vc, qg, kg, x["v_g"], cfg.grid, cfg.cube, cfg.gproxy)
    od = torch.empty_like(oc)
    A.atlas_cube_unorder(od, oc, cfg.grid, cfg.cube)
    torch.cuda.synchronize()
    return od, og


@pytest.mark.parametrize("cfg", [
    TINY,
    custom("e2e-bf16", (6, 10, 12), (3, 5, 4), (2, 3, 5), r_t=4.0, heads=2, head_dim=128),
    custom("e2e-bf16-rt8", (4, 8, 8), (2, 4, 4), (4, 3, 3), r_t=8.0, heads=2, head_dim=64),
], ids=lambda c: c.name)
def test_pipeline_end_to_end(cfg):
    say("pipeline", cfg.name)
    ins = gen_inputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    od, og = run_pipeline(cfg, x)
    ref_d, ref_g = oracle.pipeline_rows(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                        ins["v_g"], cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    assert_attn_close(host(od), ref_d, f"{cfg.name} e2e detail (raster order)")
    assert_attn_close(host(og), ref_g, f"{cfg.name} e2e global")
