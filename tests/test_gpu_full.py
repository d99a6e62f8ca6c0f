"""GPU parity at the full sizes of the five large workloads (720P, 1080P, 4K
with q/k outlier rows, long 4K, 8K), in the launch configuration the bench times.

  * reorder / unorder: the whole tensor, bit-exact against the oracle's
    permutation (the gather X[pi] is compared on the device);
  * RoPE: sampled detail (cube order) and global token rows, <= 1 bf16 ulp;
  * attention: every row of two whole windows (first window / first head,
    last window / last head), 1024 random detail (row, head) pairs, 256 random
    global pairs and, on the outlier workload, 256 outlier query rows; max abs
    <= 2e-2 and relative L2 <= 5e-3 against the fp64 oracle;
  * end to end (long 4K, 720P and 8K): reorder x3 -> RoPE x2 -> attention ->
    unorder, sampled raster rows against the oracle's row-wise pipeline.
"""
import gc

import numpy as np
import pytest

import oracle
from workload import CONFIGS, gen_inputs, outlier_rows

from ._gpu import assert_attn_close, assert_rope_close, dev, host_rows, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")

BIG = CONFIGS[1:]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import windowed_global_local_amd as atlas
    atlas.load()


def atlas():
    import windowed_global_local_amd as m
    return m


def attn_selection(cfg, rng):
    N, V, G, H = cfg.N, cfg.V, cfg.G, cfg.heads
    rows, heads, glob = [], [], []
    for c, h in ((0, 0), (cfg.C - 1, H - 1)):
        rows.append(np.arange(c * V, (c + 1) * V))
        heads.append(np.full(V, h))
        glob.append(np.zeros(V))
    rows.append(rng.integers(0, N, 1024))
    heads.append(rng.integers(0, H, 1024))
    glob.append(np.zeros(1024))
    rows.append(rng.integers(0, G, 256))
    heads.append(rng.integers(0, H, 256))
    glob.append(np.ones(256))
    if cfg.outliers:
        orows = np.nonzero(outlier_rows(cfg.seed, 0, N))[0]
        pick = rng.choice(orows, size=min(256, orows.size), replace=False)
        rows.append(pick)
        heads.append(rng.integers(0, H, pick.size))
        glob.append(np.zeros(pick.size))
    return (np.concatenate(rows).astype(np.int64), np.concatenate(heads).astype(np.int32),
            np.concatenate(glob).astype(np.int8))


def gather_sel(od, og, sel):
    rows, heads, glob = sel
    out = []
    for is_g, o in ((0, od), (1, og)):
        m = glob == is_g
        if not m.any():
            continue
        r = host_rows(o, rows[m])                   # [n, heads, D]
        out.append((m, r[np.arange(r.shape[0]), heads[m]]))
    D = od.shape[2]
    res = np.empty((rows.size, D), dtype=out[0][1].dtype)
    for m, v in out:
        res[m] = v
    return res


def check_attention(cfg, ins, x, rng):
    say(cfg.name, "attention", cfg.describe())
    od = torch.empty_like(x["q_d"])
    og = torch.empty_like(x["q_g"])
    atlas().atlas_hier_attn(od, og, x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                            cfg.grid, cfg.cube, cfg.gproxy)
    torch.cuda.synchronize()
    sel = attn_selection(cfg, rng)
    got = gather_sel(od, og, sel)
    say(cfg.name, f"oracle on {sel[0].size} sampled rows")
    ref = oracle.hier_attn(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"], ins["v_g"],
                           cfg.V, sel=sel)
    g = sel[2] == 1
    assert_attn_close(got[~g], ref[~g], f"{cfg.name} detail (sampled)")
    assert_attn_close(got[g], ref[g], f"{cfg.name} global (sampled)")
    del od, og


def check_reorder_and_rope(cfg, ins, x, rng):
    say(cfg.name, "reorder/unorder full tensor")
    pi = torch.as_tensor(oracle.cube_perm(cfg.grid, cfg.cube), device="cuda")
    y = torch.empty_like(x["q_d"])
    atlas().atlas_cube_reorder(y, x["q_d"], cfg.grid, cfg.cube)
    want = x["q_d"].index_select(0, pi)
    assert torch.equal(y.view(torch.int16), want.view(torch.int16)), "reorder mismatch"
    del want
    z = torch.empty_like(y)
    atlas().atlas_cube_unorder(z, y, cfg.grid, cfg.cube)
    assert torch.equal(z.view(torch.int16), x["q_d"].view(torch.int16)), "unorder mismatch"
    del z

    say(cfg.name, "rope (sampled rows)")
    qg = x["q_g"].clone()
    atlas().atlas_rope3d(y, qg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    torch.cuda.synchronize()
    pi_h = pi.cpu().numpy()
    p = np.unique(np.concatenate([[0, cfg.N - 1], rng.integers(0, cfg.N, 2048)]))
    want_d = oracle.rope_detail(ins["q_d"][pi_h[p]], p, cfg.grid, cfg.cube, cfg.theta)
    assert_rope_close(host_rows(y, p), want_d, f"{cfg.name} rope detail")
    r = np.unique(np.concatenate([[0, cfg.G - 1], rng.integers(0, cfg.G, 1024)]))
    want_g = oracle.rope_global(ins["q_g"][r], r, cfg.grid, cfg.gproxy, cfg.r_t, cfg.theta)
    assert_rope_close(host_rows(qg, r), want_g, f"{cfg.name} rope global")
    del y, qg, pi


def check_pipeline(cfg, ins, x, rng):
    say(cfg.name, "end to end: reorder x3, rope x2, attention, unorder")
    A = atlas()
    qc, kc, vc = (torch.empty_like(x[n]) for n in ("q_d", "k_d", "v_d"))
    A.atlas_cube_reorder(qc, x["q_d"], cfg.grid, cfg.cube)
    A.atlas_cube_reorder(kc, x["k_d"], cfg.grid, cfg.cube)
    A.atlas_cube_reorder(vc, x["v_d"], cfg.grid, cfg.cube)
    qg, kg = x["q_g"].clone(), x["k_g"].clone()
    A.atlas_rope3d(qc, qg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    A.atlas_rope3d(kc, kg, cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta)
    oc = torch.empty_like(qc)
    og = torch.empty_like(qg)
    A.atlas_hier_attn(oc, og, qc, kc, vc, qg, kg, x["v_g"], cfg.grid, cfg.cube, cfg.gproxy)
    del qc, kc, vc
    od = torch.empty_like(oc)
    A.atlas_cube_unorder(od, oc, cfg.grid, cfg.cube)
    torch.cuda.synchronize()
    del oc
    n_d, n_g = 768, 128
    rows = np.concatenate([rng.integers(0, cfg.N, n_d), rng.integers(0, cfg.G, n_g)]).astype(np.int64)
    heads = rng.integers(0, cfg.heads, n_d + n_g).astype(np.int32)
    glob = np.concatenate([np.zeros(n_d), np.ones(n_g)]).astype(np.int8)
    sel = (rows, heads, glob)
    got = gather_sel(od, og, sel)
    say(cfg.name, f"oracle pipeline on {rows.size} sampled raster rows")
    ref = oracle.pipeline_rows(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"], ins["v_g"],
                               cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, cfg.theta, sel=sel)
    g = glob == 1
    assert_attn_close(got[~g], ref[~g], f"{cfg.name} e2e detail (sampled, raster order)")
    assert_attn_close(got[g], ref[g], f"{cfg.name} e2e global (sampled)")
    del od, og


@pytest.mark.parametrize("cfg", BIG, ids=lambda c: c.name)
def test_full_size(cfg):
    rng = np.random.default_rng(1234)
    say(cfg.name, "generating inputs")
    ins = gen_inputs(cfg)
    say(cfg.name, "uploading")
    x = {k: dev(v) for k, v in ins.items()}
    try:
        check_reorder_and_rope(cfg, ins, x, rng)
        check_attention(cfg, ins, x, rng)
        if cfg.name in ("long-4k-latent", "720p-latent", "8k-latent"):
            check_pipeline(cfg, ins, x, rng)
    finally:
        del x
        gc.collect()
        torch.cuda.empty_cache()
