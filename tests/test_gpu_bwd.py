"""GPU parity of the attention backward (atlas_hier_attn_fwd + atlas_hier_attn_bwd)
against the fp64 oracle.

Small workloads (several 64-row tiles and 128-row blocks, ragged windows and
proxy lists, no-global, fp32 and bf16, head_dim 64 and 128) compare every
gradient element; the 4K workload (with its q/k outlier rows) compares
sampled dq rows, every dk/dv row of two windows, and the softmax-gradient sum
rules over all keys.

Tolerances, from the arithmetic of the kernels: P and dS are rounded to bf16
before their products (relative error <= 2^-9 each), D = dO.o uses the
bf16-rounded forward output, and each gradient is rounded once to the output
dtype (<= 2^-9).  These roundings are unbiased and add up like a random walk,
about 2e-3 of a gradient's L2 norm.  The test allows
  ||gpu - oracle||_2 <= 1e-2 ||oracle||_2  and
  max |gpu - oracle| <= 2e-2 max |oracle|   per gradient tensor;
the forward's log-sum-exp sums bf16-rounded probabilities, so
|lse_gpu - lse_oracle| <= 2^-8.
"""
import gc

import numpy as np
import pytest

import oracle
from workload import CONFIGS, bf16_bits_from_f32, custom, gen_grad_outputs, gen_inputs, outlier_rows

from ._gpu import dev, host, host_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BWD_REL_L2 = 1e-2
BWD_MAX_REL = 2e-2
LSE_ABS = 2.0 ** -8

BWD_CASES = [
    CONFIGS[0],                                                                  # tiny, fp32, D=64
    custom("bwd-bf16-ragged", (4, 12, 20), (2, 6, 10), (3, 10, 10), heads=3, head_dim=128),
    custom("bwd-bf16-d64", (3, 10, 20), (3, 10, 10), (1, 7, 11), heads=2, head_dim=64),
    custom("bwd-f32-d128", (2, 8, 12), (2, 4, 6), (1, 3, 5), heads=2, head_dim=128, dtype="f32"),
    custom("bwd-no-global", (2, 10, 20), (2, 10, 10), (0, 0, 0), heads=2, head_dim=128),
    custom("bwd-cube-4k", (6, 34, 48), (3, 17, 24), (3, 15, 26), heads=2, head_dim=128),
    custom("bwd-v1-g5", (2, 3, 4), (1, 1, 1), (1, 1, 5), heads=2, head_dim=64),
    custom("bwd-v7-h1-no-global", (1, 7, 3), (1, 7, 1), (0, 0, 0), heads=1, head_dim=128),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import windowed_global_local_amd as atlas
    atlas.load()


def atlas():
    import windowed_global_local_amd as m
    return m


def grad_errors(gpu, ref):
    g = oracle.to_f64(gpu) if gpu.dtype != np.float64 else gpu
    err = g - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(err)) / max(np.max(np.abs(ref)), 1e-300))
    return rel, mx


def assert_grad_close(gpu, ref, what):
    rel, mx = grad_errors(gpu, ref)
    say(f"{what}: rel_l2={rel:.3e} max_abs/max_ref={mx:.3e}")
    assert np.all(np.isfinite(oracle.to_f64(gpu))), f"{what}: non-finite values"
    assert rel <= BWD_REL_L2, f"{what}: rel L2 {rel} > {BWD_REL_L2}"
    assert mx <= BWD_MAX_REL, f"{what}: max abs {mx} of max|ref| > {BWD_MAX_REL}"


def run_fwd_bwd(cfg, x, dO, scale=0.0):
    """GPU forward with lse, then the backward; returns a dict of GPU tensors
    (scale 0: the default 1/sqrt(head_dim))."""
    A = atlas()
    G = cfg.G
    r = {"o_d": torch.empty_like(x["q_d"]), "o_g": torch.empty_like(x["q_g"]) if G else None,
         "lse_d": torch.empty(cfg.heads, cfg.N, dtype=torch.float32, device="cuda"),
         "lse_g": torch.empty(cfg.heads, G, dtype=torch.float32, device="cuda") if G else None}
    A.atlas_hier_attn_fwd(r["o_d"], r["o_g"], r["lse_d"], r["lse_g"], x["q_d"], x["k_d"], x["v_d"],
                          x["q_g"], x["k_g"], x["v_g"], cfg.grid, cfg.cube, cfg.gproxy, scale)
    nbytes = A.atlas_hier_attn_bwd_workspace_bytes(cfg.grid, cfg.cube, cfg.gproxy, cfg.heads,
                                                   cfg.head_dim)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    for n in ("dq_d", "dk_d", "dv_d"):
        r[n] = torch.full_like(x["q_d"], float("nan"))
    for n in ("dq_g", "dk_g", "dv_g"):
        r[n] = torch.full_like(x["q_g"], float("nan")) if G else None
    A.atlas_hier_attn_bwd(r["dq_d"], r["dk_d"], r["dv_d"], r["dq_g"], r["dk_g"], r["dv_g"],
                          x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                          r["o_d"], r["o_g"], dO["do_d"], dO["do_g"], r["lse_d"], r["lse_g"], ws,
                          cfg.grid, cfg.cube, cfg.gproxy, scale)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("cfg", BWD_CASES, ids=lambda c: c.name)
def test_bwd_matches_oracle(cfg):
    say("bwd", cfg.name, cfg.describe())
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    r = run_fwd_bwd(cfg, x, dO)
    # the forward with lse writes the same outputs as the plain forward
    od = torch.empty_like(x["q_d"])
    og = torch.empty_like(x["q_g"]) if cfg.G else None
    atlas().atlas_hier_attn(od, og, x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                            cfg.grid, cfg.cube, cfg.gproxy)
    torch.cuda.synchronize()
    assert torch.equal(od, r["o_d"]) and (og is None or torch.equal(og, r["o_g"]))
    say(cfg.name, "oracle backward")
    ref = oracle.hier_attn_bwd(ins["q_d"], ins["k_d"], ins["v_d"], gos["do_d"], ins["q_g"],
                               ins["k_g"], ins["v_g"], gos["do_g"], cfg.V)
    tags = ("d", "g") if cfg.G else ("d",)
    for t in tags:
        lse = r["lse_" + t].cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(lse - ref["lse_" + t])))
        say(f"{cfg.name} lse_{t}: max abs err {err:.3e}")
        assert err <= LSE_ABS
        for g in ("dq", "dk", "dv"):
            assert_grad_close(host(r[f"{g}_{t}"]), ref[f"{g}_{t}"], f"{cfg.name} {g}_{t}")


def test_bwd_twice_is_deterministic():
    cfg = BWD_CASES[1]
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    a = run_fwd_bwd(cfg, x, dO)
    b = run_fwd_bwd(cfg, x, dO)
    for n in ("dq_d", "dk_d", "dv_d", "dq_g", "dk_g", "dv_g"):
        assert torch.equal(a[n], b[n]), n


def test_bwd_very_negative_logits():
    """Queries whose every allowed logit is -180 (lse about -174): a key past
    the end of the list has P = exp(-lse) in the dq pass, which must not
    overflow.  V + G = 377 and G = 77 keys both end in partial 64-key tiles.
    Keys carry 4 in dimension 0 (others N(0,1)); the chosen queries are
    (-360, 0, ..., 0), so their logits are -360 * 4 / 8 for every key."""
    cfg = BWD_CASES[2]                       # bwd-bf16-d64: V = 300, G = 77, head_dim 64
    assert (cfg.V + cfg.G) % 64 and cfg.G % 64
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    four = bf16_bits_from_f32(np.float32([4.0]))[0]
    big = bf16_bits_from_f32(np.float32([-360.0]))[0]
    zero = bf16_bits_from_f32(np.float32([0.0]))[0]
    for n in ("k_d", "k_g"):
        ins[n] = ins[n].copy()
        ins[n][..., 0] = four
    qd, qg = ins["q_d"].copy(), ins["q_g"].copy()
    for q, rows in ((qd, slice(0, cfg.V)), (qg, slice(0, 5))):
        q[rows] = zero
        q[rows, :, 0] = big
    ins["q_d"], ins["q_g"] = qd, qg
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    r = run_fwd_bwd(cfg, x, dO)
    ref = oracle.hier_attn_bwd(ins["q_d"], ins["k_d"], ins["v_d"], gos["do_d"], ins["q_g"],
                               ins["k_g"], ins["v_g"], gos["do_g"], cfg.V)
    assert float(ref["lse_d"][:, : cfg.V].max()) < -150
    assert float(ref["lse_g"][:, :5].max()) < -150
    for t in ("d", "g"):
        lse = r["lse_" + t].cpu().numpy().astype(np.float64)
        assert float(np.max(np.abs(lse - ref["lse_" + t]))) <= LSE_ABS
        for g in ("dq", "dk", "dv"):
            assert_grad_close(host(r[f"{g}_{t}"]), ref[f"{g}_{t}"], f"negative logits {g}_{t}")


def test_bwd_argument_errors():
    cfg = BWD_CASES[1]
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    r = run_fwd_bwd(cfg, x, dO)
    A = atlas()
    small = torch.empty(8, dtype=torch.float32, device="cuda")
    with pytest.raises(A.AtlasError) as e:
        A.atlas_hier_attn_bwd(r["dq_d"], r["dk_d"], r["dv_d"], r["dq_g"], r["dk_g"], r["dv_g"],
                              x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                              r["o_d"], r["o_g"], dO["do_d"], dO["do_g"], r["lse_d"], r["lse_g"],
                              small, cfg.grid, cfg.cube, cfg.gproxy)
    assert e.value.code == -8
    ws = torch.empty(cfg.heads * (cfg.N + cfg.G), dtype=torch.float32, device="cuda")
    with pytest.raises(A.AtlasError) as e:   # dq_d written over q_d
        A.atlas_hier_attn_bwd(x["q_d"], r["dk_d"], r["dv_d"], r["dq_g"], r["dk_g"], r["dv_g"],
                              x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                              r["o_d"], r["o_g"], dO["do_d"], dO["do_g"], r["lse_d"], r["lse_g"],
                              ws, cfg.grid, cfg.cube, cfg.gproxy)
    assert e.value.code == -6


# ------------------------------------------------------- 720P, global keys

@pytest.mark.slow
def test_bwd_full_size_720p_global_keys():
    """dk/dv of sampled global keys at the 720P size, elementwise: each global
    key's gradient sums over all N + G = 81,120 queries (the dk/dv pass's
    global key blocks).  Keys include the last one, in the partial last
    128-key block."""
    cfg = next(c for c in CONFIGS if c.name == "720p-latent")
    rng = np.random.default_rng(7)
    say(cfg.name, "generating inputs and upstream gradients")
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    try:
        say(cfg.name, "forward + backward")
        r = run_fwd_bwd(cfg, x, dO)
        for h in (0, cfg.heads - 1):
            keys = np.concatenate([rng.choice(cfg.G - 1, 23, replace=False), [cfg.G - 1]])
            say(cfg.name, f"oracle dk/dv of {keys.size} global keys, head {h}")
            dk_ref, dv_ref = oracle.hier_attn_bwd_gkeys(ins["q_d"], ins["k_d"], ins["v_d"],
                                                        gos["do_d"], ins["q_g"], ins["k_g"],
                                                        ins["v_g"], gos["do_g"], cfg.V, h, keys)
            dk = host_rows(r["dk_g"], keys)[:, h]
            dv = host_rows(r["dv_g"], keys)[:, h]
            assert_grad_close(oracle.to_f64(dk), dk_ref, f"720P dk global keys, head {h}")
            assert_grad_close(oracle.to_f64(dv), dv_ref, f"720P dv global keys, head {h}")
    finally:
        del x, dO
        gc.collect()
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ 4K, sampled

@pytest.mark.slow
def test_bwd_full_size_4k_sampled():
    cfg = next(c for c in CONFIGS if c.name == "4k-latent")
    rng = np.random.default_rng(99)
    say(cfg.name, "generating inputs and upstream gradients")
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    try:
        say(cfg.name, "forward + backward")
        r = run_fwd_bwd(cfg, x, dO)
        N, V, G, H = cfg.N, cfg.V, cfg.G, cfg.heads
        # dq, lse of sampled query rows (detail, global, outlier rows)
        orows = np.nonzero(outlier_rows(cfg.seed, 0, N))[0]
        rows = np.concatenate([rng.integers(0, N, 384), rng.choice(orows, 64, replace=False),
                               rng.integers(0, G, 128)]).astype(np.int64)
        heads = rng.integers(0, H, rows.size).astype(np.int32)
        glob = np.concatenate([np.zeros(448), np.ones(128)]).astype(np.int8)
        say(cfg.name, f"oracle dq on {rows.size} sampled rows")
        dq_ref, lse_ref, _ = oracle.hier_attn_bwd_rows(ins["q_d"], ins["k_d"], ins["v_d"],
                                                       gos["do_d"], ins["q_g"], ins["k_g"],
                                                       ins["v_g"], gos["do_g"], V,
                                                       (rows, heads, glob))
        got = np.empty((rows.size, cfg.head_dim), dtype=np.float64)
        lse_got = np.empty(rows.size)
        for is_g, t in ((0, "d"), (1, "g")):
            m = glob == is_g
            hr = host_rows(r["dq_" + t], rows[m])
            got[m] = oracle.to_f64(hr[np.arange(hr.shape[0]), heads[m]])
            lse_got[m] = r["lse_" + t].cpu().numpy()[heads[m], rows[m]]
        assert float(np.max(np.abs(lse_got - lse_ref))) <= LSE_ABS
        assert_grad_close(got[glob == 0], dq_ref[glob == 0], "4K dq detail (sampled)")
        assert_grad_close(got[glob == 1], dq_ref[glob == 1], "4K dq global (sampled)")
        # dk, dv of every key of two windows
        for h, c in ((0, 0), (H - 1, cfg.C - 1)):
            say(cfg.name, f"oracle dk/dv of window {c}, head {h}")
            dk_ref, dv_ref = oracle.hier_attn_bwd_window(ins["q_d"], ins["k_d"], ins["v_d"],
                                                         gos["do_d"], ins["k_g"], ins["v_g"], V, h, c)
            sl = slice(c * V, (c + 1) * V)
            assert_grad_close(host(r["dk_d"][sl, h]), dk_ref, f"4K dk window {c} head {h}")
            assert_grad_close(host(r["dv_d"][sl, h]), dv_ref, f"4K dv window {c} head {h}")
        # sum rules over all keys, per head: sum dk = 0, sum dv = sum dO
        say(cfg.name, "sum rules over all keys")
        for h in range(H):
            dk = r["dk_d"][:, h].double().sum(0) + r["dk_g"][:, h].double().sum(0)
            dkabs = r["dk_d"][:, h].double().abs().sum(0) + r["dk_g"][:, h].double().abs().sum(0)
            dv = r["dv_d"][:, h].double().sum(0) + r["dv_g"][:, h].double().sum(0)
            dvabs = r["dv_d"][:, h].double().abs().sum(0) + r["dv_g"][:, h].double().abs().sum(0)
            do = dO["do_d"][:, h].double().sum(0) + dO["do_g"][:, h].double().sum(0)
            # each stored gradient carries at most ~2^-8 relative error
            assert bool(torch.all(dk.abs() <= 2.0 ** -7 * dkabs)), f"sum dk, head {h}"
            assert bool(torch.all((dv - do).abs() <= 2.0 ** -7 * dvabs + 1e-6)), f"sum dv, head {h}"
        say(cfg.name, "sum rules ok")
    finally:
        del x, dO
        gc.collect()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", BWD_CASES[:2], ids=lambda c: c.name)
def test_explicit_softmax_scale(cfg):
    """An explicit softmax scale (0.2, sharper than 1/sqrt(head_dim)) reaches
    the forward, its log-sum-exp and the backward the same way the oracle
    applies it.  fp32 inputs go through the matrix cores rounded to bf16; at
    this scale that rounding alone moves a logit by about 2^-8, so for them the
    oracle runs on the bf16-rounded operands (the arithmetic the kernels
    document) and the remaining error is that of the computation."""
    from ._gpu import assert_attn_close
    scale = 0.2
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    r = run_fwd_bwd(cfg, x, dO, scale)
    if cfg.dtype == "f32":
        ins = {k: oracle.round_bf16(v) for k, v in ins.items()}
        gos = {k: oracle.round_bf16(v) for k, v in gos.items()}
    o_ref = oracle.hier_attn(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"], ins["v_g"],
                             cfg.V, scale=scale)
    assert_attn_close(host(r["o_d"]), o_ref[0], f"{cfg.name} scale {scale} o_d")
    assert_attn_close(host(r["o_g"]), o_ref[1], f"{cfg.name} scale {scale} o_g")
    ref = oracle.hier_attn_bwd(ins["q_d"], ins["k_d"], ins["v_d"], gos["do_d"], ins["q_g"],
                               ins["k_g"], ins["v_g"], gos["do_g"], cfg.V, scale=scale)
    for t in ("d", "g"):
        lse = r["lse_" + t].cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(lse - ref["lse_" + t])))
        say(f"{cfg.name} scale {scale} lse_{t}: max abs {err:.3e}")
        assert err <= LSE_ABS, f"lse_{t}: {err}"
        for g in ("dq", "dk", "dv"):
            assert_grad_close(host(r[f"{g}_{t}"]), ref[f"{g}_{t}"], f"{cfg.name} scale {scale} {g}_{t}")
