"""Pins of the oracle's attention backward (CPU only).

The backward of "Technische Samenvatting: AtlasVid", Methodologie 2
(Asymmetrische Hierarchische Attention), is the gradient of the masked
softmax attention.  Nothing on the pages prints a gradient, so the oracle is
pinned to things outside itself:
  * automatic differentiation (PyTorch autograd, fp64, CPU) of the dense
    masked softmax over the concatenation [X_global; X_detail];
  * central finite differences of the oracle's own forward, which has its own
    pins;
  * the sum rules of softmax gradients: per head, the key gradients sum to
    zero and the value gradients sum to the sum of the upstream gradients;
    D_i = <dO_i, o_i>.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from workload import custom, gen_grad_outputs, gen_inputs

BWD_CASES = [
    custom("b1", (4, 8, 8), (2, 4, 4), (2, 4, 4), heads=2, head_dim=64, dtype="f32"),
    custom("b2", (3, 6, 4), (3, 2, 2), (1, 3, 2), heads=3, head_dim=128, dtype="bf16"),
    custom("b3", (2, 4, 6), (1, 4, 3), (0, 0, 0), heads=1, head_dim=64, dtype="f32"),
    custom("b4", (2, 6, 10), (2, 3, 5), (1, 2, 5), heads=2, head_dim=64, dtype="bf16"),
]


def _inputs(cfg):
    x = gen_inputs(cfg)
    x.update(gen_grad_outputs(cfg))
    return x


def _bwd(x, cfg, scale=None):
    return oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"],
                                x["q_g"], x["k_g"], x["v_g"], x["do_g"], cfg.V, scale=scale)


def autograd_dense(x, V, scale):
    """fp64 autograd of the dense masked softmax over [X_global; X_detail]."""
    import torch

    f = {k: (None if v is None else torch.from_numpy(oracle.to_f64(v))) for k, v in x.items()}
    G = 0 if f["q_g"] is None else f["q_g"].shape[0]
    N = f["q_d"].shape[0]
    cat = lambda a, b: b if a is None else torch.cat([a, b], 0)  # noqa: E731
    Q = cat(f["q_g"], f["q_d"]).clone().requires_grad_(True)
    K = cat(f["k_g"], f["k_d"]).clone().requires_grad_(True)
    Vv = cat(f["v_g"], f["v_d"]).clone().requires_grad_(True)
    dO = cat(f["do_g"], f["do_d"])
    L = G + N
    allow = torch.zeros(L, L, dtype=torch.bool)
    allow[:, :G] = True
    cube_of = torch.arange(N) // V
    allow[G:, G:] = cube_of[:, None] == cube_of[None, :]
    s = torch.einsum("ihd,jhd->hij", Q, K) * scale
    s = s.masked_fill(~allow, float("-inf"))
    lse = torch.logsumexp(s, -1)
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, -1), Vv)
    o.backward(dO)
    split = lambda t: (t[G:].numpy(), t[:G].numpy() if G else None)  # noqa: E731
    out = {}
    out["dq_d"], out["dq_g"] = split(Q.grad)
    out["dk_d"], out["dk_g"] = split(K.grad)
    out["dv_d"], out["dv_g"] = split(Vv.grad)
    lse = lse.detach().numpy()
    out["lse_d"], out["lse_g"] = lse[:, G:], (lse[:, :G] if G else None)
    out["o_d"], out["o_g"] = split(o.detach())
    return out


@pytest.mark.parametrize("cfg", BWD_CASES, ids=lambda c: c.name)
def test_bwd_matches_autograd_of_dense_masked_softmax(cfg):
    x = _inputs(cfg)
    scale = 1 / math.sqrt(cfg.head_dim)
    got = _bwd(x, cfg)
    want = autograd_dense(x, cfg.V, scale)
    for k in ("dq_d", "dk_d", "dv_d", "lse_d") + (("dq_g", "dk_g", "dv_g", "lse_g") if cfg.G else ()):
        np.testing.assert_allclose(got[k], want[k], rtol=1e-9, atol=1e-11, err_msg=k)
    if not cfg.G:
        assert got["dq_g"] is None and got["lse_g"] is None
    # the forward's lse output agrees with the backward's and with autograd's
    od, og, ld, lg = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                                      cfg.V, return_lse=True)
    np.testing.assert_allclose(ld, want["lse_d"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(od, want["o_d"], rtol=1e-10, atol=1e-12)
    if cfg.G:
        np.testing.assert_allclose(lg, want["lse_g"], rtol=1e-12, atol=1e-12)


def _loss(x, V, scale):
    od, og = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], V,
                              scale=scale)
    val = float(np.sum(od * x["do_d"]))
    if og is not None:
        val += float(np.sum(og * x["do_g"]))
    return val


def test_bwd_matches_central_differences_of_forward():
    cfg = custom("fd", (2, 4, 6), (1, 2, 3), (1, 2, 3), heads=2, head_dim=64, dtype="f32")
    raw = _inputs(cfg)
    x = {k: oracle.to_f64(v) for k, v in raw.items()}
    scale = 0.3           # an explicit scale, so the factor is exercised too
    got = _bwd(x, cfg, scale=scale)
    rng = np.random.default_rng(5)
    h = 1e-5
    for name, grad in (("q_d", "dq_d"), ("k_d", "dk_d"), ("v_d", "dv_d"),
                       ("q_g", "dq_g"), ("k_g", "dk_g"), ("v_g", "dv_g")):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x[name].shape)
            xp = dict(x)
            xp[name] = x[name].copy()
            xp[name][idx] += h
            lp = _loss(xp, cfg.V, scale)
            xp[name][idx] -= 2 * h
            lm = _loss(xp, cfg.V, scale)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - got[grad][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, got[grad][idx])


@pytest.mark.parametrize("cfg", BWD_CASES[:3], ids=lambda c: c.name)
def test_bwd_sum_rules(cfg):
    x = _inputs(cfg)
    r = _bwd(x, cfg)
    f = {k: (None if v is None else oracle.to_f64(v)) for k, v in x.items()}
    od, og = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V)
    # per head: sum over all keys of dk is 0; of dv, the sum of all upstream gradients
    dk_sum = r["dk_d"].sum(0) + (r["dk_g"].sum(0) if cfg.G else 0)
    dv_sum = r["dv_d"].sum(0) + (r["dv_g"].sum(0) if cfg.G else 0)
    do_sum = f["do_d"].sum(0) + (f["do_g"].sum(0) if cfg.G else 0)
    scale_k = np.abs(r["dk_d"]).sum(0).max()
    assert np.abs(dk_sum).max() <= 1e-12 * max(scale_k, 1.0)
    np.testing.assert_allclose(dv_sum, do_sum, rtol=1e-11, atol=1e-11)
    # each window's queries see only their window's detail keys: per window the
    # detail value gradients sum to sum_i dO_i * (mass of window keys for i)
    # -- checked in aggregate by the rule above; D_i = <dO_i, o_i>
    np.testing.assert_allclose(r["delta_d"].T, np.einsum("nhd,nhd->nh", f["do_d"], od),
                               rtol=1e-10, atol=1e-12)
    if cfg.G:
        np.testing.assert_allclose(r["delta_g"].T, np.einsum("nhd,nhd->nh", f["do_g"], og),
                                   rtol=1e-10, atol=1e-12)


def test_bwd_detail_keys_depend_only_on_own_window():
    """A detail key's gradients involve only the queries of its window."""
    cfg = BWD_CASES[3]
    x = _inputs(cfg)
    base = _bwd(x, cfg)
    y = dict(x)
    V = cfg.V
    for nm in ("q_d", "do_d"):
        y[nm] = x[nm].copy()
        y[nm][V:2 * V] = y[nm][V:2 * V][::-1]          # scramble window 1's queries
    r = _bwd(y, cfg)
    keep = np.ones(cfg.N, dtype=bool)
    keep[V:2 * V] = False
    np.testing.assert_array_equal(r["dk_d"][keep], base["dk_d"][keep])
    np.testing.assert_array_equal(r["dv_d"][keep], base["dv_d"][keep])


def test_bwd_sampled_functions_equal_full():
    cfg = BWD_CASES[3]
    x = _inputs(cfg)
    r = _bwd(x, cfg)
    rows = np.array([0, 7, cfg.N - 1, 3, 0, cfg.G - 1])
    hds = np.array([0, 1, 1, 0, 1, 0])
    isg = np.array([0, 0, 0, 1, 1, 1])
    dq, lse, dl = oracle.hier_attn_bwd_rows(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"],
                                            x["k_g"], x["v_g"], x["do_g"], cfg.V,
                                            (rows, hds, isg))
    for k in range(rows.size):
        tag = "g" if isg[k] else "d"
        np.testing.assert_allclose(dq[k], r["dq_" + tag][rows[k], hds[k]], rtol=1e-12, atol=1e-14)
        assert abs(lse[k] - r["lse_" + tag][hds[k], rows[k]]) <= 1e-12 * abs(lse[k]) + 1e-14
        assert abs(dl[k] - r["delta_" + tag][hds[k], rows[k]]) <= 1e-12 * abs(dl[k]) + 1e-14
    for head, c in ((0, 1), (1, cfg.C - 1)):
        dk, dv = oracle.hier_attn_bwd_window(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["k_g"],
                                             x["v_g"], cfg.V, head, c)
        s = slice(c * cfg.V, (c + 1) * cfg.V)
        np.testing.assert_allclose(dk, r["dk_d"][s, head], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dv, r["dv_d"][s, head], rtol=1e-11, atol=1e-13)
    keys = np.array([0, 3, cfg.G - 1])
    for head in range(cfg.heads):
        dk, dv = oracle.hier_attn_bwd_gkeys(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"],
                                            x["k_g"], x["v_g"], x["do_g"], cfg.V, head, keys)
        np.testing.assert_allclose(dk, r["dk_g"][keys, head], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dv, r["dv_g"][keys, head], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------- per-window subsets

def autograd_subset(x, V, scale, goff, gidx):
    """fp64 autograd of the subset attention written per window: window c's
    keys are its V detail keys followed by global rows gidx[goff[c]:goff[c+1]]
    (a row listed twice is two softmax terms); global queries see all global
    keys.  Gradients reach the global rows through the gather."""
    import torch

    f = {k: torch.from_numpy(oracle.to_f64(v)).requires_grad_(k[0] in "qkv")
         for k, v in x.items()}
    N, G = f["q_d"].shape[0], f["q_g"].shape[0]

    def attn(q, k, v):
        s = torch.einsum("ihd,jhd->hij", q, k) * scale
        return torch.einsum("hij,jhd->ihd", torch.softmax(s, -1), v)

    og = attn(f["q_g"], f["k_g"], f["v_g"])
    loss = (og * f["do_g"]).sum()
    od = []
    for c in range(N // V):
        rows = slice(c * V, (c + 1) * V)
        idx = torch.as_tensor(np.asarray(gidx[goff[c]:goff[c + 1]], dtype=np.int64))
        k = torch.cat([f["k_d"][rows], f["k_g"].index_select(0, idx)], 0)
        v = torch.cat([f["v_d"][rows], f["v_g"].index_select(0, idx)], 0)
        od.append(attn(f["q_d"][rows], k, v))
        loss = loss + (od[-1] * f["do_d"][rows]).sum()
    loss.backward()
    out = {f"d{n}_{t}": f[f"{n}_{t}"].grad.numpy() for n in "qkv" for t in "dg"}
    out["o_d"] = torch.cat(od, 0).detach().numpy()
    out["o_g"] = og.detach().numpy()
    return out


def test_bwd_subset_all_global_equals_plain():
    cfg = BWD_CASES[3]
    x = _inputs(cfg)
    goff = np.arange(cfg.C + 1, dtype=np.int64) * cfg.G
    gidx = np.tile(np.arange(cfg.G, dtype=np.int32), cfg.C)
    a = _bwd(x, cfg)
    b = oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"], x["k_g"],
                             x["v_g"], x["do_g"], cfg.V, subset=(goff, gidx))
    for k in ("dq_d", "dk_d", "dv_d", "dq_g", "dk_g", "dv_g", "lse_d", "lse_g", "delta_d", "delta_g"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-11, atol=1e-13, err_msg=k)


@pytest.mark.parametrize("seed", [0, 1])
def test_bwd_subset_matches_autograd(seed):
    cfg = BWD_CASES[3]                        # bf16, V = 30, G = 10, 2 heads
    x = _inputs(cfg)
    rng = np.random.default_rng(seed)
    lists = [rng.integers(0, cfg.G, size=int(rng.integers(0, 2 * cfg.G))) for _ in range(cfg.C)]
    lists[1] = np.zeros(0, dtype=np.int64)    # a window without global keys
    lists[0] = np.array([3, 3, 7])            # a key listed twice
    goff = np.concatenate([[0], np.cumsum([len(l) for l in lists])]).astype(np.int64)
    gidx = np.concatenate(lists).astype(np.int32)
    got = oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"], x["k_g"],
                               x["v_g"], x["do_g"], cfg.V, subset=(goff, gidx))
    want = autograd_subset(x, cfg.V, 1 / math.sqrt(cfg.head_dim), goff, gidx)
    for k in ("dq_d", "dk_d", "dv_d", "dq_g", "dk_g", "dv_g"):
        np.testing.assert_allclose(got[k], want[k], rtol=1e-9, atol=1e-11, err_msg=k)
    # the subset forward (repeated keys included) and its lse
    od, og, ld, _ = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                                     cfg.V, return_lse=True, subset=(goff, gidx))
    np.testing.assert_allclose(od, want["o_d"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(og, want["o_g"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["lse_d"], ld, rtol=1e-12, atol=1e-12)


# ------------------------------------------------- root-sum-square error scales

def dense_rss(x, V, scale, allow_fn=None):
    """Brute force, dense fp64: for every gradient element the square root of
    the sum of the squares of its terms -- scale dS_ij k_j for dq_i, scale
    dS_ij q_i for dk_j, P_ij dO_i for dv_j -- over the pairs the mask allows
    (rows [X_global; X_detail], the same dense mask as autograd_dense)."""
    f = {k: (None if v is None else oracle.to_f64(v)) for k, v in x.items()}
    G = 0 if f["q_g"] is None else f["q_g"].shape[0]
    N = f["q_d"].shape[0]
    cat = lambda a, b: b if a is None else np.concatenate([a, b], 0)  # noqa: E731
    Q, K, Vv, dO = (cat(f[a], f[b]) for a, b in (("q_g", "q_d"), ("k_g", "k_d"), ("v_g", "v_d"),
                                                  ("do_g", "do_d")))
    L = G + N
    allow = np.zeros((L, L), dtype=bool)
    allow[:, :G] = True
    cube_of = np.arange(N) // V
    allow[G:, G:] = cube_of[:, None] == cube_of[None, :]
    s = np.einsum("ihd,jhd->hij", Q, K) * scale
    s = np.where(allow[None], s, -np.inf)
    P = np.exp(s - s.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    dP = np.einsum("ihd,jhd->hij", dO, Vv)
    Dd = (P * dP).sum(-1, keepdims=True)
    dS = P * (dP - Dd)
    out = {
        "dq": scale * np.sqrt(np.einsum("hij,jhd->ihd", dS ** 2, K ** 2)),
        "dk": scale * np.sqrt(np.einsum("hij,ihd->jhd", dS ** 2, Q ** 2)),
        "dv": np.sqrt(np.einsum("hij,ihd->jhd", P ** 2, dO ** 2)),
    }
    return {f"{k}_d": v[G:] for k, v in out.items()} | {f"{k}_g": (v[:G] if G else None)
                                                         for k, v in out.items()}


@pytest.mark.parametrize("cfg", BWD_CASES, ids=lambda c: c.name)
def test_bwd_rss_matches_dense_brute_force(cfg):
    x = _inputs(cfg)
    scale = 1 / math.sqrt(cfg.head_dim)
    got = oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"], x["k_g"],
                               x["v_g"], x["do_g"], cfg.V, rss=True)
    want = dense_rss(x, cfg.V, scale)
    for k in ("dq_d", "dk_d", "dv_d") + (("dq_g", "dk_g", "dv_g") if cfg.G else ()):
        np.testing.assert_allclose(got[k], want[k], rtol=1e-9, atol=1e-13, err_msg=k)
    # a sum never exceeds the plain sum of its terms' magnitudes, and the
    # root-sum-square lies between that sum / sqrt(#terms) and the sum itself
    g = _bwd(x, cfg)
    assert np.all(np.abs(g["dv_d"]) <= np.sqrt(cfg.V + cfg.G) * got["dv_d"] * (1 + 1e-12) + 1e-300)


def test_bwd_rss_sampled_functions_equal_full():
    cfg = BWD_CASES[3]
    x = _inputs(cfg)
    r = oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"], x["k_g"],
                             x["v_g"], x["do_g"], cfg.V, rss=True)
    plain = _bwd(x, cfg)
    rows = np.array([0, 7, cfg.N - 1, 3, 0, cfg.G - 1])
    hds = np.array([0, 1, 1, 0, 1, 0])
    isg = np.array([0, 0, 0, 1, 1, 1])
    dq, lse, dl = oracle.hier_attn_bwd_rows(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"],
                                            x["k_g"], x["v_g"], x["do_g"], cfg.V,
                                            (rows, hds, isg), rss=True)
    for k in range(rows.size):
        tag = "g" if isg[k] else "d"
        np.testing.assert_allclose(dq[k], r["dq_" + tag][rows[k], hds[k]], rtol=1e-12, atol=1e-14)
        # lse and D are the plain ones in either mode
        assert abs(lse[k] - plain["lse_" + tag][hds[k], rows[k]]) <= 1e-12 * abs(lse[k]) + 1e-14
        assert abs(dl[k] - plain["delta_" + tag][hds[k], rows[k]]) <= 1e-12 * abs(dl[k]) + 1e-14
    for head, c in ((0, 1), (1, cfg.C - 1)):
        dk, dv = oracle.hier_attn_bwd_window(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["k_g"],
                                             x["v_g"], cfg.V, head, c, rss=True)
        s = slice(c * cfg.V, (c + 1) * cfg.V)
        np.testing.assert_allclose(dk, r["dk_d"][s, head], rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(dv, r["dv_d"][s, head], rtol=1e-11, atol=1e-14)
    keys = np.array([0, 3, cfg.G - 1])
    for head in range(cfg.heads):
        dk, dv = oracle.hier_attn_bwd_gkeys(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"],
                                            x["k_g"], x["v_g"], x["do_g"], cfg.V, head, keys,
                                            rss=True)
        np.testing.assert_allclose(dk, r["dk_g"][keys, head], rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(dv, r["dv_g"][keys, head], rtol=1e-11, atol=1e-14)


def test_bwd_rss_subset_all_global_equals_plain_mask():
    cfg = BWD_CASES[3]
    x = _inputs(cfg)
    goff = np.arange(cfg.C + 1, dtype=np.int64) * cfg.G
    gidx = np.tile(np.arange(cfg.G, dtype=np.int32), cfg.C)
    a = oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"], x["k_g"],
                             x["v_g"], x["do_g"], cfg.V, rss=True)
    b = oracle.hier_attn_bwd(x["q_d"], x["k_d"], x["v_d"], x["do_d"], x["q_g"], x["k_g"],
                             x["v_g"], x["do_g"], cfg.V, subset=(goff, gidx), rss=True)
    for k in ("dq_d", "dk_d", "dv_d", "dq_g", "dk_g", "dv_g"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-11, atol=1e-14, err_msg=k)
