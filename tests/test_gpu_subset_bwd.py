"""GPU parity of the backward of the per-window subset mask
(atlas_hier_attn_subset_fwd + atlas_hier_attn_subset_bwd) against the fp64
oracle: random lists with an empty window, a key listed twice and keys
listed by several windows, an index outside [0, G) (the oracle sees the
same lists over global tensors with one zero row appended at index G, whose
gradient is dropped), all-global lists, and the co-located lists of
"Technische Samenvatting: AtlasVid", Methodologie 2, at small sizes.
Tolerances as for the plain backward.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from workload import custom, gen_grad_outputs, gen_inputs

from ._gpu import dev, host, say
from .test_gpu_bwd import LSE_ABS, assert_grad_bound, assert_grad_close, derived_bounds

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


CASES = [
    custom("sbwd-bf16-ragged", (4, 12, 20), (2, 6, 10), (3, 10, 10), heads=3, head_dim=128),
    custom("sbwd-bf16-d64", (3, 10, 20), (3, 10, 10), (1, 7, 11), heads=2, head_dim=64),
    custom("sbwd-f32-d128", (2, 8, 12), (2, 4, 6), (1, 3, 5), heads=2, head_dim=128, dtype="f32"),
]


def run_subset_bwd(cfg, x, dO, goff, gidx):
    A = atlas()
    G = cfg.G
    goff_t = torch.as_tensor(np.asarray(goff, dtype=np.int32), device="cuda")
    gidx_t = torch.as_tensor(np.asarray(gidx, dtype=np.int32), device="cuda")
    r = {"o_d": torch.empty_like(x["q_d"]), "o_g": torch.empty_like(x["q_g"]),
         "lse_d": torch.empty(cfg.heads, cfg.N, dtype=torch.float32, device="cuda"),
         "lse_g": torch.empty(cfg.heads, G, dtype=torch.float32, device="cuda")}
    A.atlas_hier_attn_subset_fwd(r["o_d"], r["o_g"], r["lse_d"], r["lse_g"], x["q_d"], x["k_d"],
                                 x["v_d"], x["q_g"], x["k_g"], x["v_g"], goff_t, gidx_t, cfg.grid,
                                 cfg.cube, cfg.gproxy)
    nbytes = A.atlas_hier_attn_subset_bwd_workspace_bytes(cfg.grid, cfg.cube, cfg.gproxy, cfg.heads,
                                                          cfg.head_dim)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    for n in ("dq_d", "dk_d", "dv_d"):
        r[n] = torch.full_like(x["q_d"], float("nan"))
    for n in ("dq_g", "dk_g", "dv_g"):
        r[n] = torch.full_like(x["q_g"], float("nan"))
    A.atlas_hier_attn_subset_bwd(r["dq_d"], r["dk_d"], r["dv_d"], r["dq_g"], r["dk_g"], r["dv_g"],
                                 x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                                 r["o_d"], r["o_g"], dO["do_d"], dO["do_g"], r["lse_d"], r["lse_g"],
                                 goff_t, gidx_t, ws, cfg.grid, cfg.cube, cfg.gproxy)
    torch.cuda.synchronize()
    return r


def check_against_oracle(cfg, ins, gos, r, goff, gidx, detail_only=False):
    ref = oracle.hier_attn_bwd(ins["q_d"], ins["k_d"], ins["v_d"], gos["do_d"], ins["q_g"],
                               ins["k_g"], ins["v_g"], gos["do_g"], cfg.V, subset=(goff, gidx))
    bounds = None
    if cfg.dtype == "bf16":
        rb = dict(r)
        extra = ins["q_g"].shape[0] - r["o_g"].shape[0]
        if extra:   # the appended zero rows: their dO is zero, so any output serves
            rb["o_g"] = torch.cat([r["o_g"], r["o_g"].new_zeros((extra,) + r["o_g"].shape[1:])])
        bounds = derived_bounds(cfg, ins, gos, rb, ref, subset=(goff, gidx))
    for t in ("d",) if detail_only else ("d", "g"):
        lse = r["lse_" + t].cpu().numpy().astype(np.float64)
        assert float(np.max(np.abs(lse - ref["lse_" + t]))) <= LSE_ABS, f"lse_{t}"
        for g in ("dq", "dk", "dv"):
            what = f"{cfg.name} subset {g}_{t}"
            if bounds is None:
                assert_grad_close(host(r[f"{g}_{t}"]), ref[f"{g}_{t}"], what)
            else:
                assert_grad_bound(host(r[f"{g}_{t}"]), ref[f"{g}_{t}"], bounds[f"{g}_{t}"], what)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_subset_bwd_random_lists(cfg):
    say("subset bwd", cfg.name, cfg.describe())
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    rng = np.random.default_rng(11)
    lists = []
    for c in range(cfg.C):
        n = int(rng.integers(0, min(cfg.G, 150) + 1)) if c % 3 else 0   # every third window empty
        lists.append(np.sort(rng.choice(cfg.G, size=n, replace=False)))
    if cfg.C > 1:
        lists[1] = np.concatenate([lists[1], [5, 5]])                    # a key listed twice more
    goff = np.concatenate([[0], np.cumsum([len(l) for l in lists])]).astype(np.int64)
    gidx = np.concatenate(lists).astype(np.int32)
    r = run_subset_bwd(cfg, x, dO, goff, gidx)
    check_against_oracle(cfg, ins, gos, r, goff, gidx)


def test_subset_bwd_out_of_range_index():
    """An index outside [0, G) is a zero key and value row of the forward; in
    the oracle it is row G of global tensors with a zero row appended.  That
    row would also be a key of the oracle's global queries, so only the detail
    side (lse, dq, dk, dv of the detail rows) is compared."""
    cfg = CASES[0]
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    rng = np.random.default_rng(12)
    lists = [np.sort(rng.choice(cfg.G, size=40, replace=False)) for _ in range(cfg.C)]
    goff = np.concatenate([[0], np.cumsum([len(l) for l in lists])]).astype(np.int64)
    gidx = np.concatenate(lists).astype(np.int32)
    bad = gidx.copy()
    bad[goff[1] + 3] = cfg.G + 11
    bad[goff[2]] = -4
    r = run_subset_bwd(cfg, x, dO, goff, bad)
    emu = gidx.copy()
    emu[goff[1] + 3] = cfg.G
    emu[goff[2]] = cfg.G
    ins2, gos2 = dict(ins), dict(gos)
    for n, src in (("q_g", ins), ("k_g", ins), ("v_g", ins), ("do_g", gos)):
        z = np.zeros((1,) + src[n].shape[1:], dtype=src[n].dtype)
        (gos2 if n == "do_g" else ins2)[n] = np.concatenate([src[n], z], 0)
    check_against_oracle(cfg, ins2, gos2, r, goff, emu, detail_only=True)


def test_subset_bwd_all_global_and_aligned():
    A = atlas()
    cfg = custom("sbwd-aligned", (6, 12, 16), (3, 6, 8), (2, 6, 8), r_t=4.0, heads=2, head_dim=128)
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    # all-global lists: the plain backward's gradients, to the tolerance
    goff = np.arange(cfg.C + 1, dtype=np.int64) * cfg.G
    gidx = np.tile(np.arange(cfg.G, dtype=np.int32), cfg.C)
    r = run_subset_bwd(cfg, x, dO, goff, gidx)
    check_against_oracle(cfg, ins, gos, r, goff, gidx)
    # the co-located lists
    goff, gidx = A.atlas_aligned_subset(cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t)
    assert gidx.size > 0
    r = run_subset_bwd(cfg, x, dO, goff.astype(np.int64), gidx)
    check_against_oracle(cfg, ins, gos, r, goff.astype(np.int64), gidx)


@pytest.mark.slow
def test_subset_bwd_full_size_720p_aligned():
    """The 720P workload with the co-located lists, every element of two whole
    heads (the first and the last): heads are independent, so the oracle runs
    on one-head slices of the inputs."""
    from workload import CONFIGS
    A = atlas()
    cfg = next(c for c in CONFIGS if c.name == "720p-latent")
    say(cfg.name, "generating inputs and upstream gradients")
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    goff, gidx = A.atlas_aligned_subset(cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t)
    goff = goff.astype(np.int64)
    say(cfg.name, f"{gidx.size} listed rows; subset forward + backward")
    r = run_subset_bwd(cfg, x, dO, goff, gidx)
    del x, dO
    for h in (0, cfg.heads - 1):
        say(cfg.name, f"oracle subset backward, head {h}")
        one = {k: np.ascontiguousarray(v[:, h:h + 1]) for k, v in ins.items()}
        gone = {k: np.ascontiguousarray(v[:, h:h + 1]) for k, v in gos.items()}
        ref = oracle.hier_attn_bwd(one["q_d"], one["k_d"], one["v_d"], gone["do_d"], one["q_g"],
                                   one["k_g"], one["v_g"], gone["do_g"], cfg.V,
                                   scale=1.0 / np.sqrt(cfg.head_dim), subset=(goff, gidx))
        cfg1 = dataclasses.replace(cfg, heads=1)
        r1 = {"o_d": r["o_d"][:, h:h + 1], "o_g": r["o_g"][:, h:h + 1]}
        bounds = derived_bounds(cfg1, one, gone, r1, ref, subset=(goff, gidx))
        for t in ("d", "g"):
            lse = r["lse_" + t][h].cpu().numpy().astype(np.float64)
            assert float(np.max(np.abs(lse - ref["lse_" + t][0]))) <= LSE_ABS, f"lse_{t}, head {h}"
            for g in ("dq", "dk", "dv"):
                got = r[f"{g}_{t}"][:, h:h + 1].float().cpu().numpy().astype(np.float64)
                assert_grad_bound(got, ref[f"{g}_{t}"], bounds[f"{g}_{t}"],
                                  f"720P aligned subset {g}_{t}, head {h}")


def test_subset_bwd_all_lists_empty():
    """G > 0 but no window lists a global row (an empty index array): detail
    queries see their window only, global queries all G; the global keys'
    dk/dv come from the global queries alone."""
    cfg = CASES[0]
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    goff = np.zeros(cfg.C + 1, dtype=np.int64)
    gidx = np.zeros(0, dtype=np.int32)
    r = run_subset_bwd(cfg, x, dO, goff, gidx)
    check_against_oracle(cfg, ins, gos, r, goff, gidx)


def test_subset_bwd_one_window_lists_all():
    """One window lists every global row, in reverse order, the others none."""
    cfg = CASES[1]
    ins = gen_inputs(cfg)
    gos = gen_grad_outputs(cfg)
    x = {k: dev(v) for k, v in ins.items()}
    dO = {k: dev(v) for k, v in gos.items()}
    c = cfg.C // 2
    goff = np.concatenate([np.zeros(c + 1), np.full(cfg.C - c, cfg.G)]).astype(np.int64)
    gidx = np.arange(cfg.G - 1, -1, -1, dtype=np.int32)
    r = run_subset_bwd(cfg, x, dO, goff, gidx)
    check_against_oracle(cfg, ins, gos, r, goff, gidx)
