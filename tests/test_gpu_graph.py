"""HIP graph capture of the path and of the backward.

The path (fused cube reorder + RoPE of q and of k, cube reorder of v, the
attention with the raster epilogue) and the backward (D rows, dq, dk/dv) are
launched through the C-ABI while a stream captures them into a graph.  Each
graph is replayed several times, with eager work, a poisoning of the outputs
and synchronisations between replays, and every replay must equal the eager
result bit for bit (every kernel here is deterministic).  No call of the
library allocates, sets memory or synchronises, so capture needs nothing
else.  The RoPE pass rotates the global q/k in place: the global inputs are
restored eagerly before each replay, outside the graph.
"""
import pytest

from workload import CONFIGS, custom, gen_grad_outputs, gen_inputs

from ._gpu import dev, say

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


GRAPH_CASES = [
    custom("graph-bf16-ragged", (4, 12, 20), (2, 6, 10), (3, 10, 10), heads=3, head_dim=128),
    next(c for c in CONFIGS if c.name == "720p-latent"),
]


def _capture(fn):
    """fn() captured into a graph on a side stream (after one eager run there,
    as capture requires)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg", GRAPH_CASES, ids=lambda c: c.name)
def test_path_and_backward_graph_replays(cfg):
    A = atlas()
    say("graph", cfg.name, cfg.describe())
    x = {k: dev(v) for k, v in gen_inputs(cfg).items()}
    dO = {k: dev(v) for k, v in gen_grad_outputs(cfg).items()}
    g_, c_, gp = cfg.grid, cfg.cube, cfg.gproxy
    qc, kc, vc = (torch.empty_like(x["q_d"]) for _ in range(3))
    qg, kg = x["q_g"].clone(), x["k_g"].clone()
    od, og = torch.empty_like(x["q_d"]), torch.empty_like(x["q_g"])
    oc, ogb = torch.empty_like(x["q_d"]), torch.empty_like(x["q_g"])
    lse_d = torch.empty(cfg.heads, cfg.N, dtype=torch.float32, device="cuda")
    lse_g = torch.empty(cfg.heads, cfg.G, dtype=torch.float32, device="cuda")
    grads = [torch.empty_like(x["q_d"]) for _ in range(3)] + [torch.empty_like(x["q_g"]) for _ in range(3)]
    nbytes = A.atlas_hier_attn_bwd_workspace_bytes(g_, c_, gp, cfg.heads, cfg.head_dim)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

    def restore():
        qg.copy_(x["q_g"])
        kg.copy_(x["k_g"])

    def path():
        A.atlas_cube_reorder_rope3d(qc, x["q_d"], qg, g_, c_, gp, cfg.r_t, cfg.theta)
        A.atlas_cube_reorder_rope3d(kc, x["k_d"], kg, g_, c_, gp, cfg.r_t, cfg.theta)
        A.atlas_cube_reorder(vc, x["v_d"], g_, c_)
        A.atlas_hier_attn_raster(od, og, qc, kc, vc, qg, kg, x["v_g"], g_, c_, gp)

    def backward():
        A.atlas_hier_attn_fwd(oc, ogb, lse_d, lse_g, qc, kc, vc, qg, kg, x["v_g"], g_, c_, gp)
        A.atlas_hier_attn_bwd(*grads, qc, kc, vc, qg, kg, x["v_g"], oc, ogb, dO["do_d"], dO["do_g"],
                              lse_d, lse_g, ws, g_, c_, gp)

    # eager reference
    restore()
    path()
    backward()
    torch.cuda.synchronize()
    ref_path = [t.clone() for t in (od, og, qc, kc, vc, qg, kg)]
    ref_bwd = [t.clone() for t in (oc, ogb, lse_d, lse_g, *grads)]

    restore()
    g_path = _capture(path)
    g_bwd = _capture(backward)          # on the rotated q/k the path left behind
    for rep in range(3):
        # eager work between replays: poison every output, restore the inputs
        for t in (od, og, qc, kc, vc, oc, ogb, lse_d, lse_g, *grads):
            t.fill_(float("nan"))
        restore()
        torch.cuda.synchronize()
        g_path.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip((od, og, qc, kc, vc, qg, kg), ref_path)):
            assert torch.equal(a, b), f"path replay {rep}, output {i}"
        g_bwd.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip((oc, ogb, lse_d, lse_g, *grads), ref_bwd)):
            assert torch.equal(a, b), f"backward replay {rep}, output {i}"
    say(cfg.name, "3 replays of each graph equal the eager results")


def test_subset_forward_backward_graph_replays():
    """The subset forward with lse and its backward (accumulators cleared by a
    fill kernel inside the call) captured and replayed three times.  Every
    output equals the eager result bit for bit except dk_g and dv_g, whose
    fp32 atomic sums may round differently with the order of the adds."""
    import numpy as np
    A = atlas()
    cfg = GRAPH_CASES[0]
    x = {k: dev(v) for k, v in gen_inputs(cfg).items()}
    dO = {k: dev(v) for k, v in gen_grad_outputs(cfg).items()}
    g_, c_, gp = cfg.grid, cfg.cube, cfg.gproxy
    rng = np.random.default_rng(5)
    lists = [np.sort(rng.choice(cfg.G, size=int(rng.integers(0, 60)), replace=False)) for _ in range(cfg.C)]
    goff = torch.as_tensor(np.concatenate([[0], np.cumsum([len(l) for l in lists])]).astype(np.int32),
                           device="cuda")
    gidx = torch.as_tensor(np.concatenate(lists).astype(np.int32), device="cuda")
    od, og = torch.empty_like(x["q_d"]), torch.empty_like(x["q_g"])
    lse_d = torch.empty(cfg.heads, cfg.N, dtype=torch.float32, device="cuda")
    lse_g = torch.empty(cfg.heads, cfg.G, dtype=torch.float32, device="cuda")
    grads = [torch.empty_like(x["q_d"]) for _ in range(3)] + [torch.empty_like(x["q_g"]) for _ in range(3)]
    nbytes = A.atlas_hier_attn_subset_bwd_workspace_bytes(g_, c_, gp, cfg.heads, cfg.head_dim)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

    def run():
        A.atlas_hier_attn_subset_fwd(od, og, lse_d, lse_g, x["q_d"], x["k_d"], x["v_d"], x["q_g"],
                                     x["k_g"], x["v_g"], goff, gidx, g_, c_, gp)
        A.atlas_hier_attn_subset_bwd(*grads, x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                                     od, og, dO["do_d"], dO["do_g"], lse_d, lse_g, goff, gidx, ws,
                                     g_, c_, gp)

    run()
    torch.cuda.synchronize()
    outs = (od, og, lse_d, lse_g, *grads)
    ref = [t.clone() for t in outs]
    graph = _capture(run)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            if i in (8, 9):      # dk_g, dv_g
                d = (a.float() - b.float()).norm() / b.float().norm()
                assert float(d) <= 1e-3, f"subset replay {rep}, output {i}: rel {float(d)}"
            else:
                assert torch.equal(a, b), f"subset replay {rep}, output {i}"
    say(cfg.name, "3 replays of the subset forward + backward graph match the eager results")
