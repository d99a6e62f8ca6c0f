"""The no-allocation backward entry point (atlas_hier_attn_bwd_noalloc)
against the workspace entry point (atlas_hier_attn_bwd), through the C ABI.

Two calls in a row on one GPU, the second on a smaller problem, so the fixed
device array still holds the first call's D rows when the second starts; a
third call has no global tokens.  The cube-mask backward is deterministic, so
every gradient must match the workspace entry point's bit for bit.  A problem
whose workspace exceeds the array is rejected before any launch.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import windowed_global_local_amd as atlas
    atlas.load()


def _inputs(grid, cube, gproxy, heads, hd, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    N = int(np.prod(grid))
    G = int(np.prod(gproxy))

    def t(n):
        return torch.randn(n, heads, hd, generator=gen).to(dtype).to("cuda")

    x = {n: t(N) for n in ("q_d", "k_d", "v_d", "do_d")}
    x.update({n: t(G) if G else None for n in ("q_g", "k_g", "v_g", "do_g")})
    return x, N, G


def _case(grid, cube, gproxy, heads, hd, dtype, seed):
    import windowed_global_local_amd as A
    print(f"[gpu-test] noalloc bwd grid={grid} cube={cube} gproxy={gproxy} heads={heads} "
          f"hd={hd} dtype={dtype}", flush=True)
    x, N, G = _inputs(grid, cube, gproxy, heads, hd, dtype, seed)
    o_d = torch.empty_like(x["q_d"])
    o_g = torch.empty_like(x["q_g"]) if G else None
    lse_d = torch.empty(heads, N, dtype=torch.float32, device="cuda")
    lse_g = torch.empty(heads, G, dtype=torch.float32, device="cuda") if G else None
    A.atlas_hier_attn_fwd(o_d, o_g, lse_d, lse_g, x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"],
                          x["v_g"], grid, cube, gproxy)

    def grads():
        d = [torch.empty_like(x[n]) for n in ("q_d", "k_d", "v_d")]
        g = [torch.empty_like(x[n]) if G else None for n in ("q_g", "k_g", "v_g")]
        return d + g

    ins = (x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], o_d, o_g, x["do_d"], x["do_g"],
           lse_d, lse_g)
    ref = grads()
    ws = torch.empty(A.atlas_hier_attn_bwd_workspace_bytes(grid, cube, gproxy, heads, hd) // 4,
                     dtype=torch.float32, device="cuda")
    A.atlas_hier_attn_bwd(*ref, *ins, ws, grid, cube, gproxy)
    got = grads()
    A.atlas_hier_attn_bwd_noalloc(*got, *ins, grid, cube, gproxy)
    torch.cuda.synchronize()
    names = ("dq_d", "dk_d", "dv_d", "dq_g", "dk_g", "dv_g")
    for n, r, g in zip(names, ref, got):
        if r is None:
            continue
        assert torch.isfinite(r.float()).all(), n
        iv = torch.int16 if r.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(r.view(iv), g.view(iv)), f"{n} differs from the workspace entry point"


def test_noalloc_matches_workspace_entry_point():
    _case((4, 16, 24), (2, 8, 8), (2, 4, 6), 3, 128, torch.bfloat16, 11)
    _case((2, 4, 8), (1, 4, 4), (1, 2, 3), 2, 128, torch.bfloat16, 12)
    _case((2, 4, 8), (2, 2, 4), (0, 0, 0), 1, 64, torch.float32, 13)


def test_noalloc_rejects_oversize_before_launch():
    import windowed_global_local_amd as A
    from windowed_global_local_amd import Dim3
    lib = A.load()
    # long 4K latent grid, 40 heads: 4 * 40 * (N + G) bytes > the fixed array
    grid, cube, gp = Dim3(42, 136, 240), Dim3(3, 17, 24), Dim3(21, 30, 52)
    need = lib.atlas_hier_attn_bwd_workspace_bytes(grid, cube, gp, 40, 128)
    assert need > A.NOALLOC_SCRATCH_BYTES
    fake = [0x7F0000000000 + (i << 36) for i in range(18)]
    rc = lib.atlas_hier_attn_bwd_noalloc(*fake, grid, cube, gp, 40, 128, 0.0, 0, None)
    assert rc == -9
