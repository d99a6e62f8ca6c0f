"""Pins of the fp64 oracle against what the pages and mathematics fix.

Every test here runs on the CPU.  None of them re-types the oracle's formula:
each compares it with an independent construction (brute-force enumeration, a
hand-worked fixture, a dense masked softmax over the concatenated sequence, a
complex-number rotation), an invariant (bijection, round trip, norm
preservation, relative-position identity, mask one-wayness) or a closed form
(uniform softmax, dominant logit, log-sum-exp merge).

Operations pinned (sources cited by page title and section):
  * cube reorder -- "Technische Samenvatting: AtlasVid", Methodologie 1, Fase 2;
  * temporally scaled 3D RoPE and position alignment -- same page, Methodologie 1
    Fase 1 and Methodologie 2 Positie-uitlijning;
  * asymmetric global-local mask -- same page, Methodologie 2, Asymmetrische
    Hierarchische Attention.
"""
import math
import os

import numpy as np
import pytest

import oracle
from workload import bf16_bits_from_f32, custom, f32_from_bf16_bits, gen_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

GRIDS = [
    ((4, 8, 8), (2, 4, 4)),
    ((2, 2, 4), (1, 2, 2)),
    ((6, 10, 12), (3, 5, 4)),
    ((3, 4, 5), (3, 4, 5)),     # one cube = whole volume
    ((4, 6, 10), (1, 3, 10)),   # cube spans full rows: identity
    ((5, 3, 7), (1, 1, 1)),     # 1-token cubes: identity
]


# ------------------------------------------------------------------ permutation

def brute_force_perm(grid, cube):
    """Enumerate cubes in raster order, then tokens of each cube in raster order."""
    T, H, W = grid
    ct, ch, cw = cube
    out = []
    for a in range(T // ct):
        for b in range(H // ch):
            for e in range(W // cw):
                for dt in range(ct):
                    for dh in range(ch):
                        for dw in range(cw):
                            t, h, w = a * ct + dt, b * ch + dh, e * cw + dw
                            out.append((t * H + h) * W + w)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("grid,cube", GRIDS)
def test_perm_matches_brute_force(grid, cube):
    np.testing.assert_array_equal(oracle.cube_perm(grid, cube), brute_force_perm(grid, cube))


def test_perm_golden_fixture():
    fields = {}
    with open(os.path.join(GOLDEN, "cube_perm_2x2x4_c1x2x2.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            fields[k] = [int(x) for x in v]
    pi = oracle.cube_perm(tuple(fields["grid"]), tuple(fields["cube"]))
    np.testing.assert_array_equal(pi, np.array(fields["pi"]))


@pytest.mark.parametrize("grid,cube", GRIDS)
def test_perm_is_bijection_and_blocks_are_boxes(grid, cube):
    pi = oracle.cube_perm(grid, cube)
    T, H, W = grid
    ct, ch, cw = cube
    N, V = T * H * W, ct * ch * cw
    np.testing.assert_array_equal(np.sort(pi), np.arange(N))
    t, h, w = pi // (H * W), (pi // W) % H, pi % W
    for c in range(N // V):
        s = slice(c * V, (c + 1) * V)
        # the V consecutive positions cover exactly one ct x ch x cw box
        assert t[s].max() - t[s].min() == ct - 1 and t[s].min() % ct == 0
        assert h[s].max() - h[s].min() == ch - 1 and h[s].min() % ch == 0
        assert w[s].max() - w[s].min() == cw - 1 and w[s].min() % cw == 0
        assert len({(a, b, e) for a, b, e in zip(t[s], h[s], w[s])}) == V
    for p in range(0, N, max(1, N // 37)):
        r = oracle.cube_src(p, grid, cube)
        assert oracle.cube_dst(r, grid, cube) == p


@pytest.mark.parametrize("grid,cube", [((3, 4, 5), (3, 4, 5)), ((4, 6, 10), (1, 3, 10)),
                                       ((5, 3, 7), (1, 1, 1)), ((2, 6, 8), (1, 2, 8))])
def test_perm_identity_special_cases(grid, cube):
    T, H, W = grid
    np.testing.assert_array_equal(oracle.cube_perm(grid, cube), np.arange(T * H * W))


@pytest.mark.parametrize("grid,cube", GRIDS[:3])
def test_reorder_unorder_round_trip(grid, cube):
    rng = np.random.default_rng(1)
    N = grid[0] * grid[1] * grid[2]
    x = rng.integers(0, 2**16, size=(N, 3, 8), dtype=np.uint16)
    y = oracle.cube_reorder(x, grid, cube)
    np.testing.assert_array_equal(oracle.cube_unorder(y, grid, cube), x)
    np.testing.assert_array_equal(oracle.cube_reorder(oracle.cube_unorder(x, grid, cube), grid, cube), x)
    np.testing.assert_array_equal(y, x[brute_force_perm(grid, cube)])


# ------------------------------------------------------------------ bf16 rounding

def test_round_bf16_ties_and_no_double_rounding():
    one = 1.0
    u = 2.0 ** -7                  # bf16 ulp at 1
    cases = {
        one: one,
        one + u / 2: one,                        # tie -> even (1.0)
        one + 3 * u / 2: one + 2 * u,            # tie -> even (1 + 2u)
        one + u / 2 + 2.0 ** -40: one + u,       # just above the tie: up
        one + u / 2 - 2.0 ** -40: one,           # just below: down
        -(one + 3 * u / 2): -(one + 2 * u),
        2.0 ** -130: 2.0 ** -130,                # subnormal, exact
        3.0 * 2.0 ** -135: 2.0 ** -133,          # 0.75 subnormal quanta -> 1 quantum
    }
    for x, want in cases.items():
        got = f32_from_bf16_bits(oracle.round_bf16(np.array([x])))[0]
        assert float(got) == want, (x, float(got), want)
    # exact bf16 values map to themselves; fp32 values agree with the textbook
    # integer round-half-even on the fp32 bit pattern
    rng = np.random.default_rng(5)
    xs = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(xs.astype(np.float64)), bf16_bits_from_f32(xs))
    ex = f32_from_bf16_bits(bf16_bits_from_f32(xs)).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(ex), bf16_bits_from_f32(ex.astype(np.float32)))


# ------------------------------------------------------------------ RoPE

def complex_rope(x, pos, theta=10000.0):
    """Textbook RoPE as complex multiplication per axis sub-band (RoFormer):
    pairs (2i, 2i+1) are the real and imaginary parts of z_i, and
    z_i <- z_i * exp(1j * p_axis(i) * omega_i)."""
    n, heads, D = x.shape
    nhw = D // 6
    nt = D // 2 - 2 * nhw
    bands = [(0, nt), (1, nhw), (2, nhw)]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    out = []
    start = 0
    for axis, na in bands:
        j = np.arange(na)
        omega = theta ** (-(j / na))
        ang = pos[:, axis][:, None] * omega[None, :]
        out.append(z[..., start:start + na] * np.exp(1j * ang)[:, None, :])
        start += na
    zr = np.concatenate(out, axis=-1)
    res = np.empty_like(x)
    res[..., 0::2] = zr.real
    res[..., 1::2] = zr.imag
    return res


@pytest.mark.parametrize("D", [64, 128, 6, 12])
def test_rope_matches_complex_form(D):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 3, D))
    pos = rng.uniform(-50, 300, size=(9, 3))
    np.testing.assert_allclose(oracle.rope_rows(x, pos), complex_rope(x, pos), rtol=0, atol=1e-12)


def test_rope_closed_form_small_head():
    # D = 6: one pair per axis, each at frequency theta^0 = 1
    x = np.array([[[1.0, 0.0, 1.0, 0.0, 1.0, 0.0]]])
    pos = np.array([[1.0, 2.0, 3.0]])
    want = [math.cos(1), math.sin(1), math.cos(2), math.sin(2), math.cos(3), math.sin(3)]
    np.testing.assert_allclose(oracle.rope_rows(x, pos)[0, 0], want, atol=1e-15)


@pytest.mark.parametrize("D", [64, 128])
def test_rope_invariants(D):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 2, D))
    pos = rng.integers(0, 200, size=(16, 3)).astype(np.float64)
    y = oracle.rope_rows(x, pos)
    # pair norms preserved
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-13)
    # position zero is the identity
    np.testing.assert_array_equal(oracle.rope_rows(x, np.zeros((16, 3))), x)
    # the inverse rotation recovers x
    np.testing.assert_allclose(oracle.rope_rows(y, -pos), x, atol=1e-12)
    # relative position: <R(p)q, R(p')k> = <R(p - p')q, k>
    q, k = x[:8], x[8:]
    p1, p2 = pos[:8], pos[8:]
    lhs = np.einsum("nhd,nhd->nh", oracle.rope_rows(q, p1), oracle.rope_rows(k, p2))
    rhs = np.einsum("nhd,nhd->nh", oracle.rope_rows(q, p1 - p2), k)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_rope_axis_split_128():
    # the temporal band is elements 0..43, height 44..85, width 86..127
    x = np.ones((1, 1, 128))
    for axis, lo, hi in [(0, 0, 44), (1, 44, 86), (2, 86, 128)]:
        pos = np.zeros((1, 3))
        pos[0, axis] = 7.0
        changed = np.nonzero(np.abs(oracle.rope_rows(x, pos) - x)[0, 0] > 0)[0]
        assert changed.min() == lo and changed.max() == hi - 1


def test_rope_rt_one_global_equals_detail():
    # with r_t = 1 and the proxy grid equal to the detail grid, global
    # coordinates are the integer detail coordinates (standard 3D RoPE)
    grid, cube = (4, 6, 8), (2, 3, 4)
    N = 4 * 6 * 8
    rng = np.random.default_rng(4)
    x = rng.standard_normal((N, 2, 64))
    g = oracle.rope_global(x, np.arange(N), grid, grid, 1.0)
    d_raster = oracle.rope_detail(x, np.arange(N), grid, grid)   # cube = grid: identity order
    np.testing.assert_allclose(g, d_raster, atol=1e-13)
    np.testing.assert_allclose(g, complex_rope(x, np.stack(np.unravel_index(np.arange(N), grid), 1)
                                               .astype(np.float64)), atol=1e-12)


def test_rope_temporal_scale_and_alignment():
    # proxy at half spatial resolution and r_t = 4: proxy token (tg, hg, wg)
    # rotates like a detail token at (4 tg, 2 hg, 2 wg)
    grid, gproxy = (16, 8, 12), (4, 4, 6)
    G = 4 * 4 * 6
    rng = np.random.default_rng(6)
    x = rng.standard_normal((G, 2, 128))
    g = oracle.rope_global(x, np.arange(G), grid, gproxy, 4.0)
    tg, hg, wg = np.unravel_index(np.arange(G), gproxy)
    raster = (4 * tg * 8 + 2 * hg) * 12 + 2 * wg
    d = oracle.rope_detail(x, raster, grid, grid)
    np.testing.assert_allclose(g, d, atol=1e-13)
    # fractional ratio (e.g. 45/23) is used as is
    pos = oracle.pos_global([23 * 40 + 40 + 1], (21, 45, 80), (6, 23, 40), 4.0)
    np.testing.assert_allclose(pos[0], [4.0, 45 / 23, 2.0 * 1], rtol=1e-15)


def test_rope_commutes_with_reorder():
    grid, cube = (4, 8, 8), (2, 4, 4)
    N = 256
    rng = np.random.default_rng(7)
    x = rng.standard_normal((N, 2, 64))
    a = oracle.rope_detail(oracle.cube_reorder(x, grid, cube), np.arange(N), grid, cube)
    b = oracle.cube_reorder(oracle.rope_detail(x, np.arange(N), grid, grid), grid, cube)
    np.testing.assert_allclose(a, b, atol=0, rtol=0)


# ------------------------------------------------------------------ attention

def dense_masked_attention(qd, kd, vd, qg, kg, vg, V, scale):
    """Textbook masked softmax over the concatenated sequence [X_global; X_detail]:
    a global row may see global columns only (global -> detail is -inf);
    a detail row sees the global columns and the detail columns of its cube."""
    N, heads, D = qd.shape
    G = 0 if qg is None else qg.shape[0]
    cat = lambda a, b: b if a is None else np.concatenate([a, b], 0)  # noqa: E731
    Q, K, Vv = cat(qg, qd), cat(kg, kd), cat(vg, vd)
    L = G + N
    allow = np.zeros((L, L), dtype=bool)
    allow[:G, :G] = True
    cube_of = np.arange(N) // V
    allow[G:, :G] = True
    allow[G:, G:] = cube_of[:, None] == cube_of[None, :]
    out = np.empty_like(Q)
    for h in range(heads):
        s = (Q[:, h] @ K[:, h].T) * scale
        s = np.where(allow, s, -np.inf)
        s = s - s.max(1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(1, keepdims=True)
        out[:, h] = p @ Vv[:, h]
    return out[G:], (out[:G] if G else None)


def _f64_inputs(cfg):
    ins = gen_inputs(cfg)
    return {k: (None if v is None else oracle.to_f64(v)) for k, v in ins.items()}


@pytest.mark.parametrize("cfg", [
    custom("t1", (4, 8, 8), (2, 4, 4), (2, 4, 4), heads=2, head_dim=64, dtype="f32"),
    custom("t2", (3, 6, 4), (3, 2, 2), (1, 3, 2), heads=3, head_dim=128, dtype="bf16"),
    custom("t3", (2, 4, 6), (1, 4, 3), (0, 0, 0), heads=1, head_dim=64, dtype="f32"),
])
def test_attention_matches_dense_masked_softmax(cfg):
    x = _f64_inputs(cfg)
    scale = 1 / math.sqrt(cfg.head_dim)
    od, og = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V)
    wd, wg = dense_masked_attention(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"],
                                    cfg.V, scale)
    np.testing.assert_allclose(od, wd, rtol=1e-11, atol=1e-12)
    if cfg.G:
        np.testing.assert_allclose(og, wg, rtol=1e-11, atol=1e-12)


def test_attention_bf16_bits_equal_upcast():
    cfg = custom("b", (2, 4, 4), (1, 2, 4), (1, 2, 2), heads=2, head_dim=64, dtype="bf16")
    raw = gen_inputs(cfg)
    up = {k: oracle.to_f64(v) for k, v in raw.items()}
    a = oracle.hier_attn(raw["q_d"], raw["k_d"], raw["v_d"], raw["q_g"], raw["k_g"], raw["v_g"], cfg.V)
    b = oracle.hier_attn(up["q_d"], up["k_d"], up["v_d"], up["q_g"], up["k_g"], up["v_g"], cfg.V)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_single_cube_no_global_is_full_attention():
    rng = np.random.default_rng(8)
    N, heads, D = 48, 2, 64
    q, k, v = (rng.standard_normal((N, heads, D)) for _ in range(3))
    od, og = oracle.hier_attn(q, k, v, None, None, None, V=N)
    assert og is None
    for h in range(heads):
        s = q[:, h] @ k[:, h].T / math.sqrt(D)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(od[:, h], p @ v[:, h], rtol=1e-12, atol=1e-13)


def test_window_brute_force_per_cube():
    cfg = custom("w", (4, 8, 8), (2, 4, 4), (2, 4, 4), heads=2, head_dim=64, dtype="f32")
    x = _f64_inputs(cfg)
    od, _ = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V)
    V = cfg.V
    for c in range(cfg.C):
        s = slice(c * V, (c + 1) * V)
        for h in range(cfg.heads):
            K = np.concatenate([x["k_d"][s, h], x["k_g"][:, h]])
            Vv = np.concatenate([x["v_d"][s, h], x["v_g"][:, h]])
            logits = x["q_d"][s, h] @ K.T / 8.0
            p = np.exp(logits - logits.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            np.testing.assert_allclose(od[s, h], p @ Vv, rtol=1e-12, atol=1e-13)


def test_mask_one_way_and_cube_independence():
    cfg = custom("m", (4, 8, 8), (2, 4, 4), (2, 4, 4), heads=2, head_dim=64, dtype="f32")
    x = _f64_inputs(cfg)
    od, og = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V)
    rng = np.random.default_rng(9)
    kd2 = x["k_d"].copy()
    vd2 = x["v_d"].copy()
    V = cfg.V
    # perturb every cube except cube 3
    mask = np.ones(cfg.N, bool)
    mask[3 * V:4 * V] = False
    kd2[mask] += rng.standard_normal(kd2[mask].shape)
    vd2[mask] += rng.standard_normal(vd2[mask].shape)
    od2, og2 = oracle.hier_attn(x["q_d"], kd2, vd2, x["q_g"], x["k_g"], x["v_g"], V)
    np.testing.assert_array_equal(og2, og)                         # global never sees detail
    np.testing.assert_array_equal(od2[3 * V:4 * V], od[3 * V:4 * V])  # cube 3 never sees others
    assert not np.allclose(od2[:V], od[:V])


def test_log_sum_exp_merge():
    cfg = custom("l", (2, 4, 8), (2, 2, 4), (1, 3, 5), heads=1, head_dim=64, dtype="f32")
    x = _f64_inputs(cfg)
    od, _ = oracle.hier_attn(x["q_d"], x["k_d"], x["v_d"], x["q_g"], x["k_g"], x["v_g"], cfg.V)
    V, sc = cfg.V, 1 / 8.0
    for c in range(cfg.C):
        s = slice(c * V, (c + 1) * V)
        q = x["q_d"][s, 0]

        def part(K, Vv):
            lg = q @ K.T * sc
            m = lg.max(1, keepdims=True)
            e = np.exp(lg - m)
            return m, e.sum(1, keepdims=True), (e @ Vv) / e.sum(1, keepdims=True)
        mw, lw, ow = part(x["k_d"][s, 0], x["v_d"][s, 0])
        mg, lg_, og = part(x["k_g"][:, 0], x["v_g"][:, 0])
        m = np.maximum(mw, mg)
        aw, ag = lw * np.exp(mw - m), lg_ * np.exp(mg - m)
        np.testing.assert_allclose(od[s, 0], (aw * ow + ag * og) / (aw + ag), rtol=1e-12, atol=1e-13)


def test_closed_form_special_cases():
    rng = np.random.default_rng(10)
    N, V, G, heads, D = 32, 8, 5, 2, 64
    k = rng.standard_normal((N, heads, D))
    kg = rng.standard_normal((G, heads, D))
    v = rng.standard_normal((N, heads, D))
    vg = rng.standard_normal((G, heads, D))
    # q = 0: uniform weights -> mean of the allowed values
    q0, qg0 = np.zeros((N, heads, D)), np.zeros((G, heads, D))
    od, og = oracle.hier_attn(q0, k, v, qg0, kg, vg, V)
    for c in range(N // V):
        want = (v[c * V:(c + 1) * V].sum(0) + vg.sum(0)) / (V + G)
        np.testing.assert_allclose(od[c * V:(c + 1) * V], np.broadcast_to(want, (V, heads, D)),
                                   rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(og, np.broadcast_to(vg.mean(0), (G, heads, D)), rtol=1e-12, atol=1e-13)
    # constant values -> constant output
    const = np.full((N, heads, D), 0.375)
    od, og = oracle.hier_attn(rng.standard_normal((N, heads, D)), k, const,
                              rng.standard_normal((G, heads, D)), kg, np.full((G, heads, D), 0.375), V)
    np.testing.assert_allclose(od, 0.375, rtol=1e-13)
    np.testing.assert_allclose(og, 0.375, rtol=1e-13)
    # one dominant logit selects that key's value row
    q = np.zeros((N, heads, D))
    kk = np.zeros((N, heads, D))
    kgz = np.zeros((G, heads, D))
    q[:, :, 0] = 1.0
    kk[V + 3, :, 0] = 4000.0          # key 3 of cube 1
    od, _ = oracle.hier_attn(q, kk, v, np.zeros((G, heads, D)), kgz, vg, V)
    np.testing.assert_allclose(od[V:2 * V], np.broadcast_to(v[V + 3], (V, heads, D)), rtol=1e-12)


# ------------------------------------------------------------------ end to end

def raster_pipeline_dense(qd, kd, vd, qg, kg, vg, grid, cube, gproxy, r_t, round_fn):
    """Attention computed directly in raster order with the mask "same cube or
    global", RoPE at raster coordinates: no permutation involved."""
    T, H, W = grid
    ct, ch, cw = cube
    N = T * H * W
    r = np.arange(N)
    t, h, w = r // (H * W), (r // W) % H, r % W
    cube_id = ((t // ct) * (H // ch) + h // ch) * (W // cw) + w // cw
    posd = np.stack([t, h, w], 1).astype(np.float64)
    G = qg.shape[0]
    gr = np.arange(G)
    Tg, Hg, Wg = gproxy
    posg = np.stack([r_t * (gr // (Hg * Wg)), H / Hg * ((gr // Wg) % Hg), W / Wg * (gr % Wg)], 1)
    q = round_fn(complex_rope(oracle.to_f64(qd), posd))
    k = round_fn(complex_rope(oracle.to_f64(kd), posd))
    qgr = round_fn(complex_rope(oracle.to_f64(qg), posg))
    kgr = round_fn(complex_rope(oracle.to_f64(kg), posg))
    v, vgf = oracle.to_f64(vd), oracle.to_f64(vg)
    D = qd.shape[2]
    out = np.empty_like(q)
    for hh in range(qd.shape[1]):
        s_dd = q[:, hh] @ k[:, hh].T / math.sqrt(D)
        s_dd = np.where(cube_id[:, None] == cube_id[None, :], s_dd, -np.inf)
        s_dg = q[:, hh] @ kgr[:, hh].T / math.sqrt(D)
        s = np.concatenate([s_dd, s_dg], 1)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        out[:, hh] = p @ np.concatenate([v[:, hh], vgf[:, hh]])
    return out


@pytest.mark.parametrize("cfg", [
    custom("e1", (4, 8, 8), (2, 4, 4), (2, 4, 4), r_t=4.0, heads=2, head_dim=64, dtype="f32"),
    custom("e2", (3, 6, 8), (3, 2, 4), (1, 3, 2), r_t=8.0, heads=2, head_dim=128, dtype="bf16"),
])
def test_pipeline_rows_equivariance(cfg):
    ins = gen_inputs(cfg)
    od, og = oracle.pipeline_rows(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                  ins["v_g"], cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t)
    if cfg.dtype == "bf16":
        rnd = lambda a: oracle.to_f64(oracle.round_bf16(a))  # noqa: E731
    else:
        rnd = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    want = raster_pipeline_dense(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                 ins["v_g"], cfg.grid, cfg.cube, cfg.gproxy, cfg.r_t, rnd)
    np.testing.assert_allclose(od, want, rtol=1e-9, atol=1e-10)


def test_pipeline_rows_equals_stagewise_composition():
    cfg = custom("e3", (3, 6, 8), (3, 2, 4), (1, 3, 2), r_t=4.0, heads=2, head_dim=64, dtype="bf16")
    ins = gen_inputs(cfg)
    g, cb, gp = cfg.grid, cfg.cube, cfg.gproxy
    qd, kd, vd = (oracle.cube_reorder(ins[n], g, cb) for n in ("q_d", "k_d", "v_d"))
    qd = oracle.round_bf16(oracle.rope_detail(qd, np.arange(cfg.N), g, cb))
    kd = oracle.round_bf16(oracle.rope_detail(kd, np.arange(cfg.N), g, cb))
    qg = oracle.round_bf16(oracle.rope_global(ins["q_g"], np.arange(cfg.G), g, gp, cfg.r_t))
    kg = oracle.round_bf16(oracle.rope_global(ins["k_g"], np.arange(cfg.G), g, gp, cfg.r_t))
    od, og = oracle.hier_attn(qd, kd, vd, qg, kg, ins["v_g"], cfg.V)
    od = oracle.cube_unorder(od, g, cb)
    pd, pg = oracle.pipeline_rows(ins["q_d"], ins["k_d"], ins["v_d"], ins["q_g"], ins["k_g"],
                                  ins["v_g"], g, cb, gp, cfg.r_t)
    np.testing.assert_allclose(pd, od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pg, og, rtol=1e-12, atol=1e-13)
