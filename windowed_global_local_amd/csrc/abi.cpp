// abi.cpp -- the extern "C" entry points of include/atlas.h: argument
// validation on the host (before any HIP call), launch geometry, status codes.
#include "atlas.h"
#include "atlas_internal.hpp"

#include <cmath>
#include <algorithm>
#include <cstdint>

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxTokens = (int64_t)1 << 31;   // per tensor, detail or global
constexpr int32_t kMaxHeads = 4096;

bool all_pos(atlas_dim3 d) { return d.t > 0 && d.h > 0 && d.w > 0; }
bool all_zero(atlas_dim3 d) { return d.t == 0 && d.h == 0 && d.w == 0; }

// product of three positive dims, or -1 on overflow of kMaxTokens
int64_t volume(atlas_dim3 d)
{
    const int64_t v = (int64_t)d.t * d.h;
    if (v >= kMaxTokens)
        return -1;
    const int64_t w = v * d.w;
    return w >= kMaxTokens ? -1 : w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (!a || !b || na <= 0 || nb <= 0)
        return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int elem_size(int32_t dtype) { return dtype == ATLAS_BF16 ? 2 : 4; }

// heads, head_dim, dtype; cube must divide grid
int check_common(atlas_dim3 grid, atlas_dim3 cube, int32_t heads, int32_t head_dim,
                 int32_t dtype, int64_t *N, int64_t *V)
{
    if (dtype != ATLAS_BF16 && dtype != ATLAS_F32)
        return ATLAS_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128)
        return ATLAS_ERR_UNSUPPORTED;
    if (heads <= 0 || heads > kMaxHeads)
        return ATLAS_ERR_SHAPE;
    if (!all_pos(grid) || !all_pos(cube))
        return ATLAS_ERR_SHAPE;
    if (grid.t % cube.t || grid.h % cube.h || grid.w % cube.w)
        return ATLAS_ERR_SHAPE;
    *N = volume(grid);
    *V = volume(cube);
    if (*N < 0 || *V < 0)
        return ATLAS_ERR_SHAPE;
    return ATLAS_OK;
}

// proxy grid: all zero (G = 0) or all positive
int check_proxy(atlas_dim3 gproxy, int64_t *G)
{
    if (all_zero(gproxy)) {
        *G = 0;
        return ATLAS_OK;
    }
    if (!all_pos(gproxy))
        return ATLAS_ERR_SHAPE;
    *G = volume(gproxy);
    return *G < 0 ? ATLAS_ERR_SHAPE : ATLAS_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return ATLAS_OK;
    g_last_hip_error = (int)e;
    return ATLAS_ERR_HIP;
}

int cube_copy(void *dst, const void *src, atlas_dim3 grid, atlas_dim3 cube, int32_t heads,
              int32_t head_dim, int32_t dtype, void *stream, int inverse)
{
    if (!dst || !src)
        return ATLAS_ERR_NULL;
    int64_t N, V;
    const int rc = check_common(grid, cube, heads, head_dim, dtype, &N, &V);
    if (rc != ATLAS_OK)
        return rc;
    if (!aligned16(dst) || !aligned16(src))
        return ATLAS_ERR_ALIGN;
    const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
    const int64_t bytes = N * row_bytes;
    if (overlap(dst, bytes, src, bytes))
        return ATLAS_ERR_ALIAS;
    atlas::CopyRunsArgs a{};
    a.src = static_cast<const char *>(src);
    a.dst = static_cast<char *>(dst);
    a.row_bytes = row_bytes;
    a.H = grid.h;
    a.W = grid.w;
    a.ct = cube.t;
    a.ch = cube.h;
    a.cw = cube.w;
    a.nH = grid.h / cube.h;
    a.nW = grid.w / cube.w;
    const int64_t run_chunks = (int64_t)cube.w * row_bytes / 16;
    if (run_chunks >= ((int64_t)1 << 32))
        return ATLAS_ERR_SHAPE;
    a.run_chunks = (uint32_t)run_chunks;
    a.inverse = inverse;
    return hip_status(atlas::launch_copy_runs(a, N / cube.w, static_cast<hipStream_t>(stream)));
}

}  // namespace

namespace atlas {
void note_hip_error(int e) { g_last_hip_error = e; }
}  // namespace atlas

extern "C" {

int atlas_cube_reorder(void *dst, const void *src, atlas_dim3 grid, atlas_dim3 cube,
                       int32_t heads, int32_t head_dim, int32_t dtype, void *stream)
{
    return cube_copy(dst, src, grid, cube, heads, head_dim, dtype, stream, 0);
}

int atlas_cube_unorder(void *dst, const void *src, atlas_dim3 grid, atlas_dim3 cube,
                       int32_t heads, int32_t head_dim, int32_t dtype, void *stream)
{
    return cube_copy(dst, src, grid, cube, heads, head_dim, dtype, stream, 1);
}

namespace {

// x_detail in cube order, rotated in place, or -- when src_raster is given --
// written from the raster-order rows of src_raster (the fused reorder)
int rope_impl(void *x_detail, const void *src_raster, void *x_global, atlas_dim3 grid,
              atlas_dim3 cube, atlas_dim3 gproxy, float r_t, float theta, int32_t heads,
              int32_t head_dim, int32_t dtype, void *stream)
{
    if (!x_detail && !x_global)
        return ATLAS_ERR_NULL;
    int64_t N, V, G;
    int rc = check_common(grid, cube, heads, head_dim, dtype, &N, &V);
    if (rc != ATLAS_OK)
        return rc;
    rc = check_proxy(gproxy, &G);
    if (rc != ATLAS_OK)
        return rc;
    if (x_global && G == 0)
        return ATLAS_ERR_SHAPE;
    if (!std::isfinite(r_t) || !(r_t > 0.0f) || !std::isfinite(theta) || !(theta > 1.0f))
        return ATLAS_ERR_VALUE;
    if ((x_detail && !aligned16(x_detail)) || (x_global && !aligned16(x_global)))
        return ATLAS_ERR_ALIGN;
    if (src_raster && !aligned16(src_raster))
        return ATLAS_ERR_ALIGN;
    const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
    if (x_detail && x_global && overlap(x_detail, N * row_bytes, x_global, G * row_bytes))
        return ATLAS_ERR_ALIAS;
    if (src_raster && (overlap(src_raster, N * row_bytes, x_detail, N * row_bytes) ||
                       (x_global && overlap(src_raster, N * row_bytes, x_global, G * row_bytes))))
        return ATLAS_ERR_ALIAS;

    atlas::RopeArgs a{};
    a.xd = x_detail;
    a.src_d = src_raster;
    a.xg = x_global;
    a.N = x_detail ? N : 0;
    a.G = x_global ? G : 0;
    a.heads = heads;
    a.T = grid.t;
    a.H = grid.h;
    a.W = grid.w;
    a.ct = cube.t;
    a.ch = cube.h;
    a.cw = cube.w;
    a.nH = grid.h / cube.h;
    a.nW = grid.w / cube.w;
    a.Hg = x_global ? gproxy.h : 1;
    a.Wg = x_global ? gproxy.w : 1;
    a.r_t = (double)r_t;
    a.sh = x_global ? (double)grid.h / (double)gproxy.h : 1.0;
    a.sw = x_global ? (double)grid.w / (double)gproxy.w : 1.0;
    const int n_hw = head_dim / 6;
    const int n_t = head_dim / 2 - 2 * n_hw;
    a.n_t = n_t;
    a.n_h = n_hw;
    for (int i = 0; i < head_dim / 2; ++i) {
        int j, n;
        if (i < n_t) {
            j = i;
            n = n_t;
        } else if (i < n_t + n_hw) {
            j = i - n_t;
            n = n_hw;
        } else {
            j = i - n_t - n_hw;
            n = n_hw;
        }
        a.omega[i] = std::pow((double)theta, -(double)j / (double)n);
    }
    const int tok = atlas::rope_tokens_per_block(head_dim);
    const int64_t blocks_d = (a.N + tok - 1) / tok;
    const int64_t blocks_g = (a.G + tok - 1) / tok;
    if (blocks_d > 0x7fffffffLL)
        return ATLAS_ERR_SHAPE;
    a.blocks_d = (int32_t)blocks_d;
    a.row_chunks = (uint32_t)(row_bytes / 16);
    a.fd_mul = (((uint64_t)1 << 40) + a.row_chunks - 1) / a.row_chunks;
    return hip_status(atlas::launch_rope(a, head_dim, dtype == ATLAS_F32, blocks_g,
                                         static_cast<hipStream_t>(stream)));
}

}  // namespace

int atlas_rope3d(void *x_detail, void *x_global, atlas_dim3 grid, atlas_dim3 cube,
                 atlas_dim3 gproxy, float r_t, float theta, int32_t heads, int32_t head_dim,
                 int32_t dtype, void *stream)
{
    return rope_impl(x_detail, nullptr, x_global, grid, cube, gproxy, r_t, theta, heads, head_dim,
                     dtype, stream);
}

int atlas_cube_reorder_rope3d(void *x_detail, const void *x_raster, void *x_global, atlas_dim3 grid,
                              atlas_dim3 cube, atlas_dim3 gproxy, float r_t, float theta,
                              int32_t heads, int32_t head_dim, int32_t dtype, void *stream)
{
    if ((x_detail == nullptr) != (x_raster == nullptr))
        return ATLAS_ERR_NULL;
    return rope_impl(x_detail, x_raster, x_global, grid, cube, gproxy, r_t, theta, heads, head_dim,
                     dtype, stream);
}

namespace {

int hier_attn_impl(void *o_detail, void *o_global, const void *q_d, const void *k_d,
                   const void *v_d, const void *q_g, const void *k_g, const void *v_g,
                   atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                   int32_t head_dim, float softmax_scale, int32_t dtype, int raster, void *stream,
                   float *lse_d = nullptr, float *lse_g = nullptr, bool want_lse = false,
                   const int32_t *goff = nullptr, const int32_t *gidx = nullptr, int64_t n_gidx = 0)
{
    if (!o_detail || !q_d || !k_d || !v_d)
        return ATLAS_ERR_NULL;
    int64_t N, V, G;
    int rc = check_common(grid, cube, heads, head_dim, dtype, &N, &V);
    if (rc != ATLAS_OK)
        return rc;
    rc = check_proxy(gproxy, &G);
    if (rc != ATLAS_OK)
        return rc;
    if (G > 0 && (!o_global || !q_g || !k_g || !v_g))
        return ATLAS_ERR_NULL;
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
        return ATLAS_ERR_VALUE;
    const void *ptrs[] = {o_detail, q_d, k_d, v_d, o_global, q_g, k_g, v_g};
    for (int i = 0; i < 8; ++i) {
        if (i >= 4 && G == 0)
            break;
        if (!aligned16(ptrs[i]))
            return ATLAS_ERR_ALIGN;
    }
    const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
    const int64_t bd = N * row_bytes, bg = G * row_bytes;
    const void *ins[] = {q_d, k_d, v_d, q_g, k_g, v_g};
    const int64_t ins_b[] = {bd, bd, bd, bg, bg, bg};
    for (int i = 0; i < 6; ++i) {
        if (overlap(o_detail, bd, ins[i], ins_b[i]))
            return ATLAS_ERR_ALIAS;
        if (G > 0 && overlap(o_global, bg, ins[i], ins_b[i]))
            return ATLAS_ERR_ALIAS;
    }
    if (G > 0 && overlap(o_detail, bd, o_global, bg))
        return ATLAS_ERR_ALIAS;
    if (want_lse) {
        if (!lse_d || (G > 0 && !lse_g))
            return ATLAS_ERR_NULL;
        if (!aligned16(lse_d) || (G > 0 && !aligned16(lse_g)))
            return ATLAS_ERR_ALIGN;
        const int64_t ld = (int64_t)heads * N * 4, lg = (int64_t)heads * G * 4;
        const void *all[] = {o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g};
        const int64_t all_b[] = {bd, bg, bd, bd, bd, bg, bg, bg};
        for (int i = 0; i < 8; ++i) {
            if (overlap(lse_d, ld, all[i], all_b[i]) || (G > 0 && overlap(lse_g, lg, all[i], all_b[i])))
                return ATLAS_ERR_ALIAS;
        }
        if (G > 0 && overlap(lse_d, ld, lse_g, lg))
            return ATLAS_ERR_ALIAS;
    }

    const double scale = softmax_scale > 0.0f ? (double)softmax_scale
                                              : 1.0 / std::sqrt((double)head_dim);
    const int bq = atlas::hier_attn_block_rows();
    atlas::AttnArgs a{};
    a.qd = q_d;
    a.kd = k_d;
    a.vd = v_d;
    a.qg = G ? q_g : nullptr;
    a.kg = G ? k_g : nullptr;
    a.vg = G ? v_g : nullptr;
    a.od = o_detail;
    a.og = G ? o_global : nullptr;
    a.lse_d = want_lse ? lse_d : nullptr;
    a.lse_g = (want_lse && G) ? lse_g : nullptr;
    a.goff = G ? goff : nullptr;
    a.gidx = G ? gidx : nullptr;
    a.n_gidx = (int32_t)n_gidx;
    a.V = V;
    a.G = G;
    a.C = N / V;
    a.heads = heads;
    a.qb_win = (int32_t)((V + bq - 1) / bq);
    a.qb_glob = (int32_t)((G + bq - 1) / bq);
    a.items_per_head = a.C * a.qb_win + a.qb_glob;
    a.items = (int64_t)heads * a.items_per_head;
    if (a.items > 0x7fffffffLL)
        return ATLAS_ERR_SHAPE;
    a.c_log2 = (float)(scale * 1.4426950408889634);
    a.raster = raster;
    a.ct = cube.t;
    a.ch = cube.h;
    a.cw = cube.w;
    a.nH = grid.h / cube.h;
    a.nW = grid.w / cube.w;
    a.H = grid.h;
    a.W = grid.w;
    return hip_status(atlas::launch_hier_attn(a, head_dim, dtype == ATLAS_F32,
                                              static_cast<hipStream_t>(stream)));
}

}  // namespace

int atlas_hier_attn(void *o_detail, void *o_global, const void *q_d, const void *k_d,
                    const void *v_d, const void *q_g, const void *k_g, const void *v_g,
                    atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                    int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    return hier_attn_impl(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                          heads, head_dim, softmax_scale, dtype, 0, stream);
}

int atlas_hier_attn_raster(void *o_detail, void *o_global, const void *q_d, const void *k_d,
                           const void *v_d, const void *q_g, const void *k_g, const void *v_g,
                           atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                           int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    return hier_attn_impl(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                          heads, head_dim, softmax_scale, dtype, 1, stream);
}

namespace {
// validation of a per-window subset (lists, their alignment and overlaps)
int check_subset(const void *o_detail, const void *o_global, const int32_t *win_goff,
                 const int32_t *win_gidx, int64_t n_gidx, atlas_dim3 grid, atlas_dim3 cube,
                 atlas_dim3 gproxy, int32_t heads, int32_t head_dim, int32_t dtype)
{
    int64_t G;
    if (check_proxy(gproxy, &G) != ATLAS_OK)
        return ATLAS_ERR_SHAPE;
    if (G > 0) {
        if (!win_goff || (!win_gidx && n_gidx > 0))
            return ATLAS_ERR_NULL;
        if (n_gidx < 0 || n_gidx > 0x7fffffffLL)
            return ATLAS_ERR_VALUE;
        if (((uintptr_t)win_goff & 3u) || ((uintptr_t)win_gidx & 3u))
            return ATLAS_ERR_ALIGN;
        // gathered rows are addressed by 32-bit offsets into one head's global rows
        const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
        if (G * row_bytes >= ((int64_t)1 << 31))
            return ATLAS_ERR_SHAPE;
    }
    // a list array may not overlap an output
    int64_t N, V;
    int rc = check_common(grid, cube, heads, head_dim, dtype, &N, &V);
    if (rc != ATLAS_OK)
        return rc;
    if (G > 0) {
        const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
        const int64_t C = N / V;
        if (overlap(win_goff, 4 * (C + 1), o_detail, N * row_bytes) ||
            overlap(win_goff, 4 * (C + 1), o_global, G * row_bytes) ||
            overlap(win_gidx, 4 * n_gidx, o_detail, N * row_bytes) ||
            overlap(win_gidx, 4 * n_gidx, o_global, G * row_bytes))
            return ATLAS_ERR_ALIAS;
    }
    return ATLAS_OK;
}

// a list with no entries still needs a non-null pointer for the kernel (never read)
const int32_t kNoIndex = 0;
}  // namespace

int atlas_hier_attn_subset(void *o_detail, void *o_global, const void *q_d, const void *k_d,
                           const void *v_d, const void *q_g, const void *k_g, const void *v_g,
                           const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
                           atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                           int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    const int rc = check_subset(o_detail, o_global, win_goff, win_gidx, n_gidx, grid, cube,
                                gproxy, heads, head_dim, dtype);
    if (rc != ATLAS_OK)
        return rc;
    return hier_attn_impl(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                          heads, head_dim, softmax_scale, dtype, 0, stream, nullptr, nullptr, false,
                          win_goff, n_gidx > 0 ? win_gidx : &kNoIndex, n_gidx);
}

int atlas_hier_attn_subset_fwd(void *o_detail, void *o_global, float *lse_detail,
                               float *lse_global, const void *q_d, const void *k_d,
                               const void *v_d, const void *q_g, const void *k_g, const void *v_g,
                               const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
                               atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                               int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    const int rc = check_subset(o_detail, o_global, win_goff, win_gidx, n_gidx, grid, cube,
                                gproxy, heads, head_dim, dtype);
    if (rc != ATLAS_OK)
        return rc;
    return hier_attn_impl(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                          heads, head_dim, softmax_scale, dtype, 0, stream, lse_detail, lse_global,
                          true, win_goff, n_gidx > 0 ? win_gidx : &kNoIndex, n_gidx);
}

int64_t atlas_aligned_subset(int32_t *win_goff, int32_t *win_gidx, int64_t capacity,
                             atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, float r_t)
{
    int64_t N, V, G;
    if (check_common(grid, cube, 1, 64, ATLAS_BF16, &N, &V) != ATLAS_OK)
        return ATLAS_ERR_SHAPE;
    if (check_proxy(gproxy, &G) != ATLAS_OK)
        return ATLAS_ERR_SHAPE;
    if (!(r_t > 0.0f) || std::isinf(r_t))
        return ATLAS_ERR_VALUE;
    const int64_t nT = grid.t / cube.t, nH = grid.h / cube.h, nW = grid.w / cube.w;
    const int64_t C = nT * nH * nW;
    if (C > 0x7ffffffeLL || G > 0x7fffffffLL)
        return ATLAS_ERR_SHAPE;
    // cube (a, b, e) takes, per axis, the proxy indices whose mapped
    // coordinate lies in the box: hg with b*ch <= H*hg/Hg < (b+1)*ch, i.e.
    // ceil(b*ch*Hg/H) <= hg < ceil((b+1)*ch*Hg/H) (exact in integers); likewise
    // wg; tg by comparing r_t*tg in fp64.  Looping tg, hg, wg in increasing
    // order lists each cube's tokens in increasing raster order.
    auto cdiv = [](int64_t x, int64_t y) { return (x + y - 1) / y; };
    int64_t total = 0;
    for (int64_t c = 0; c < C; ++c) {
        const int64_t ca = c / (nH * nW), cb = (c / nW) % nH, ce = c % nW;
        const int64_t h0 = cdiv(cb * cube.h * gproxy.h, grid.h);
        const int64_t h1 = std::min<int64_t>(gproxy.h, cdiv((cb + 1) * cube.h * gproxy.h, grid.h));
        const int64_t w0 = cdiv(ce * cube.w * gproxy.w, grid.w);
        const int64_t w1 = std::min<int64_t>(gproxy.w, cdiv((ce + 1) * cube.w * gproxy.w, grid.w));
        if (win_goff)
            win_goff[c] = (int32_t)total;
        for (int64_t tg = 0; tg < gproxy.t; ++tg) {
            const double pt = (double)r_t * (double)tg;
            if (!(pt >= (double)(ca * cube.t) && pt < (double)((ca + 1) * cube.t)))
                continue;
            for (int64_t hg = h0; hg < h1; ++hg)
                for (int64_t wg = w0; wg < w1; ++wg) {
                    if (win_gidx) {
                        if (total >= capacity)
                            return ATLAS_ERR_VALUE;
                        win_gidx[total] = (int32_t)((tg * gproxy.h + hg) * gproxy.w + wg);
                    }
                    ++total;
                }
        }
    }
    if (win_goff)
        win_goff[C] = (int32_t)total;
    return total;
}

int atlas_hier_attn_fwd(void *o_detail, void *o_global, float *lse_detail, float *lse_global,
                        const void *q_d, const void *k_d, const void *v_d, const void *q_g,
                        const void *k_g, const void *v_g, atlas_dim3 grid, atlas_dim3 cube,
                        atlas_dim3 gproxy, int32_t heads, int32_t head_dim, float softmax_scale,
                        int32_t dtype, void *stream)
{
    return hier_attn_impl(o_detail, o_global, q_d, k_d, v_d, q_g, k_g, v_g, grid, cube, gproxy,
                          heads, head_dim, softmax_scale, dtype, 0, stream, lse_detail, lse_global,
                          true);
}

int64_t atlas_hier_attn_bwd_workspace_bytes(atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                                            int32_t heads, int32_t head_dim)
{
    int64_t N, V, G;
    if (check_common(grid, cube, heads, head_dim, ATLAS_BF16, &N, &V) != ATLAS_OK)
        return -1;
    if (check_proxy(gproxy, &G) != ATLAS_OK)
        return -1;
    return 4 * (int64_t)heads * (N + G);
}

namespace {
// bytes of the D rows, rounded up so that the subset accumulators that follow
// them stay 256-byte aligned
int64_t bwd_delta_bytes(int64_t N, int64_t G, int32_t heads)
{
    return (4 * (int64_t)heads * (N + G) + 255) / 256 * 256;
}

int bwd_impl(void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g, void *dv_g,
             const void *q_d, const void *k_d, const void *v_d, const void *q_g,
             const void *k_g, const void *v_g, const void *o_d, const void *o_g,
             const void *do_d, const void *do_g, const float *lse_detail,
             const float *lse_global, void *workspace, int64_t workspace_bytes,
             atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
             int32_t head_dim, float softmax_scale, int32_t dtype, void *stream,
             const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
             atlas::ScratchFn get_scratch = nullptr);
}  // namespace

int atlas_hier_attn_bwd(void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g, void *dv_g,
                        const void *q_d, const void *k_d, const void *v_d, const void *q_g,
                        const void *k_g, const void *v_g, const void *o_d, const void *o_g,
                        const void *do_d, const void *do_g, const float *lse_detail,
                        const float *lse_global, void *workspace, int64_t workspace_bytes,
                        atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                        int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    return bwd_impl(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g, v_g, o_d, o_g,
                    do_d, do_g, lse_detail, lse_global, workspace, workspace_bytes, grid, cube,
                    gproxy, heads, head_dim, softmax_scale, dtype, stream, nullptr, nullptr, 0);
}

int64_t atlas_hier_attn_subset_bwd_workspace_bytes(atlas_dim3 grid, atlas_dim3 cube,
                                                   atlas_dim3 gproxy, int32_t heads,
                                                   int32_t head_dim)
{
    int64_t N, V, G;
    if (check_common(grid, cube, heads, head_dim, ATLAS_BF16, &N, &V) != ATLAS_OK)
        return -1;
    if (check_proxy(gproxy, &G) != ATLAS_OK)
        return -1;
    return bwd_delta_bytes(N, G, heads) + 2 * 4 * G * (int64_t)heads * head_dim;
}

int atlas_hier_attn_subset_bwd(void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g,
                               void *dv_g, const void *q_d, const void *k_d, const void *v_d,
                               const void *q_g, const void *k_g, const void *v_g, const void *o_d,
                               const void *o_g, const void *do_d, const void *do_g,
                               const float *lse_detail, const float *lse_global,
                               const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
                               void *workspace, int64_t workspace_bytes, atlas_dim3 grid,
                               atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                               int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    int rc = check_subset(dq_d, dq_g, win_goff, win_gidx, n_gidx, grid, cube, gproxy, heads,
                          head_dim, dtype);
    if (rc != ATLAS_OK)
        return rc;
    int64_t G;
    check_proxy(gproxy, &G);
    if (G > 0) {
        // the lists may not overlap any gradient either
        int64_t N, V;
        check_common(grid, cube, heads, head_dim, dtype, &N, &V);
        const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
        const int64_t C = N / V;
        const void *outs[] = {dk_d, dv_d, dk_g, dv_g};
        const int64_t sz[] = {N * row_bytes, N * row_bytes, G * row_bytes, G * row_bytes};
        for (int i = 0; i < 4; ++i)
            if (overlap(win_goff, 4 * (C + 1), outs[i], sz[i]) ||
                overlap(win_gidx, 4 * n_gidx, outs[i], sz[i]))
                return ATLAS_ERR_ALIAS;
    }
    return bwd_impl(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g, v_g, o_d, o_g,
                    do_d, do_g, lse_detail, lse_global, workspace, workspace_bytes, grid, cube,
                    gproxy, heads, head_dim, softmax_scale, dtype, stream,
                    G > 0 ? win_goff : nullptr, n_gidx > 0 ? win_gidx : &kNoIndex, n_gidx);
}

namespace {
int bwd_impl(void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g, void *dv_g,
             const void *q_d, const void *k_d, const void *v_d, const void *q_g,
             const void *k_g, const void *v_g, const void *o_d, const void *o_g,
             const void *do_d, const void *do_g, const float *lse_detail,
             const float *lse_global, void *workspace, int64_t workspace_bytes,
             atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
             int32_t head_dim, float softmax_scale, int32_t dtype, void *stream,
             const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
             atlas::ScratchFn get_scratch)
{
    // get_scratch != null: the workspace is the library's fixed device array of
    // workspace_bytes bytes, looked up only once every other check has passed
    if (!dq_d || !dk_d || !dv_d || !q_d || !k_d || !v_d || !o_d || !do_d || !lse_detail ||
        (!workspace && !get_scratch))
        return ATLAS_ERR_NULL;
    int64_t N, V, G;
    int rc = check_common(grid, cube, heads, head_dim, dtype, &N, &V);
    if (rc != ATLAS_OK)
        return rc;
    rc = check_proxy(gproxy, &G);
    if (rc != ATLAS_OK)
        return rc;
    if (G > 0 && (!dq_g || !dk_g || !dv_g || !q_g || !k_g || !v_g || !o_g || !do_g || !lse_global))
        return ATLAS_ERR_NULL;
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
        return ATLAS_ERR_VALUE;
    const bool subset = win_goff != nullptr;
    const int64_t ws_need = subset ? bwd_delta_bytes(N, G, heads) + 2 * 4 * G * (int64_t)heads * head_dim
                                   : 4 * (int64_t)heads * (N + G);
    if (workspace_bytes < ws_need)
        return get_scratch ? ATLAS_ERR_SCRATCH : ATLAS_ERR_VALUE;
    const int64_t row_bytes = (int64_t)heads * head_dim * elem_size(dtype);
    const int64_t bd = N * row_bytes, bg = G * row_bytes;
    const int64_t ld = (int64_t)heads * N * 4, lg = (int64_t)heads * G * 4;
    // every buffer with its size; the first six are outputs, the seventh the
    // workspace (left out until the fixed array's address is known)
    const void *buf[] = {dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, workspace,
                         q_d, k_d, v_d, o_d, do_d, lse_detail,
                         q_g, k_g, v_g, o_g, do_g, lse_global};
    int64_t nb[] = {bd, bd, bd, bg, bg, bg, get_scratch ? 0 : ws_need,
                    bd, bd, bd, bd, bd, ld,
                    bg, bg, bg, bg, bg, lg};
    constexpr int kBufs = 19, kOuts = 7, kWs = 6;   // outputs and the workspace are written
    auto check_buffers = [&]() {
        for (int i = 0; i < kBufs; ++i) {
            if (nb[i] > 0 && !aligned16(buf[i]))
                return ATLAS_ERR_ALIGN;
        }
        for (int i = 0; i < kOuts; ++i)
            for (int j = 0; j < kBufs; ++j)
                if (j != i && overlap(buf[i], nb[i], buf[j], nb[j]))
                    return ATLAS_ERR_ALIAS;
        return ATLAS_OK;
    };
    rc = check_buffers();
    if (rc != ATLAS_OK)
        return rc;
    if (get_scratch) {
        rc = get_scratch(&workspace);
        if (rc != ATLAS_OK)
            return rc;
        buf[kWs] = workspace;
        nb[kWs] = ws_need;
        rc = check_buffers();
        if (rc != ATLAS_OK)
            return rc;
    }

    const double scale = softmax_scale > 0.0f ? (double)softmax_scale
                                              : 1.0 / std::sqrt((double)head_dim);
    const int br = atlas::hier_attn_bwd_block_rows();
    atlas::BwdArgs a{};
    a.qd = q_d;
    a.kd = k_d;
    a.vd = v_d;
    a.dod = do_d;
    a.qg = G ? q_g : nullptr;
    a.kg = G ? k_g : nullptr;
    a.vg = G ? v_g : nullptr;
    a.dog = G ? do_g : nullptr;
    a.dqd = dq_d;
    a.dkd = dk_d;
    a.dvd = dv_d;
    a.dqg = G ? dq_g : nullptr;
    a.dkg = G ? dk_g : nullptr;
    a.dvg = G ? dv_g : nullptr;
    a.lse_d = lse_detail;
    a.lse_g = G ? lse_global : nullptr;
    float *ws = static_cast<float *>(workspace);
    a.dl_d = ws;
    a.dl_g = G ? ws + (int64_t)heads * N : nullptr;
    if (subset) {
        float *acc = reinterpret_cast<float *>(static_cast<char *>(workspace) + bwd_delta_bytes(N, G, heads));
        a.goff = win_goff;
        a.gidx = win_gidx;
        a.n_gidx = (int32_t)n_gidx;
        a.acc_k = acc;                                       // acc_v follows contiguously
        a.acc_v = acc + G * (int64_t)heads * head_dim;
    }
    a.N = N;
    a.V = V;
    a.G = G;
    a.C = N / V;
    a.heads = heads;
    const int bq = atlas::hier_attn_bwd_dq_rows();
    a.qb_win = (int32_t)((V + bq - 1) / bq);
    a.qb_glob = (int32_t)((G + bq - 1) / bq);
    a.kb_win = (int32_t)((V + br - 1) / br);
    a.kb_glob = (int32_t)((G + br - 1) / br);
    a.dq_items_per_head = a.C * a.qb_win + a.qb_glob;
    a.dq_items = (int64_t)heads * a.dq_items_per_head;
    a.kv_items_glob = (int64_t)heads * a.kb_glob;
    a.kv_items = a.kv_items_glob + (int64_t)heads * a.C * a.kb_win;
    if (a.dq_items > 0x7fffffffLL || a.kv_items > 0x7fffffffLL)
        return ATLAS_ERR_SHAPE;
    a.c_log2 = (float)(scale * 1.4426950408889634);
    a.scale = (float)scale;
    return hip_status(atlas::launch_hier_attn_bwd(a, o_d, G ? o_g : nullptr, head_dim,
                                                  dtype == ATLAS_F32,
                                                  static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C++" {
namespace atlas {
int hier_attn_bwd_scratch(void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g, void *dv_g,
                          const void *q_d, const void *k_d, const void *v_d, const void *q_g,
                          const void *k_g, const void *v_g, const void *o_d, const void *o_g,
                          const void *do_d, const void *do_g, const float *lse_detail,
                          const float *lse_global, ScratchFn get_scratch, int64_t scratch_bytes,
                          atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                          int32_t head_dim, float softmax_scale, int32_t dtype, void *stream)
{
    return bwd_impl(dq_d, dk_d, dv_d, dq_g, dk_g, dv_g, q_d, k_d, v_d, q_g, k_g, v_g, o_d, o_g,
                    do_d, do_g, lse_detail, lse_global, nullptr, scratch_bytes, grid, cube,
                    gproxy, heads, head_dim, softmax_scale, dtype, stream, nullptr, nullptr, 0,
                    get_scratch);
}
}  // namespace atlas
}  // extern "C++"

double atlas_hier_attn_useful_flops(atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                                    int32_t heads, int32_t head_dim)
{
    int64_t N, V, G;
    if (heads <= 0 || head_dim <= 0 || !all_pos(grid) || !all_pos(cube))
        return -1.0;
    if (grid.t % cube.t || grid.h % cube.h || grid.w % cube.w)
        return -1.0;
    N = volume(grid);
    V = volume(cube);
    if (N < 0 || V < 0 || check_proxy(gproxy, &G) != ATLAS_OK)
        return -1.0;
    const double pairs = (double)N * (double)(V + G) + (double)G * (double)G;
    return 4.0 * (double)head_dim * (double)heads * pairs;
}

const char *atlas_status_string(int status)
{
    switch (status) {
    case ATLAS_OK: return "ok";
    case ATLAS_ERR_NULL: return "a required pointer is NULL";
    case ATLAS_ERR_SHAPE: return "bad shape: non-positive dim, cube does not divide grid, "
                                 "partly-zero proxy grid, or a size overflows";
    case ATLAS_ERR_DTYPE: return "unsupported dtype (expected ATLAS_BF16 or ATLAS_F32)";
    case ATLAS_ERR_UNSUPPORTED: return "unsupported head_dim (expected 64 or 128)";
    case ATLAS_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATLAS_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATLAS_ERR_HIP: return "HIP launch failed (see atlas_last_hip_error)";
    case ATLAS_ERR_VALUE: return "a scalar argument is not finite or out of range";
    case ATLAS_ERR_SCRATCH: return "the call needs more scratch memory than the library's "
                                   "fixed device array holds";
    default: return "unknown status";
    }
}

int atlas_last_hip_error(void) { return g_last_hip_error; }

int atlas_version(void) { return 10200; }

}  // extern "C"
