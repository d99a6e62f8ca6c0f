// rope3d.hip -- in-place 3D rotary embedding with temporal scale r_t and proxy
// alignment, on gfx950.
//
// "Technische Samenvatting: AtlasVid", Methodologie 1, Fase 1: the proxy's
// temporal RoPE indices are multiplied by r_t.  Methodologie 2,
// Positie-uitlijning: proxy RoPE coordinates are scaled by the resolution
// ratios onto the detail grid.  Detail tokens (cube order) sit at the integer
// (t, h, w) of their raster token; proxy token (tg, hg, wg) sits at
// (r_t * tg, (H/Hg) * hg, (W/Wg) * wg).  head_dim/2 pairs (2i, 2i+1): the
// first n_t turn with t, the next n_h with h, the rest with w.
//
// Angles depend on the token, not the head, so a workgroup first builds the
// cos/sin table of its token in LDS (one sin/cos per pair), then streams its
// share of the token row (all heads) through 16-byte loads and stores.
// HBM bound: 2 * tokens * row_bytes per call.
#include "atlas_internal.hpp"

namespace atlas {

namespace {

// Launch shape: the fastest of a sweep on MI355X at the 4K workload (fused
// reorder + RoPE): a token row is split over kSeg = 5 workgroups of 64
// threads (2 KiB each for head_dim 128: two 16-byte chunks per thread, all in
// flight at once), each building the token's table; non-temporal loads and
// stores (the rows are touched exactly once) -- 6.2 TB/s, against 5.6 TB/s
// with one workgroup per token.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64;
constexpr int kBatch = 2;      // 16-byte chunks in flight per thread
constexpr int kSeg = 5;        // workgroups per token block
constexpr int kTokMul = 1;     // table passes per workgroup (tokens = kTokMul * kThreads / pairs)

template <int D>
struct RopeShape {
    static constexpr int kPairs = D / 2;
    static constexpr int kTabRows = kThreads / kPairs;             // table rows per pass
    static constexpr int kTok = kTabRows * kTokMul;                // tokens per workgroup
};

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline uint32_t pack_bf16(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

// cube-order token -> raster (t, h, w) (the cube enumeration of the layout passes)
__device__ inline void cube_to_thw(const RopeArgs &a, int64_t tok, int32_t &t, int32_t &h, int32_t &w)
{
    const int64_t V = (int64_t)a.ct * a.ch * a.cw;
    const int64_t c = tok / V;
    const int32_t o = (int32_t)(tok - c * V);
    const int32_t cubes_per_frame = a.nH * a.nW;
    const int32_t ca = (int32_t)(c / cubes_per_frame);
    const int32_t crem = (int32_t)(c - (int64_t)ca * cubes_per_frame);
    const int32_t cb = crem / a.nW, ce = crem - cb * a.nW;
    const int32_t dt = o / (a.ch * a.cw);
    const int32_t orem = o - dt * (a.ch * a.cw);
    const int32_t dh = orem / a.cw, dw = orem - dh * a.cw;
    t = ca * a.ct + dt;
    h = cb * a.ch + dh;
    w = ce * a.cw + dw;
}

// REORDER: the detail rows are read from their raster position in src_d and
// written in cube order to xd (the cube reorder fused into the rotation: one
// pass over HBM instead of two); proxy rows are rotated in place either way.
template <int D, bool F32, bool REORDER>
__global__ __launch_bounds__(kThreads) void rope_kernel(const RopeArgs a)
{
    using S = RopeShape<D>;
    __shared__ __attribute__((aligned(16))) float2 cs[S::kTok][S::kPairs];

    // workgroup -> (token block, segment of its chunks)
    const int seg = (int)(blockIdx.x % kSeg);
    const int64_t bidx = blockIdx.x / kSeg;
    const bool detail = bidx < a.blocks_d;
    const int64_t blk = detail ? bidx : bidx - a.blocks_d;
    const int64_t tok0 = blk * S::kTok;
    const int64_t ntok_all = detail ? a.N : a.G;
    const int ntok = (int)min<int64_t>(S::kTok, ntok_all - tok0);
    char *base = reinterpret_cast<char *>(detail ? a.xd : a.xg);

    // ---- rows: chunk idx -> (token, chunk within row)
    constexpr int kElemsPerChunk = F32 ? 4 : 8;
    constexpr int kChunksPerHead = D / kElemsPerChunk;
    const uint32_t seg_len = ((uint32_t)S::kTok * a.row_chunks + kSeg - 1) / kSeg;
    const uint32_t seg0 = (uint32_t)seg * seg_len;
    const uint32_t total = min((uint32_t)ntok * a.row_chunks, seg0 + seg_len);   // end of this segment
    uint4 *rows = reinterpret_cast<uint4 *>(base + tok0 * (int64_t)a.row_chunks * 16);
    // fused reorder: raster row of each of the workgroup's tokens
    int64_t src_row[S::kTok];
    const bool fused = REORDER && detail;
    if constexpr (REORDER) {
#pragma unroll
        for (int tk = 0; tk < S::kTok; ++tk) {
            int32_t t, h, w;
            cube_to_thw(a, tok0 + min(tk, max(ntok - 1, 0)), t, h, w);
            src_row[tk] = ((int64_t)t * a.H + h) * a.W + w;
        }
    }
    auto src_ptr = [&](uint32_t idx) -> const u32x4 * {
        if (REORDER && fused) {
            const uint32_t tk = (uint32_t)(((uint64_t)idx * a.fd_mul) >> 40);
            const uint32_t ci = idx - tk * a.row_chunks;
            int64_t r = src_row[0];
#pragma unroll
            for (int j = 1; j < S::kTok; ++j)
                r = (int)tk == j ? src_row[j] : r;
            return reinterpret_cast<const u32x4 *>(a.src_d) + r * (int64_t)a.row_chunks + ci;
        }
        return reinterpret_cast<const u32x4 *>(rows) + idx;
    };

    auto load_batch = [&](uint32_t b0, uint4 *v) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const uint32_t idx = b0 + u * kThreads;
            if (idx < total) {
                v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(src_ptr(idx)));
            }
        }
    };

    // the first batch of rows is requested before the table is built, so the
    // fp64 sin/cos work overlaps the memory latency
    uint4 v[kBatch];
    load_batch(seg0 + threadIdx.x, v);

    // ---- cos/sin table: thread -> (token tk, pair i)
#pragma unroll
    for (int pass = 0; pass < kTokMul; ++pass) {
        const int tk = threadIdx.x / S::kPairs + pass * S::kTabRows;
        const int i = threadIdx.x % S::kPairs;
        if (tk < ntok) {
            const int64_t tok = tok0 + tk;
            double pt, ph, pw;
            if (detail) {
                // cube-order position -> raster (t, h, w)
                int32_t t, h, w;
                cube_to_thw(a, tok, t, h, w);
                pt = (double)t;
                ph = (double)h;
                pw = (double)w;
            } else {
                const int32_t r = (int32_t)tok;
                const int32_t plane = a.Hg * a.Wg;
                const int32_t tg = r / plane;
                const int32_t rem = r - tg * plane;
                const int32_t hg = rem / a.Wg, wg = rem - hg * a.Wg;
                pt = a.r_t * (double)tg;
                ph = a.sh * (double)hg;
                pw = a.sw * (double)wg;
            }
            const double p = i < a.n_t ? pt : (i < a.n_t + a.n_h ? ph : pw);
            // coordinates and angle in fp64 (in fp32 the angle alone would
            // carry an absolute error of up to ~1e-5 rad at coordinates
            // ~240), reduced to [-pi, pi] with 2 pi split in two parts; the
            // reduced angle's fp32 rounding leaves at most ~2e-7 rad
            const double ang = p * a.omega[i];
            const double k = rint(ang * 0.15915494309189535);
            const double r = fma(-k, 6.283185307179586, ang) - k * 2.4492935982947064e-16;
            float sn, cn;
            sincosf((float)r, &sn, &cn);
            cs[tk][i] = make_float2(cn, sn);
        }
    }
    __syncthreads();

    for (uint32_t b0 = seg0 + threadIdx.x; b0 < total; b0 += kThreads * kBatch) {
        if (b0 != seg0 + threadIdx.x)
            load_batch(b0, v);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const uint32_t idx = b0 + u * kThreads;
            if (idx >= total)
                continue;
            const uint32_t tk = (uint32_t)(((uint64_t)idx * a.fd_mul) >> 40);
            const uint32_t ci = idx - tk * a.row_chunks;
            const int pair0 = (int)(ci % kChunksPerHead) * (kElemsPerChunk / 2);
            uint4 r;
            if constexpr (F32) {
                const float4 c01 = *reinterpret_cast<const float4 *>(&cs[tk][pair0]);
                float x0 = __uint_as_float(v[u].x), x1 = __uint_as_float(v[u].y);
                float x2 = __uint_as_float(v[u].z), x3 = __uint_as_float(v[u].w);
                r.x = __float_as_uint(fmaf(x0, c01.x, -x1 * c01.y));
                r.y = __float_as_uint(fmaf(x0, c01.y, x1 * c01.x));
                r.z = __float_as_uint(fmaf(x2, c01.z, -x3 * c01.w));
                r.w = __float_as_uint(fmaf(x2, c01.w, x3 * c01.z));
            } else {
                const float4 c01 = *reinterpret_cast<const float4 *>(&cs[tk][pair0]);
                const float4 c23 = *reinterpret_cast<const float4 *>(&cs[tk][pair0 + 2]);
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
                const float ss[4] = {c01.y, c01.w, c23.y, c23.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x0 = bf16_lo(w[j]), x1 = bf16_hi(w[j]);
                    o[j] = pack_bf16(fmaf(x0, cc[j], -x1 * ss[j]), fmaf(x0, ss[j], x1 * cc[j]));
                }
                r = make_uint4(o[0], o[1], o[2], o[3]);
            }
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, r), reinterpret_cast<u32x4 *>(rows) + idx);
        }
    }
}

template <int D, bool F32>
hipError_t launch_t(const RopeArgs &a, int64_t blocks_g, hipStream_t s)
{
    const int64_t blocks = ((int64_t)a.blocks_d + blocks_g) * kSeg;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (a.src_d != nullptr)
        hipLaunchKernelGGL((rope_kernel<D, F32, true>), dim3((uint32_t)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((rope_kernel<D, F32, false>), dim3((uint32_t)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int rope_tokens_per_block(int head_dim) { return kThreads / (head_dim / 2) * kTokMul; }

hipError_t launch_rope(const RopeArgs &a, int head_dim, int is_f32, int64_t blocks_g,
                       hipStream_t s)
{
    if (head_dim == 128)
        return is_f32 ? launch_t<128, true>(a, blocks_g, s) : launch_t<128, false>(a, blocks_g, s);
    if (head_dim == 64)
        return is_f32 ? launch_t<64, true>(a, blocks_g, s) : launch_t<64, false>(a, blocks_g, s);
    return hipErrorInvalidValue;
}

}  // namespace atlas
