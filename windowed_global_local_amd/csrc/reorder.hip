// reorder.hip -- cube reorder / unorder of token rows on gfx950.
//
// "Technische Samenvatting: AtlasVid", Methodologie 1, Fase 2: the latent
// volume is cut into spatiotemporal cubes and the tokens of one cube are made
// contiguous.  Cube order enumerates cubes in raster order over the cube grid
// and the tokens of a cube in raster order.
//
// A run = the cw tokens of one (cube, frame, row): contiguous in both orders,
// cw * row_bytes bytes (245,760 B for cw = 24 at 40 heads x 128 bf16).  The
// kernel is a batched copy of runs: every workgroup moves one segment of one
// run with 16-byte non-temporal loads and stores, so both sides stream at
// full cache-line granularity and nothing lingers in L2/MALL.  HBM bound:
// 2 * N * row_bytes bytes per call.
#include "atlas_internal.hpp"

namespace atlas {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Launch shape: the fastest of a sweep on MI355X at the 4K workload (64 to
// 256 threads, 1 to 4 chunks per thread): small workgroups spread the 14 GB
// copy most evenly over the 256 CUs -- 6.7 TB/s for reorder, 6.3 TB/s for
// unorder.
constexpr int kThreads = 64;
constexpr int kUnroll = 1;
constexpr uint32_t kSegChunks = kThreads * kUnroll;   // 16-byte chunks per workgroup

__global__ __launch_bounds__(kThreads) void copy_runs_kernel(const CopyRunsArgs a)
{
    const uint32_t wg = blockIdx.x;
    const uint32_t run = wg / a.segs_per_run;
    const uint32_t seg = wg - run * a.segs_per_run;

    // run -> (cube c, frame-in-cube dt, row-in-cube dh)
    const uint32_t runs_per_cube = (uint32_t)(a.ct * a.ch);
    const uint32_t c = run / runs_per_cube;
    const uint32_t k = run - c * runs_per_cube;
    const uint32_t dt = k / (uint32_t)a.ch;
    const uint32_t dh = k - dt * (uint32_t)a.ch;
    const uint32_t cubes_per_frame = (uint32_t)(a.nH * a.nW);
    const uint32_t ca = c / cubes_per_frame;
    const uint32_t crem = c - ca * cubes_per_frame;
    const uint32_t cb = crem / (uint32_t)a.nW;
    const uint32_t ce = crem - cb * (uint32_t)a.nW;

    const int64_t raster_tok =
        ((int64_t)(ca * a.ct + dt) * a.H + (int64_t)(cb * a.ch + dh)) * a.W + (int64_t)ce * a.cw;
    const int64_t cube_tok = (int64_t)run * a.cw;
    const int64_t src_tok = a.inverse ? cube_tok : raster_tok;
    const int64_t dst_tok = a.inverse ? raster_tok : cube_tok;

    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.src + src_tok * a.row_bytes);
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.dst + dst_tok * a.row_bytes);

    const uint32_t base = seg * kSegChunks + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const uint32_t idx = base + i * kThreads;
        if (idx < a.run_chunks)
            v[i] = __builtin_nontemporal_load(src + idx);
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const uint32_t idx = base + i * kThreads;
        if (idx < a.run_chunks)
            __builtin_nontemporal_store(v[i], dst + idx);
    }
}

}  // namespace

hipError_t launch_copy_runs(const CopyRunsArgs &a0, int64_t n_runs, hipStream_t s)
{
    CopyRunsArgs a = a0;
    a.segs_per_run = (a.run_chunks + kSegChunks - 1) / kSegChunks;
    const int64_t blocks = n_runs * (int64_t)a.segs_per_run;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(copy_runs_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace atlas
