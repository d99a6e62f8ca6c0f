// atlas_internal.hpp -- launch descriptors shared by the C-ABI layer and the
// gfx950 kernels of the hierarchical locality-preserving attention path.
// Nothing here is part of the public ABI (that is include/atlas.h).
#pragma once

#include <hip/hip_runtime.h>
#include "atlas.h"
#include <stdint.h>

namespace atlas {

// ---------------------------------------------------------------- reorder
// One "run" is cw consecutive tokens of one raster row of one cube: it is
// contiguous both in raster order and in cube order, so a reorder is a set of
// run copies of cw * row_bytes bytes each.
struct CopyRunsArgs {
    const char *src;
    char *dst;
    int64_t row_bytes;      // bytes of one token row (multiple of 16)
    int32_t H, W;           // detail grid rows / columns
    int32_t ct, ch, cw;     // cube
    int32_t nH, nW;         // cube grid (H/ch, W/cw)
    uint32_t run_chunks;    // 16-byte chunks per run = cw * row_bytes / 16
    uint32_t segs_per_run;  // workgroups per run
    int32_t inverse;        // 0: dst(cube order) <- src(raster); 1: the reverse
};

hipError_t launch_copy_runs(const CopyRunsArgs &a, int64_t n_runs, hipStream_t s);

// ---------------------------------------------------------------- rope
constexpr int kMaxPairs = 64;   // head_dim <= 128

struct RopeArgs {
    void *xd;               // detail tensor (cube order) or nullptr
    const void *src_d;      // fused reorder: raster-order source of xd (else nullptr)
    void *xg;               // global tensor (proxy raster order) or nullptr
    int64_t N, G;           // tokens in xd / xg (0 when skipped)
    int32_t heads;
    int32_t T, H, W;
    int32_t ct, ch, cw, nH, nW;
    int32_t Hg, Wg;
    double r_t;             // temporal scale of proxy coordinates
    double sh, sw;          // H / Hg and W / Wg
    int32_t n_t, n_h;       // pairs on the t axis, on the h axis (rest: w)
    int32_t blocks_d;       // workgroups that cover xd
    uint32_t row_chunks;    // 16-byte chunks per token row
    uint64_t fd_mul;        // ceil(2^40 / row_chunks): n / row_chunks = (n * fd_mul) >> 40
                            // exactly whenever n * row_chunks <= 2^40 (here n < 2^21,
                            // row_chunks <= 2^17)
    double omega[kMaxPairs];   // per-pair angular frequency
};

hipError_t launch_rope(const RopeArgs &a, int head_dim, int is_f32, int64_t blocks_g,
                       hipStream_t s);   // fused reorder when a.src_d != nullptr
int rope_tokens_per_block(int head_dim);

// ---------------------------------------------------------------- attention
struct AttnArgs {
    const void *qd, *kd, *vd;
    const void *qg, *kg, *vg;
    void *od, *og;
    float *lse_d, *lse_g;   // log-sum-exp outputs [heads][N], [heads][G] (or nullptr)
    // per-window global subset (nullptr: every window sees all G global keys):
    // window c sees rows gidx[goff[c] .. goff[c+1]) of the global K/V
    const int32_t *goff, *gidx;
    int32_t n_gidx;         // entries of gidx
    int64_t V;              // tokens per cube window
    int64_t G;              // global tokens
    int64_t C;              // number of windows
    int32_t heads;
    int32_t qb_win;         // query blocks per window
    int32_t qb_glob;        // query blocks over the global queries
    int64_t items_per_head; // C * qb_win + qb_glob
    int64_t items;          // heads * items_per_head
    float c_log2;           // softmax scale * log2(e)
    // raster epilogue: detail outputs go to the raster row of their token
    int32_t raster;         // 0: cube order, 1: raster order
    int32_t ct, ch, cw;     // cube
    int32_t nH, nW;         // cubes per frame along h, w
    int32_t H, W;           // detail grid height, width
};

hipError_t launch_hier_attn(const AttnArgs &a, int head_dim, int is_f32, hipStream_t s);
int hier_attn_block_rows();

// ---------------------------------------------------------------- attention backward
struct BwdArgs {
    const void *qd, *kd, *vd, *dod;     // detail tensors (cube order)
    const void *qg, *kg, *vg, *dog;     // global tensors
    void *dqd, *dkd, *dvd;              // detail gradients
    void *dqg, *dkg, *dvg;              // global gradients
    const float *lse_d, *lse_g;         // forward log-sum-exp [heads][N], [heads][G]
    const float *dl_d, *dl_g;           // D = dO.o [heads][N], [heads][G] (workspace)
    int64_t N, V, G, C;
    int32_t heads;
    int32_t qb_win, qb_glob;            // dq: query blocks per window / over global queries
    int32_t kb_win, kb_glob;            // dk/dv: key blocks per window / over global keys
    int64_t dq_items_per_head;          // C * qb_win + qb_glob
    int64_t dq_items;                   // heads * dq_items_per_head
    int64_t kv_items_glob;              // heads * kb_glob (launched first)
    int64_t kv_items;                   // kv_items_glob + heads * C * kb_win
    float c_log2;                       // softmax scale * log2(e)
    float scale;                        // softmax scale
    // per-window global subset (null: every detail query sees all G global keys):
    // window c lists global rows gidx[goff[c] .. goff[c+1]) (clamped to n_gidx; an
    // index outside [0, G) reads as a zero row and receives no gradient)
    const int32_t *goff, *gidx;
    int32_t n_gidx;
    float *acc_k, *acc_v;               // fp32 [G][heads][D]: detail share of dk/dv (workspace)
};

// delta (into dl_d / dl_g), then dq, then dk/dv; od / og are the forward outputs
hipError_t launch_hier_attn_bwd(const BwdArgs &a, const void *od, const void *og, int head_dim,
                                int is_f32, hipStream_t s);
int hier_attn_bwd_block_rows();   // keys per dk/dv workgroup
int hier_attn_bwd_dq_rows();      // queries per dq workgroup

// records a HIP error for atlas_last_hip_error() on the calling thread
void note_hip_error(int e);

// Supplies the device address of a fixed scratch array (ATLAS_OK, or an
// ATLAS_ERR_* code after note_hip_error).
typedef int (*ScratchFn)(void **ptr);

// atlas_hier_attn_bwd with the workspace taken from get_scratch (called only
// after every argument check has passed) instead of a caller buffer; a problem
// needing more than scratch_bytes is ATLAS_ERR_SCRATCH.
int hier_attn_bwd_scratch(void *dq_d, void *dk_d, void *dv_d, void *dq_g, void *dk_g, void *dv_g,
                          const void *q_d, const void *k_d, const void *v_d, const void *q_g,
                          const void *k_g, const void *v_g, const void *o_d, const void *o_g,
                          const void *do_d, const void *do_g, const float *lse_detail,
                          const float *lse_global, ScratchFn get_scratch, int64_t scratch_bytes,
                          atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, int32_t heads,
                          int32_t head_dim, float softmax_scale, int32_t dtype, void *stream);

}  // namespace atlas
