/*
 * atlas.h -- C ABI of the hierarchical locality-preserving attention path for
 * AMD Instinct MI355X (gfx950): cube reorder, 3D RoPE with temporal scale r_t,
 * asymmetric global-local attention, cube unorder.
 *
 * Sources (web pages, cited by title and section):
 *   [TS] "Technische Samenvatting: AtlasVid" (gist.science), sections
 *        Methodologie 1 "Ontkoppeld Tweestapsproces" (Fase 1, Fase 2) and
 *        Methodologie 2 "Efficiente Gezamenlijke Denoising" (Asymmetrische
 *        Hierarchische Attention, Positie-uitlijning).
 *   [AB] "AtlasVid: Efficient Ultra-High-Resolution Long Video Generation via
 *        Decoupled Global-Local Modeling" (arxivdaily), English abstract.
 *
 * Conventions shared by every call
 *   - Tensors are device buffers laid out [tokens][heads][head_dim], row-major
 *     and contiguous (batch 1).  One token row holds heads*head_dim elements.
 *   - dtype: ATLAS_BF16 (bfloat16) or ATLAS_F32 (float32); all tensors of one
 *     call share it.  Attention always multiplies in bf16 on the matrix cores
 *     with fp32 accumulation: fp32 inputs are rounded to bf16 (nearest even)
 *     when staged, fp32 outputs are written without a final rounding.
 *   - Detail grid (T,H,W) with N = T*H*W tokens; cube (ct,ch,cw) must divide
 *     it, V = ct*ch*cw tokens per cube, N/V cubes.  Global proxy grid
 *     (Tg,Hg,Wg) with G = Tg*Hg*Wg tokens; {0,0,0} means no global tokens.
 *   - Cube order: cubes in raster order over the cube grid (t, then h, then
 *     w), tokens inside a cube in raster order.  Position p of the cube-order
 *     sequence holds the raster token pi(p) (the reading of [TS] Fase 2 used
 *     here; the pages say only that a cube's tokens become contiguous).
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call is asynchronous on it and never synchronises.
 *   - Ownership: the caller owns every buffer.  The library allocates and
 *     frees nothing, keeps no mutable global state beyond the last HIP error
 *     code (thread-local) and is re-entrant.
 *   - Errors: every call returns ATLAS_OK (0) or a negative ATLAS_ERR_* code.
 *     Arguments are validated on the host before any HIP call; on an error
 *     nothing is launched and no buffer is touched.  Device pointers are not
 *     dereferenced on the host and their kind is not checked.  Faults inside
 *     a kernel surface at the caller's next synchronisation of the stream.
 */
#ifndef ATLAS_H
#define ATLAS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t t, h, w;
} atlas_dim3;

enum {
    ATLAS_BF16 = 0,
    ATLAS_F32 = 1
};

enum {
    ATLAS_OK = 0,
    ATLAS_ERR_NULL = -1,        /* a required pointer is NULL */
    ATLAS_ERR_SHAPE = -2,       /* non-positive dim, cube does not divide grid,
                                   partly-zero proxy grid, or a size overflows */
    ATLAS_ERR_DTYPE = -3,       /* dtype is not ATLAS_BF16 / ATLAS_F32 */
    ATLAS_ERR_UNSUPPORTED = -4, /* head_dim not in {64, 128} */
    ATLAS_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    ATLAS_ERR_ALIAS = -6,       /* an output overlaps an input or another output */
    ATLAS_ERR_HIP = -7,         /* the kernel launch failed; see atlas_last_hip_error */
    ATLAS_ERR_VALUE = -8,       /* a scalar (r_t, theta, softmax_scale) is not finite
                                   or out of range */
    ATLAS_ERR_SCRATCH = -9      /* the problem needs more scratch memory than the
                                   fixed device array of the no-allocation entry
                                   point holds */
};

/*
 * atlas_cube_reorder -- [TS] Fase 2: the latent volume T x H x W is cut into
 * spatiotemporal cubes and tokens are rearranged so that the tokens of one
 * cube are contiguous ([AB]: reordered spatiotemporal windows).
 *   dst[p, :, :] = src[pi(p), :, :] for p in [0, N).
 *   dst, src: device, [N][heads][head_dim] of dtype; src in raster order,
 *   dst in cube order; must not overlap (ATLAS_ERR_ALIAS).  Bit-exact copy.
 */
int atlas_cube_reorder(void *dst, const void *src, atlas_dim3 grid, atlas_dim3 cube,
                       int32_t heads, int32_t head_dim, int32_t dtype, void *stream);

/*
 * atlas_cube_unorder -- inverse of atlas_cube_reorder: returns the detail
 * tokens to raster order after attention.
 *   dst[pi(p), :, :] = src[p, :, :].  Same arguments and rules as reorder.
 */
int atlas_cube_unorder(void *dst, const void *src, atlas_dim3 grid, atlas_dim3 cube,
                       int32_t heads, int32_t head_dim, int32_t dtype, void *stream);

/*
 * atlas_rope3d -- in-place 3D rotary position embedding of one tensor (call it
 * once for q and once for k).
 *   [TS] Fase 1: temporal RoPE indices of the global proxy are multiplied by
 *   r_t.  [TS] Positie-uitlijning: global-token RoPE coordinates are scaled by
 *   the resolution ratios onto the detail grid.
 *   Coordinates: the detail token at cube-order position p sits at the
 *   integer (t,h,w) of pi(p); the global token at raster position (tg,hg,wg)
 *   of the proxy grid sits at (r_t*tg, (H/Hg)*hg, (W/Wg)*wg).
 *   Rotation: head_dim/2 pairs (2i, 2i+1); the first head_dim/2 -
 *   2*floor(head_dim/6) pairs rotate with t, the next floor(head_dim/6) with
 *   h, the last floor(head_dim/6) with w; pair j of an axis with n pairs turns
 *   by coordinate * theta^(-j/n).  Every head of a token turns alike.
 *   x_detail: device [N][heads][head_dim] in cube order, or NULL to skip.
 *     Passing cube = grid (or ct = 1, ch | H, cw = W) makes pi the identity, so
 *     raster-order tensors can be rotated too.
 *   x_global: device [G][heads][head_dim] in raster order over gproxy, or NULL
 *     to skip; must be NULL when gproxy = {0,0,0}.  At least one is non-NULL.
 *   r_t > 0, theta > 1, both finite (ATLAS_ERR_VALUE).  Arithmetic in fp32,
 *   one rounding to dtype on the store.
 */
int atlas_rope3d(void *x_detail, void *x_global, atlas_dim3 grid, atlas_dim3 cube,
                 atlas_dim3 gproxy, float r_t, float theta, int32_t heads,
                 int32_t head_dim, int32_t dtype, void *stream);

/*
 * atlas_cube_reorder_rope3d -- atlas_cube_reorder followed by atlas_rope3d on
 * its output, in one pass over the detail rows ([TS] Methodologie 1, Fase 1
 * and Fase 2; Methodologie 2, Positie-uitlijning).  Same result, bit for bit,
 * as the two calls.
 *   x_detail: device [N][heads][head_dim], cube order (output).
 *   x_raster: device [N][heads][head_dim], raster order (input, unchanged).
 *   x_global: as for atlas_rope3d (rotated in place; may be NULL).
 *   x_detail and x_raster are both NULL (proxy only) or both given
 *   (ATLAS_ERR_NULL otherwise); neither may overlap the other or x_global
 *   (ATLAS_ERR_ALIAS).  Other arguments and errors as atlas_rope3d.
 */
int atlas_cube_reorder_rope3d(void *x_detail, const void *x_raster, void *x_global,
                              atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                              float r_t, float theta, int32_t heads, int32_t head_dim,
                              int32_t dtype, void *stream);

/*
 * atlas_hier_attn -- asymmetric hierarchical attention ([TS] Methodologie 2,
 * Asymmetrische Hierarchische Attention; [TS] Fase 2, locality-preserving
 * window attention; [AB]).  Global and detail tokens form one logical
 * sequence (no concatenated copy is made).  Per head:
 *   - a detail query at cube-order position p in cube c = p / V takes ONE
 *     softmax over the V keys of cube c and all G global keys;
 *   - a global query takes a softmax over the G global keys only (global ->
 *     detail is masked with -inf);
 *   o = sum_j softmax(scale * <q, k_j>)_j v_j.
 *   (The pages do not spell out which global tokens are "aligned" with a
 *   detail query; all of them are used.)
 *   o_detail: device [N][heads][head_dim], cube order (output).
 *   o_global: device [G][heads][head_dim] (output); ignored when G = 0.
 *   q_d, k_d, v_d: device [N][heads][head_dim], cube order (inputs).
 *   q_g, k_g, v_g: device [G][heads][head_dim] (inputs); ignored when G = 0.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim); NaN/inf -> ATLAS_ERR_VALUE.
 *   Outputs must not overlap any input or each other (ATLAS_ERR_ALIAS).
 *   Windows are the consecutive V-row blocks of the detail tensors as passed:
 *   given raster-order tensors (and RoPE at raster positions, i.e.
 *   atlas_rope3d with cube = grid), this is the naive block attention over the
 *   raster sequence that [TS] Experimentele Resultaten (Ablatiestudies)
 *   compares against.
 */
int atlas_hier_attn(void *o_detail, void *o_global,
                    const void *q_d, const void *k_d, const void *v_d,
                    const void *q_g, const void *k_g, const void *v_g,
                    atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                    int32_t heads, int32_t head_dim, float softmax_scale,
                    int32_t dtype, void *stream);

/*
 * atlas_hier_attn_raster -- atlas_hier_attn with the detail output written in
 * raster order: the output row of the cube-order query p is the raster token
 * of p (atlas_cube_unorder fused into the attention epilogue; [TS] Fase 2,
 * the cube reorder being a relabelling).  Same values, bit for bit, as
 * atlas_hier_attn followed by atlas_cube_unorder of o_detail.  Inputs as for
 * atlas_hier_attn (detail q, k, v in cube order); o_global unchanged.
 */
int atlas_hier_attn_raster(void *o_detail, void *o_global,
                           const void *q_d, const void *k_d, const void *v_d,
                           const void *q_g, const void *k_g, const void *v_g,
                           atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                           int32_t heads, int32_t head_dim, float softmax_scale,
                           int32_t dtype, void *stream);

/*
 * atlas_hier_attn_subset -- atlas_hier_attn (cube order) in which detail
 * window c sees, besides its V window keys, only the global keys listed for
 * it: rows win_gidx[win_goff[c]] .. win_gidx[win_goff[c+1] - 1] of k_g / v_g.
 * Global queries still see all G global keys.  This is the mask variant of
 * "aligned" global tokens ([TS] Methodologie 2, Asymmetrische Hierarchische
 * Attention): atlas_aligned_subset builds the co-located lists.  win_goff
 * (C + 1 entries, C = number of windows) and win_gidx (n_gidx entries) are
 * int32 arrays in device memory, 4-byte aligned, owned by the caller.  Lists
 * may be empty.  Valid lists have non-decreasing offsets from 0 to at most
 * n_gidx and indices in [0, G); for others the call still never reads outside
 * the arrays: offsets are clamped to [0, n_gidx], and an index outside [0, G)
 * reads as a zero key and value row (one extra key with logit 0 and value 0).
 * With G = 0 the lists are ignored (may be NULL).
 * Requires G * heads * head_dim * sizeof(dtype) < 2^31 (ATLAS_ERR_SHAPE).
 * Errors as for atlas_hier_attn; a list array overlapping an output is
 * ATLAS_ERR_ALIAS.
 */
int atlas_hier_attn_subset(void *o_detail, void *o_global,
                           const void *q_d, const void *k_d, const void *v_d,
                           const void *q_g, const void *k_g, const void *v_g,
                           const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
                           atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                           int32_t heads, int32_t head_dim, float softmax_scale,
                           int32_t dtype, void *stream);

/*
 * atlas_aligned_subset -- host-only.  The co-located global subset: proxy
 * token (tg, hg, wg) sits at (r_t*tg, (H/Hg)*hg, (W/Wg)*wg) on the detail
 * grid ([TS] Methodologie 2, Positie-uitlijning), and cube c = (a, b, e) (raster
 * order over the cube grid) lists the tokens whose position lies in its box
 * [a*ct, (a+1)*ct) x [b*ch, (b+1)*ch) x [e*cw, (e+1)*cw), in increasing raster
 * order over the proxy grid.  Spatial comparisons are exact; the temporal one
 * is made in fp64.  Writes win_goff[0 .. C] (host array of C + 1 int32) and,
 * when win_gidx is not NULL, the indices (host array of `capacity` int32).
 * Returns the number of listed tokens (with win_goff == NULL: only counts), or
 * a negative status: ATLAS_ERR_SHAPE, ATLAS_ERR_VALUE (r_t not positive and
 * finite, or capacity too small).
 */
int64_t atlas_aligned_subset(int32_t *win_goff, int32_t *win_gidx, int64_t capacity,
                             atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy, float r_t);

/*
 * atlas_hier_attn_fwd -- atlas_hier_attn (cube order) that also writes, for
 * every query, the natural log of its softmax denominator,
 *   lse_i = log sum_{j in K(i)} exp(scale * q_i.k_j),
 * which the backward pass needs.  lse_detail: float [heads][N] (head-major:
 * element h*N + p is cube-order query p of head h); lse_global: float
 * [heads][G] (NULL when G = 0).  o_detail, o_global and every input as for
 * atlas_hier_attn, bit for bit the same outputs.  lse buffers must be 16-byte
 * aligned and overlap no other buffer (ATLAS_ERR_ALIGN / ATLAS_ERR_ALIAS).
 */
int atlas_hier_attn_fwd(void *o_detail, void *o_global, float *lse_detail, float *lse_global,
                        const void *q_d, const void *k_d, const void *v_d,
                        const void *q_g, const void *k_g, const void *v_g,
                        atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                        int32_t heads, int32_t head_dim, float softmax_scale,
                        int32_t dtype, void *stream);

/* Bytes of device workspace atlas_hier_attn_bwd needs: 4 * heads * (N + G)
 * (the per-query products D_i = dO_i.o_i in fp32).  -1 on a bad shape. */
int64_t atlas_hier_attn_bwd_workspace_bytes(atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                                            int32_t heads, int32_t head_dim);

/*
 * atlas_hier_attn_bwd -- gradients of the asymmetric attention ([TS]
 * Methodologie 2, Asymmetrische Hierarchische Attention, whose LoRA
 * fine-tuning of the attention projections needs them) with respect to its
 * inputs.  For query i with key set K(i) (detail query of window c: the V keys
 * of window c and all G global keys; global query: the G global keys) and
 * P_ij = exp(scale q_i.k_j - lse_i), D_i = dO_i.o_i,
 * dS_ij = P_ij (dO_i.v_j - D_i):
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *   dv_j = sum_i P_ij dO_i   (sums over the allowed pairs).
 * Inputs: q/k/v, the forward outputs o and the upstream gradients dO, detail
 * tensors [N][heads][head_dim] in cube order and global tensors
 * [G][heads][head_dim], all of dtype `dtype`; lse_detail / lse_global from
 * atlas_hier_attn_fwd on the same inputs and scale.  Outputs dq/dk/dv in the
 * same layouts and dtype (fp32 accumulation, one rounding to the output dtype;
 * every row written).  `workspace` is caller-owned device memory of at least
 * atlas_hier_attn_bwd_workspace_bytes (16-byte aligned, contents on entry
 * irrelevant, overwritten).  The global pointers may be NULL when G = 0.
 * Outputs must not overlap any input, the workspace or each other
 * (ATLAS_ERR_ALIAS); a short workspace is ATLAS_ERR_VALUE.  Asynchronous on
 * `stream`; the library allocates nothing.
 */
int atlas_hier_attn_bwd(void *dq_d, void *dk_d, void *dv_d,
                        void *dq_g, void *dk_g, void *dv_g,
                        const void *q_d, const void *k_d, const void *v_d,
                        const void *q_g, const void *k_g, const void *v_g,
                        const void *o_d, const void *o_g, const void *do_d, const void *do_g,
                        const float *lse_detail, const float *lse_global,
                        void *workspace, int64_t workspace_bytes,
                        atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                        int32_t heads, int32_t head_dim, float softmax_scale,
                        int32_t dtype, void *stream);

/* Bytes of the fixed device array atlas_hier_attn_bwd_noalloc uses as its
 * workspace: 128 MiB (134217728), i.e. 4 * heads * (N + G) <= 128 MiB. */
#define ATLAS_NOALLOC_SCRATCH_BYTES 134217728

/*
 * atlas_hier_attn_bwd_noalloc -- atlas_hier_attn_bwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc).  Same arguments, outputs
 * and errors as atlas_hier_attn_bwd without the workspace: the D rows live in
 * a file-scope device array of ATLAS_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends.  The call allocates
 * nothing (no hipMalloc / hipFree, no allocating library routine); its first
 * call on a device looks up that device's copy of the array.  A problem whose
 * workspace (atlas_hier_attn_bwd_workspace_bytes) exceeds the array is
 * rejected with ATLAS_ERR_SCRATCH before anything is launched.  The array
 * keeps the last call's contents; every byte the call reads is first written
 * by the same call, so nothing needs clearing.  All calls on one GPU share
 * the array: calls that overlap in time on one GPU (several streams or host
 * threads without ordering between them) race on it.
 */
int atlas_hier_attn_bwd_noalloc(void *dq_d, void *dk_d, void *dv_d,
                                void *dq_g, void *dk_g, void *dv_g,
                                const void *q_d, const void *k_d, const void *v_d,
                                const void *q_g, const void *k_g, const void *v_g,
                                const void *o_d, const void *o_g, const void *do_d,
                                const void *do_g, const float *lse_detail,
                                const float *lse_global, atlas_dim3 grid, atlas_dim3 cube,
                                atlas_dim3 gproxy, int32_t heads, int32_t head_dim,
                                float softmax_scale, int32_t dtype, void *stream);

/*
 * atlas_hier_attn_subset_fwd -- atlas_hier_attn_subset that also writes the
 * log-sum-exp of every query over its key set (the window keys and the
 * listed global keys for a detail query), laid out as in atlas_hier_attn_fwd.
 * Arguments and errors as for atlas_hier_attn_subset and atlas_hier_attn_fwd.
 */
int atlas_hier_attn_subset_fwd(void *o_detail, void *o_global,
                               float *lse_detail, float *lse_global,
                               const void *q_d, const void *k_d, const void *v_d,
                               const void *q_g, const void *k_g, const void *v_g,
                               const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
                               atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                               int32_t heads, int32_t head_dim, float softmax_scale,
                               int32_t dtype, void *stream);

/* Bytes of device workspace atlas_hier_attn_subset_bwd needs: the D rows
 * (4 * heads * (N + G), rounded up to 256) and two fp32 accumulators of the
 * global keys' gradients (2 * 4 * G * heads * head_dim).  -1 on a bad shape. */
int64_t atlas_hier_attn_subset_bwd_workspace_bytes(atlas_dim3 grid, atlas_dim3 cube,
                                                   atlas_dim3 gproxy, int32_t heads,
                                                   int32_t head_dim);

/*
 * atlas_hier_attn_subset_bwd -- gradients of atlas_hier_attn_subset ([TS]
 * Methodologie 2: the attention with the "aligned" global tokens, whose LoRA
 * fine-tuning needs them), as atlas_hier_attn_bwd with the key set of a
 * detail query in window c restricted to its window keys and the global rows
 * listed for it.  A global key's dk / dv sums over every global query and
 * over the detail queries of every window that lists it (a row listed twice
 * for one window counts twice, as in the forward's softmax); an index
 * outside [0, G) is the zero key of the forward and receives no gradient.
 * lse_detail / lse_global from atlas_hier_attn_subset_fwd with the same lists.
 * The lists are the device arrays of atlas_hier_attn_subset (same validation;
 * they may not overlap any gradient either).  `workspace` holds at least
 * atlas_hier_attn_subset_bwd_workspace_bytes (16-byte aligned, overwritten).
 * The global keys' detail share is summed with fp32 atomic adds, so dk_g and
 * dv_g may differ in the last bits from run to run; every other output is
 * deterministic.  Errors as for atlas_hier_attn_bwd.
 */
int atlas_hier_attn_subset_bwd(void *dq_d, void *dk_d, void *dv_d,
                               void *dq_g, void *dk_g, void *dv_g,
                               const void *q_d, const void *k_d, const void *v_d,
                               const void *q_g, const void *k_g, const void *v_g,
                               const void *o_d, const void *o_g, const void *do_d, const void *do_g,
                               const float *lse_detail, const float *lse_global,
                               const int32_t *win_goff, const int32_t *win_gidx, int64_t n_gidx,
                               void *workspace, int64_t workspace_bytes,
                               atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                               int32_t heads, int32_t head_dim, float softmax_scale,
                               int32_t dtype, void *stream);

/* Useful attention FLOPs of one atlas_hier_attn call: 4 * head_dim * heads *
 * (N*(V+G) + G*G), i.e. 2*head_dim per (q,k) pair for q.k and 2*head_dim for
 * p*v over the unmasked pairs only.  Host-only; returns -1 on a bad shape. */
double atlas_hier_attn_useful_flops(atlas_dim3 grid, atlas_dim3 cube, atlas_dim3 gproxy,
                                    int32_t heads, int32_t head_dim);

/* Static description of a status code (never NULL). */
const char *atlas_status_string(int status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int atlas_last_hip_error(void);

/* ABI version: major*10000 + minor*100 + patch. */
int atlas_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATLAS_H */
