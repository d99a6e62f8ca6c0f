// hier_attn_bwd.hip -- backward of the asymmetric hierarchical attention on gfx950.
//
// The attention is the one of "Technische Samenvatting: AtlasVid",
// Methodologie 2 (Asymmetrische Hierarchische Attention): a detail query in
// cube window c takes one softmax over the V keys of its window plus all G
// global keys, a global query one softmax over the G global keys.  The pages
// fine-tune attention projections (LoRA at 720P, same section), which needs the
// gradients of this attention with respect to q, k and v.  With the forward's
// log-sum-exp lse_i of the scaled logits and the upstream gradient dO:
//   P_ij = exp(scale q_i.k_j - lse_i),  dP_ij = dO_i.v_j,  D_i = dO_i.o_i,
//   dS_ij = P_ij (dP_ij - D_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i,
// each sum over the (query, key) pairs the mask allows.
//
// Three kernels, no atomics, every gradient row written once:
//   delta  D_i = dO_i.o_i per (query, head), fp32, into the caller's workspace;
//   dq     one workgroup per 128 queries of one head (a window block or a
//          global block), streaming that query's key list in 64-key tiles, as
//          the forward does: S^T = K Q^T and dP^T = V dO^T put one query in each
//          lane, dS^T = P^T o (dP^T - D) is formed in registers and
//          dq^T += K^T dS^T (K^T staged transposed, in the permuted key order
//          that matches the S^T register layout);
//   dk/dv  one workgroup per 128 keys of one head, streaming every query that
//          sees those keys in 64-query tiles (a window's keys: the window's V
//          queries; a global key block: all N detail and G global queries):
//          S = Q K^T and dP = dO V^T put one key in each lane,
//          dv^T += dO^T P and dk^T += Q^T dS with dO^T and Q^T staged
//          transposed.  K and V of the block stay in registers.
// Splitting dq from dk/dv recomputes S and dP once more, but a key-major pass
// that also produced dq would have to add every global key block's partial
// dq into every query row (hundreds of partial sums per row), and a
// query-major pass the same for dk/dv of the global keys.
//
// All rows outside a list read as zeros (buffer range checks); rows past the
// end of a query tile get lse = +inf, so their P and dS are exactly 0, and
// keys past the end of a key block only fill accumulator columns that are
// never stored.  Matrix products run on v_mfma_f32_32x32x16_bf16 with bf16
// operands (P and dS rounded to bf16) and fp32 accumulation.
#include "atlas_internal.hpp"
#include "mfma_util.hpp"

#include <type_traits>

namespace atlas {

namespace {

using namespace mfma;

constexpr int kBW = 4;                  // waves per workgroup (one per SIMD)
constexpr int kBThreads = kBW * 64;
constexpr int kBRows = kBW * 32;        // queries (dq) or keys (dk/dv) per workgroup
constexpr int kT = 64;                  // rows per streamed tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BTile {
    // row stages pad rows by 16 bytes, transposed stages hold 64 rows padded to
    // 72 elements (the bank-conflict-free strides of the forward kernel)
    static constexpr int kRStr = D + 8;
    static constexpr int kTStr = kT + 8;
    static constexpr int kRElems = kT * kRStr;
    static constexpr int kTElems = D * kTStr;
    static constexpr int kKs = D / 16;                        // k-steps over head_dim
    static constexpr int kDt = D / 32;                        // 32-row tiles of a D x 32 result
    static constexpr int kRC = kT * (D / 8) / kBThreads;      // row-stage chunks per thread
    static constexpr int kTC = 32 * (D / 8) / kBThreads;      // transposed-stage tasks per thread
};

// Per-thread staging offsets.  Row stage: chunk e = tid + 256u is row e/(D/8),
// 8-element column e%(D/8).  Transposed stage: a task is a row pair
// (2pp, 2pp+1) times an 8-element column block dc; its eight 4-byte stores pair
// the two rows at one column (64 lanes of a wave hit 64 distinct banks).
template <int D, int kEsize>
struct StageMap {
    using TL = BTile<D>;
    uint32_t rgoff[TL::kRC];
    int rlds[TL::kRC];
    uint32_t tgoff[TL::kTC];
    int tlds[TL::kTC];

    __device__ StageMap(int tid, int wave, int lane, uint32_t rb)
    {
#pragma unroll
        for (int u = 0; u < TL::kRC; ++u) {
            const int e = tid + kBThreads * u;
            const int row = e / (D / 8), ch = e % (D / 8);
            rgoff[u] = (uint32_t)row * rb + (uint32_t)(ch * 8 * kEsize);
            rlds[u] = row * TL::kRStr + ch * 8;
        }
#pragma unroll
        for (int u = 0; u < TL::kTC; ++u) {
            const int pp = lane & 31;
            const int dc = 2 * (wave + kBW * u) + (lane >> 5);
            const int r0 = 2 * pp;
            tgoff[u] = (uint32_t)r0 * rb + (uint32_t)(dc * 8 * kEsize);
            tlds[u] = (8 * dc) * TL::kTStr + tperm(r0);
        }
    }
};

// registers of a transposed-stage task -> LDS (rows 2pp, 2pp+1 at 8 columns)
template <int D>
__device__ inline void tstore(__bf16 *col, const u32x4 x, const u32x4 y)
{
    using TL = BTile<D>;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint32_t *>(col + (2 * m) * TL::kTStr) = __builtin_amdgcn_perm(y[m], x[m], 0x05040100u);
        *reinterpret_cast<uint32_t *>(col + (2 * m + 1) * TL::kTStr) = __builtin_amdgcn_perm(y[m], x[m], 0x07060302u);
    }
}

// 4 consecutive fp32 results -> output row (bf16 rounds to nearest even)
template <bool F32>
__device__ inline void store4(void *base, int64_t off, float v0, float v1, float v2, float v3)
{
    if constexpr (F32) {
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + off) = make_float4(v0, v1, v2, v3);
    } else {
        bf16x4 w;
        w[0] = (__bf16)v0; w[1] = (__bf16)v1; w[2] = (__bf16)v2; w[3] = (__bf16)v3;
        *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(base) + off) = w;
    }
}

// ------------------------------------------------------------------ delta
// D_i = dO_i . o_i for every (row, head): D/8 lanes per (row, head), 8
// elements per lane, a butterfly over the D/8 lanes.
template <int D, bool F32>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void *o, const void *dO, float *delta,
                                                        int64_t rows, int32_t heads)
{
    constexpr int kL = D / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t pair = t / kL;            // row * heads + head
    const int sub = threadIdx.x % kL;
    float acc = 0.0f;
    if (pair < rows * heads) {
        const int64_t off = pair * D + sub * 8;
        if constexpr (F32) {
            const float4 *a = reinterpret_cast<const float4 *>(static_cast<const float *>(o) + off);
            const float4 *b = reinterpret_cast<const float4 *>(static_cast<const float *>(dO) + off);
            const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
            acc = a0.x * b0.x + a0.y * b0.y + a0.z * b0.z + a0.w * b0.w
                + a1.x * b1.x + a1.y * b1.y + a1.z * b1.z + a1.w * b1.w;
        } else {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(o) + off);
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(dO) + off);
#pragma unroll
            for (int m = 0; m < 8; ++m)
                acc = fmaf((float)a[m], (float)b[m], acc);
        }
    }
#pragma unroll
    for (int w = kL / 2; w >= 1; w >>= 1)
        acc += __shfl_xor(acc, w);
    if (pair < rows * heads && sub == 0) {
        const int64_t row = pair / heads;
        const int32_t head = (int32_t)(pair - row * heads);
        delta[(int64_t)head * rows + row] = acc;
    }
}

// --------------------------------------------------------------------- dq
template <int D, bool F32>
__global__ __launch_bounds__(kBThreads) void bwd_dq_kernel(const BwdArgs a)
{
    using TL = BTile<D>;
    constexpr int kEsize = F32 ? 4 : 2;
    constexpr int kStage = 2 * TL::kRElems + TL::kTElems;     // K rows | V rows | K^T
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int64_t head = item / a.dq_items_per_head;
    const int64_t rem = item - head * a.dq_items_per_head;
    const int64_t ndet = a.C * a.qb_win;
    const bool glob = rem >= ndet;
    const int64_t rs = (int64_t)a.heads * D;
    const uint32_t rb = (uint32_t)(rs * kEsize);
    const int64_t hoff = head * D;

    int64_t q_row0, n_q, kw_row0;
    int32_t n_win;
    const void *qptr, *doptr;
    void *dqptr;
    const float *lse, *dl;
    if (!glob) {
        const int64_t c = rem / a.qb_win;
        const int64_t qb = rem - c * a.qb_win;
        q_row0 = c * a.V + qb * kBRows;
        n_q = min<int64_t>(kBRows, a.V - qb * kBRows);
        n_win = (int32_t)a.V;
        kw_row0 = c * a.V;
        qptr = a.qd;
        doptr = a.dod;
        dqptr = a.dqd;
        lse = a.lse_d + head * a.N;
        dl = a.dl_d + head * a.N;
    } else {
        const int64_t gb = rem - ndet;
        q_row0 = gb * kBRows;
        n_q = min<int64_t>(kBRows, a.G - gb * kBRows);
        n_win = 0;
        kw_row0 = 0;
        qptr = a.qg;
        doptr = a.dog;
        dqptr = a.dqg;
        lse = a.lse_g + head * a.G;
        dl = a.dl_g + head * a.G;
    }
    const int32_t nkeys = n_win + (int32_t)a.G;
    const int ntiles = (nkeys + kT - 1) / kT;

    // B operands of S^T = K Q^T and dP^T = V dO^T: column = query l32, k-half hh
    const int my_q = wave * 32 + l32;
    const bool wave_active = wave * 32 < n_q;
    const bool row_ok = my_q < n_q;
    bf16x8 qf[TL::kKs], df[TL::kKs];
    const int64_t qoff = (q_row0 + my_q) * rs + hoff + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < TL::kKs; ++ks) {
        qf[ks] = row_ok ? gload8<F32>(qptr, qoff + ks * 16) : zero8();
        df[ks] = row_ok ? gload8<F32>(doptr, qoff + ks * 16) : zero8();
    }
    const float lse2 = row_ok ? lse[q_row0 + my_q] * kLog2e : 0.0f;
    const float dlt = row_ok ? dl[q_row0 + my_q] : 0.0f;

    const StageMap<D, kEsize> sm(tid, wave, lane, rb);
    const char *kwin = static_cast<const char *>(a.kd) + (kw_row0 * rs + hoff) * kEsize;
    const char *vwin = static_cast<const char *>(a.vd) + (kw_row0 * rs + hoff) * kEsize;
    const char *kglb = static_cast<const char *>(a.kg) + hoff * kEsize;
    const char *vglb = static_cast<const char *>(a.vg) + hoff * kEsize;

    u32x4 kst[TL::kRC], vst[TL::kRC], tst[TL::kTC][2];

    // global -> registers for key tile t (window keys, global keys, or the
    // one tile that straddles the two lists: then both are read and OR-ed, each
    // read returning zeros outside its own list)
    auto gload = [&](int t) {
        const int32_t k0 = t * kT;
        if (k0 + kT <= n_win || k0 >= n_win) {
            const bool in_win = k0 < n_win;
            const int32_t g0 = k0 - n_win;
            const int32_t rows = in_win ? kT : max(0, min(kT, (int32_t)a.G - g0));
            const char *kb = in_win ? kwin + (int64_t)k0 * rb : kglb + (int64_t)g0 * rb;
            const char *vb = in_win ? vwin + (int64_t)k0 * rb : vglb + (int64_t)g0 * rb;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)rows * rb);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)rows * rb);
#pragma unroll
            for (int u = 0; u < TL::kRC; ++u) {
                kst[u] = bload8<F32>(rk, sm.rgoff[u]);
                vst[u] = bload8<F32>(rv, sm.rgoff[u]);
            }
#pragma unroll
            for (int u = 0; u < TL::kTC; ++u) {
                tst[u][0] = bload8<F32>(rk, sm.tgoff[u]);
                tst[u][1] = bload8<F32>(rk, sm.tgoff[u] + rb);
            }
        } else {
            const int32_t r0 = n_win - k0;
            const int32_t ng = max(0, min(kT - r0, (int32_t)a.G));
            const __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            const __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            const __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)ng * rb);
            const __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)ng * rb);
            // rows < r0 give offsets that wrap to huge unsigned values in the
            // global buffer (out of range -> 0); rows >= r0 are past the window
            const uint32_t gs = (uint32_t)r0 * rb;
#pragma unroll
            for (int u = 0; u < TL::kRC; ++u) {
                kst[u] = bload8<F32>(rkw, sm.rgoff[u]) | bload8<F32>(rkg, sm.rgoff[u] - gs);
                vst[u] = bload8<F32>(rvw, sm.rgoff[u]) | bload8<F32>(rvg, sm.rgoff[u] - gs);
            }
#pragma unroll
            for (int u = 0; u < TL::kTC; ++u)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t off = sm.tgoff[u] + (uint32_t)j * rb;
                    tst[u][j] = bload8<F32>(rkw, off) | bload8<F32>(rkg, off - gs);
                }
        }
    };

    auto lstore = [&](int buf) {
        __bf16 *Ks = lds + buf * kStage;
        __bf16 *Vs = Ks + TL::kRElems;
        __bf16 *Ts = Vs + TL::kRElems;
#pragma unroll
        for (int u = 0; u < TL::kRC; ++u) {
            *reinterpret_cast<u32x4 *>(Ks + sm.rlds[u]) = kst[u];
            *reinterpret_cast<u32x4 *>(Vs + sm.rlds[u]) = vst[u];
        }
#pragma unroll
        for (int u = 0; u < TL::kTC; ++u)
            tstore<D>(Ts + sm.tlds[u], tst[u][0], tst[u][1]);
    };

    f32x16 dq[TL::kDt];
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dq[dt][r] = 0.0f;
    const float cl = a.c_log2;

    auto tile = [&](int buf, int t, auto masked_c) {
        constexpr bool kMasked = decltype(masked_c)::value;
        const __bf16 *Ks = lds + buf * kStage;
        const __bf16 *Vs = Ks + TL::kRElems;
        const __bf16 *Ts = Vs + TL::kRElems;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kt][r] = 0.0f;
                dp[kt][r] = 0.0f;
            }
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                    Ks + (kt * 32 + l32) * TL::kRStr + ks * 16 + 8 * hh);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[kt], 0, 0, 0);
            }
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 va = *reinterpret_cast<const bf16x8 *>(
                    Vs + (kt * 32 + l32) * TL::kRStr + ks * 16 + 8 * hh);
                dp[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp[kt], 0, 0, 0);
            }
        if constexpr (kMasked) {
            const int32_t kbase = t * kT;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (kbase + key >= nkeys)
                        s[kt][r] = -INFINITY;
                }
        }
        // dS^T = P^T o (dP^T - D), P^T = exp2(S^T cl - lse2), in bf16
        bf16x8 ds[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int r = 8 * i2 + m;
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], cl, -lse2));
                    ds[kt][i2][m] = (__bf16)(p * (dp[kt][r] - dlt));
                }
        // dq^T += K^T dS^T
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int dt = 0; dt < TL::kDt; ++dt) {
                    const bf16x8 ta = *reinterpret_cast<const bf16x8 *>(
                        Ts + (dt * 32 + l32) * TL::kTStr + 8 * hh + 16 * (2 * kt + i2));
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, ds[kt][i2], dq[dt], 0, 0, 0);
                }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t + 1 < ntiles; ++t) {
        const int buf = t & 1;
        gload(t + 1);
        if (wave_active)
            tile(buf, t, std::false_type{});
        lstore(buf ^ 1);
        __syncthreads();
    }
    if (!wave_active)
        return;
    tile((ntiles - 1) & 1, ntiles - 1, std::true_type{});
    if (!row_ok)
        return;

    const float sc = a.scale;
    const int64_t obase = (q_row0 + my_q) * rs + hoff;
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = dt * 32 + 8 * i + 4 * hh;
            store4<F32>(dqptr, obase + d, dq[dt][4 * i] * sc, dq[dt][4 * i + 1] * sc,
                        dq[dt][4 * i + 2] * sc, dq[dt][4 * i + 3] * sc);
        }
}

// ------------------------------------------------------------------ dk/dv
template <int D, bool F32>
__global__ __launch_bounds__(kBThreads) void bwd_dkdv_kernel(const BwdArgs a)
{
    using TL = BTile<D>;
    constexpr int kEsize = F32 ? 4 : 2;
    constexpr int kStage = 2 * TL::kRElems + 2 * TL::kTElems;   // Q rows | dO rows | Q^T | dO^T
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * kStage];
    __shared__ __attribute__((aligned(16))) float lsd[2][2][kT];  // [buf][lse2 | D][row]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // global key blocks first (long query lists), then the window key blocks;
    // within each phase an XCD walks a contiguous range, i.e. one head at a time
    const uint32_t n1 = (uint32_t)a.kv_items_glob;
    const uint32_t bid = blockIdx.x;
    const bool glob = bid < n1;
    int64_t head, k_row0, n_k;
    const void *kptr, *vptr;
    void *dkptr, *dvptr;
    // query segments: [q0, q0 + nq) of (qp, dop, lsp, dlp)
    const void *qp0, *dop0, *qp1, *dop1;
    const float *ls0, *dl0, *ls1, *dl1;
    int64_t q00, nq0, nq1;
    if (glob) {
        const int64_t item = xcd_item(bid, n1);
        head = item / a.kb_glob;
        const int64_t gb = item - head * a.kb_glob;
        k_row0 = gb * kBRows;
        n_k = min<int64_t>(kBRows, a.G - k_row0);
        kptr = a.kg;
        vptr = a.vg;
        dkptr = a.dkg;
        dvptr = a.dvg;
        qp0 = a.qd; dop0 = a.dod; ls0 = a.lse_d + head * a.N; dl0 = a.dl_d + head * a.N;
        q00 = 0; nq0 = a.N;
        qp1 = a.qg; dop1 = a.dog; ls1 = a.lse_g + head * a.G; dl1 = a.dl_g + head * a.G;
        nq1 = a.G;
    } else {
        const int64_t per_head = a.C * a.kb_win;
        const int64_t item = xcd_item(bid - n1, gridDim.x - n1);
        head = item / per_head;
        const int64_t r = item - head * per_head;
        const int64_t c = r / a.kb_win;
        const int64_t kb = r - c * a.kb_win;
        k_row0 = c * a.V + kb * kBRows;
        n_k = min<int64_t>(kBRows, a.V - kb * kBRows);
        kptr = a.kd;
        vptr = a.vd;
        dkptr = a.dkd;
        dvptr = a.dvd;
        qp0 = a.qd; dop0 = a.dod; ls0 = a.lse_d + head * a.N; dl0 = a.dl_d + head * a.N;
        q00 = c * a.V; nq0 = a.V;
        qp1 = nullptr; dop1 = nullptr; ls1 = nullptr; dl1 = nullptr;
        nq1 = 0;
    }
    const int64_t rs = (int64_t)a.heads * D;
    const uint32_t rb = (uint32_t)(rs * kEsize);
    const int64_t hoff = head * D;
    const int tiles0 = (int)((nq0 + kT - 1) / kT);
    const int ntiles = tiles0 + (int)((nq1 + kT - 1) / kT);

    // B operands of S = Q K^T and dP = dO V^T: column = key l32, k-half hh
    const int my_k = wave * 32 + l32;
    const bool wave_active = wave * 32 < n_k;
    const bool key_ok = my_k < n_k;
    bf16x8 kf[TL::kKs], vf[TL::kKs];
    const int64_t koff = (k_row0 + my_k) * rs + hoff + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < TL::kKs; ++ks) {
        kf[ks] = key_ok ? gload8<F32>(kptr, koff + ks * 16) : zero8();
        vf[ks] = key_ok ? gload8<F32>(vptr, koff + ks * 16) : zero8();
    }

    const StageMap<D, kEsize> sm(tid, wave, lane, rb);
    u32x4 qst[TL::kRC], ost[TL::kRC], qtst[TL::kTC][2], otst[TL::kTC][2];
    float lsv = 0.0f;   // this thread's lse2 (tid < 64) or D (64 <= tid < 128) value

    auto gload = [&](int t) {
        const bool s1 = t >= tiles0;
        const int64_t r0 = (int64_t)(s1 ? t - tiles0 : t) * kT;
        const int64_t nq = s1 ? nq1 : nq0;
        const int64_t qrow = (s1 ? 0 : q00) + r0;
        const int32_t rows = (int32_t)min<int64_t>(kT, nq - r0);
        const char *qb = static_cast<const char *>(s1 ? qp1 : qp0) + (qrow * rs + hoff) * kEsize;
        const char *ob = static_cast<const char *>(s1 ? dop1 : dop0) + (qrow * rs + hoff) * kEsize;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)rows * rb);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(ob, (uint32_t)rows * rb);
#pragma unroll
        for (int u = 0; u < TL::kRC; ++u) {
            qst[u] = bload8<F32>(rq, sm.rgoff[u]);
            ost[u] = bload8<F32>(ro, sm.rgoff[u]);
        }
#pragma unroll
        for (int u = 0; u < TL::kTC; ++u) {
            qtst[u][0] = bload8<F32>(rq, sm.tgoff[u]);
            qtst[u][1] = bload8<F32>(rq, sm.tgoff[u] + rb);
            otst[u][0] = bload8<F32>(ro, sm.tgoff[u]);
            otst[u][1] = bload8<F32>(ro, sm.tgoff[u] + rb);
        }
        if (tid < 2 * kT) {
            const int j = tid & (kT - 1);
            const int64_t i = qrow + j;
            if (tid < kT)
                lsv = j < rows ? (s1 ? ls1 : ls0)[i] * kLog2e : INFINITY;
            else
                lsv = j < rows ? (s1 ? dl1 : dl0)[i] : 0.0f;
        }
    };

    auto lstore = [&](int buf) {
        __bf16 *Qs = lds + buf * kStage;
        __bf16 *Os = Qs + TL::kRElems;
        __bf16 *QT = Os + TL::kRElems;
        __bf16 *OT = QT + TL::kTElems;
#pragma unroll
        for (int u = 0; u < TL::kRC; ++u) {
            *reinterpret_cast<u32x4 *>(Qs + sm.rlds[u]) = qst[u];
            *reinterpret_cast<u32x4 *>(Os + sm.rlds[u]) = ost[u];
        }
#pragma unroll
        for (int u = 0; u < TL::kTC; ++u) {
            tstore<D>(QT + sm.tlds[u], qtst[u][0], qtst[u][1]);
            tstore<D>(OT + sm.tlds[u], otst[u][0], otst[u][1]);
        }
        if (tid < 2 * kT)
            lsd[buf][tid >> 6][tid & (kT - 1)] = lsv;
    };

    f32x16 dkT[TL::kDt], dvT[TL::kDt];
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dkT[dt][r] = 0.0f;
            dvT[dt][r] = 0.0f;
        }
    const float cl = a.c_log2;

    auto tile = [&](int buf) {
        const __bf16 *Qs = lds + buf * kStage;
        const __bf16 *Os = Qs + TL::kRElems;
        const __bf16 *QT = Os + TL::kRElems;
        const __bf16 *OT = QT + TL::kTElems;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[qt][r] = 0.0f;
                dp[qt][r] = 0.0f;
            }
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(
                    Qs + (qt * 32 + l32) * TL::kRStr + ks * 16 + 8 * hh);
                s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s[qt], 0, 0, 0);
            }
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(
                    Os + (qt * 32 + l32) * TL::kRStr + ks * 16 + 8 * hh);
                dp[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[ks], dp[qt], 0, 0, 0);
            }
        // P = exp2(S cl - lse2) and dS = P o (dP - D), rows = queries of this
        // lane's registers (8i + 4hh + j), in bf16
        bf16x8 pb[2][2], db[2][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 L = *reinterpret_cast<const float4 *>(&lsd[buf][0][qt * 32 + 8 * g + 4 * hh]);
                const float4 Dv = *reinterpret_cast<const float4 *>(&lsd[buf][1][qt * 32 + 8 * g + 4 * hh]);
                const float lv[4] = {L.x, L.y, L.z, L.w};
                const float dv[4] = {Dv.x, Dv.y, Dv.z, Dv.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * g + j;
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[qt][r], cl, -lv[j]));
                    pb[qt][g >> 1][4 * (g & 1) + j] = (__bf16)p;
                    db[qt][g >> 1][4 * (g & 1) + j] = (__bf16)(p * (dp[qt][r] - dv[j]));
                }
            }
        // dv^T += dO^T P, dk^T += Q^T dS
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int dt = 0; dt < TL::kDt; ++dt) {
                    const int off = (dt * 32 + l32) * TL::kTStr + 8 * hh + 16 * (2 * qt + i2);
                    const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(OT + off);
                    const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(QT + off);
                    dvT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb[qt][i2], dvT[dt], 0, 0, 0);
                    dkT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, db[qt][i2], dkT[dt], 0, 0, 0);
                }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t + 1 < ntiles; ++t) {
        const int buf = t & 1;
        gload(t + 1);
        if (wave_active)
            tile(buf);
        lstore(buf ^ 1);
        __syncthreads();
    }
    if (!wave_active)
        return;
    tile((ntiles - 1) & 1);
    if (!key_ok)
        return;

    const float sc = a.scale;
    const int64_t obase = (k_row0 + my_k) * rs + hoff;
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = dt * 32 + 8 * i + 4 * hh;
            store4<F32>(dkptr, obase + d, dkT[dt][4 * i] * sc, dkT[dt][4 * i + 1] * sc,
                        dkT[dt][4 * i + 2] * sc, dkT[dt][4 * i + 3] * sc);
            store4<F32>(dvptr, obase + d, dvT[dt][4 * i], dvT[dt][4 * i + 1], dvT[dt][4 * i + 2],
                        dvT[dt][4 * i + 3]);
        }
}

template <int D, bool F32>
hipError_t launch_delta(const void *o, const void *dO, float *delta, int64_t rows, int32_t heads,
                        hipStream_t s)
{
    const int64_t threads = rows * heads * (D / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_delta_kernel<D, F32>), dim3((uint32_t)blocks), dim3(256), 0, s, o, dO,
                       delta, rows, heads);
    return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_t(const BwdArgs &a, const void *od, const void *og, hipStream_t s)
{
    hipError_t e = launch_delta<D, F32>(od, a.dod, const_cast<float *>(a.dl_d), a.N, a.heads, s);
    if (e != hipSuccess)
        return e;
    if (a.G > 0) {
        e = launch_delta<D, F32>(og, a.dog, const_cast<float *>(a.dl_g), a.G, a.heads, s);
        if (e != hipSuccess)
            return e;
    }
    if (a.dq_items > 0x7fffffffLL || a.kv_items > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, F32>), dim3((uint32_t)a.dq_items), dim3(kBThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32>), dim3((uint32_t)a.kv_items), dim3(kBThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int hier_attn_bwd_block_rows() { return kBRows; }

hipError_t launch_hier_attn_bwd(const BwdArgs &a, const void *od, const void *og, int head_dim,
                                int is_f32, hipStream_t s)
{
    if (head_dim == 128)
        return is_f32 ? launch_t<128, true>(a, od, og, s) : launch_t<128, false>(a, od, og, s);
    if (head_dim == 64)
        return is_f32 ? launch_t<64, true>(a, od, og, s) : launch_t<64, false>(a, od, og, s);
    return hipErrorInvalidValue;
}

}  // namespace atlas
