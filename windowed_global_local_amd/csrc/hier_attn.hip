// hier_attn.hip -- asymmetric hierarchical (window + global) attention on gfx950.
//
// "Technische Samenvatting: AtlasVid", Methodologie 2, Asymmetrische
// Hierarchische Attention, with the window attention of Methodologie 1, Fase 2:
// a detail query in cube c takes one softmax over the V keys of cube c plus all
// G global keys; a global query takes a softmax over the G global keys only.
// o = softmax(scale * q.K^T) V per head, fp32 accumulation, bf16 matrix cores.
//
// Work decomposition.  One workgroup = 8 waves = 256 query rows of one head:
// either a block of one cube window (the key list is [V window keys | G global
// keys], walked as one sequence of 64-key tiles, so a tile may straddle the
// window/global boundary) or a block of global queries (key list = G global
// keys).  Workgroups are numbered head-major and remapped so that each XCD
// (consecutive workgroup ids round-robin over the 8 XCDs) walks a contiguous
// range of (head, window) items: concurrent workgroups of one XCD then share
// the head's global K/V in that XCD's L2.
//
// Per 64-key tile, K (64 x D) and V (transposed, D x 64) are staged in LDS
// (double buffered through registers, one barrier per tile).  Each wave owns
// 32 query rows and computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so one
// lane holds 16 keys of ONE query column: the row max needs one cross-half
// exchange and the row sum none.  P^T (bf16) feeds O^T += V^T P^T directly
// from the S^T registers: the key order inside each 16-key MFMA step is
// permuted to match the S^T register layout, and V^T is stored in LDS in that
// same permuted order.  Online softmax in base 2 (scale folded with log2 e),
// with lazy rescaling: the running max is only raised when a tile's max
// exceeds it by more than 8 (so p <= 256), which is exact after the final
// division by the running sum.
#include "atlas_internal.hpp"

#include <type_traits>

namespace atlas {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;                 // query rows per wave
constexpr int kBQ = kWaves * kQW;       // query rows per workgroup
constexpr int kKT = 64;                 // keys per tile
constexpr int kVStr = kKT + 8;          // V^T LDS row stride (elements)
constexpr float kLazy = 8.0f;           // log2 headroom before a rescale

template <int D>
struct Tile {
    static constexpr int kKStr = D + 8;                    // K LDS row stride
    static constexpr int kKElems = kKT * kKStr;
    static constexpr int kVElems = D * kVStr;
    static constexpr int kStage = kKElems + kVElems;
    static constexpr int kKs = D / 16;                     // k-steps of q.k
    static constexpr int kDt = D / 32;                     // 32-row tiles of O^T
    static constexpr int kKChunks = kKT * (D / 8) / kThreads;   // K chunks per thread
};

template <bool F32>
__device__ inline bf16x8 load8(const void *base, int64_t off)
{
    if constexpr (F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
        const float4 x = p[0], y = p[1];
        bf16x8 r;
        r[0] = (__bf16)x.x; r[1] = (__bf16)x.y; r[2] = (__bf16)x.z; r[3] = (__bf16)x.w;
        r[4] = (__bf16)y.x; r[5] = (__bf16)y.y; r[6] = (__bf16)y.z; r[7] = (__bf16)y.w;
        return r;
    } else {
        return *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(base) + off);
    }
}

__device__ inline bf16x8 zero8()
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = (__bf16)0.0f;
    return r;
}

template <int D, bool F32>
__global__ __launch_bounds__(kThreads) void hier_attn_kernel(const AttnArgs a)
{
    using TL = Tile<D>;
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * TL::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;      // MFMA row/column index of this lane
    const int hh = lane >> 5;       // MFMA k-half of this lane

    // ---- XCD-aware item: XCD x (= blockIdx % 8) walks a contiguous item range
    const uint32_t nb = gridDim.x, bid = blockIdx.x;
    const uint32_t xcd = bid & 7u, jx = bid >> 3, q8 = nb >> 3, r8 = nb & 7u;
    const int64_t item = (xcd < r8) ? (int64_t)xcd * (q8 + 1) + jx
                                    : (int64_t)r8 * (q8 + 1) + (int64_t)(xcd - r8) * q8 + jx;

    const int64_t head = item / a.items_per_head;
    const int64_t rem = item - head * a.items_per_head;
    const int64_t ndet = a.C * a.qb_win;
    const bool glob = rem >= ndet;
    const int64_t rs = (int64_t)a.heads * D;        // token row stride (elements)

    int64_t q_row0, n_q, n_win, kw_row0;
    const void *qptr;
    void *optr;
    if (!glob) {
        const int64_t c = rem / a.qb_win;
        const int64_t qb = rem - c * a.qb_win;
        q_row0 = c * a.V + qb * kBQ;
        n_q = min<int64_t>(kBQ, a.V - qb * kBQ);
        n_win = a.V;
        kw_row0 = c * a.V;
        qptr = a.qd;
        optr = a.od;
    } else {
        const int64_t gb = rem - ndet;
        q_row0 = gb * kBQ;
        n_q = min<int64_t>(kBQ, a.G - gb * kBQ);
        n_win = 0;
        kw_row0 = 0;
        qptr = a.qg;
        optr = a.og;
    }
    const int64_t nkeys = n_win + a.G;
    const int ntiles = (int)((nkeys + kKT - 1) / kKT);
    const int64_t hoff = head * D;

    // ---- Q fragment: B operand of S^T = K Q^T (column = query l32, k-half hh)
    const int my_q = wave * kQW + l32;
    const bool wave_active = wave * kQW < n_q;
    const bool row_ok = my_q < n_q;
    bf16x8 qf[TL::kKs];
#pragma unroll
    for (int ks = 0; ks < TL::kKs; ++ks)
        qf[ks] = row_ok ? load8<F32>(qptr, (q_row0 + my_q) * rs + hoff + ks * 16 + 8 * hh) : zero8();

    // ---- staging maps
    // K: chunk e = tid + kThreads*u -> key row e / (D/8), 8-element column chunk e % (D/8)
    // V: (group gi, pair kq, d-chunk dch) -> keys key0, key0+1 and d = 8*dch .. 8*dch+7,
    //    written transposed with a bank-spreading XOR on the 16-byte chunk index.
    bool v_on;
    int gi, kq, dch;
    if constexpr (D == 128) {
        v_on = true;
        gi = wave;
        dch = (lane & 7) + 8 * (lane >> 5);
        kq = (lane >> 3) & 3;
    } else {
        v_on = wave < 4;
        gi = 2 * wave + (lane >> 5);
        dch = lane & 7;
        kq = (lane >> 3) & 3;
    }
    const int key0 = 16 * (gi >> 1) + 4 * (gi & 1) + 8 * (kq >> 1) + 2 * (kq & 1);
    const int pos0 = 16 * (gi >> 1) + 8 * (gi & 1) + 4 * (kq >> 1) + 2 * (kq & 1);
    const int vt_off = (((pos0 >> 3) ^ (dch & 7)) << 3) + (pos0 & 7);

    auto key_off = [&](int64_t kk) -> int64_t {   // element offset of key kk, head `head`
        return kk < n_win ? (kw_row0 + kk) * rs + hoff : (kk - n_win) * rs + hoff;
    };
    auto key_base = [&](int64_t kk, bool v) -> const void * {
        return kk < n_win ? (v ? a.vd : a.kd) : (v ? a.vg : a.kg);
    };

    bf16x8 kst[TL::kKChunks];
    bf16x8 vst[2];

    auto gload = [&](int t) {
        const int64_t k0 = (int64_t)t * kKT;
#pragma unroll
        for (int u = 0; u < TL::kKChunks; ++u) {
            const int e = tid + kThreads * u;
            const int row = e / (D / 8), ch = e % (D / 8);
            const int64_t kk = k0 + row;
            kst[u] = kk < nkeys ? load8<F32>(key_base(kk, false), key_off(kk) + ch * 8) : zero8();
        }
        if (v_on) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t kk = k0 + key0 + u;
                vst[u] = kk < nkeys ? load8<F32>(key_base(kk, true), key_off(kk) + dch * 8) : zero8();
            }
        }
    };

    auto lstore = [&](int buf) {
        __bf16 *Ks = lds + buf * TL::kStage;
        __bf16 *Vt = Ks + TL::kKElems;
#pragma unroll
        for (int u = 0; u < TL::kKChunks; ++u) {
            const int e = tid + kThreads * u;
            const int row = e / (D / 8), ch = e % (D / 8);
            *reinterpret_cast<bf16x8 *>(Ks + row * TL::kKStr + ch * 8) = kst[u];
        }
        if (v_on) {
            const uint4 x = __builtin_bit_cast(uint4, vst[0]);
            const uint4 y = __builtin_bit_cast(uint4, vst[1]);
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
            const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
            __bf16 *col = Vt + (8 * dch) * kVStr + vt_off;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t lo = (xs[m] & 0xffffu) | (ys[m] << 16);          // d = 8dch+2m
                const uint32_t hi = (xs[m] >> 16) | (ys[m] & 0xffff0000u);      // d = 8dch+2m+1
                *reinterpret_cast<uint32_t *>(col + (2 * m) * kVStr) = lo;
                *reinterpret_cast<uint32_t *>(col + (2 * m + 1) * kVStr) = hi;
            }
        }
    };

    f32x16 o[TL::kDt];
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[dt][r] = 0.0f;
    float m_run = -INFINITY;     // running max, log2 domain
    float l_run = 0.0f;          // this lane's half of the running sum
    const float cl = a.c_log2;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles)
            gload(t + 1);

        if (wave_active) {
            const __bf16 *Ks = lds + buf * TL::kStage;
            const __bf16 *Vt = Ks + TL::kKElems;

            // S^T = K Q^T : two 32-key subtiles
            f32x16 s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[kt][r] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < TL::kKs; ++ks) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                        Ks + (kt * 32 + l32) * TL::kKStr + ks * 16 + 8 * hh);
                    s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[kt], 0, 0, 0);
                }
            }

            // keys past the end of the list (last tile only)
            const int64_t kbase = (int64_t)t * kKT;
            if (kbase + kKT > nkeys) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (kbase + key >= nkeys)
                            s[kt][r] = -INFINITY;
                    }
            }

            // tile max over this query's 64 keys (32 here, 32 in lane ^ 32)
            float mx = s[0][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, s[kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = mx * cl;
            if (__any(mnew > m_run + kLazy)) {
                const float m2 = fmaxf(m_run, mnew);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m2);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[dt][r] *= alpha;
                m_run = m2;
            }

            // P^T in bf16, in the S^T register order
            bf16x8 p[2][2];
            float ls = 0.0f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const float e = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * i2 + m], cl, -m_run));
                        ls += e;
                        p[kt][i2][m] = (__bf16)e;
                    }
            l_run += ls;

            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < TL::kDt; ++dt) {
                const int d = dt * 32 + l32;
                const __bf16 *vrow = Vt + d * kVStr;
                const int sw = (d >> 3) & 7;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i2 = 0; i2 < 2; ++i2) {
                        const int chunk = (4 * kt + 2 * i2 + hh) ^ sw;
                        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vrow + chunk * 8);
                        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kt][i2], o[dt], 0, 0, 0);
                    }
            }
        }

        if (t + 1 < ntiles)
            lstore(buf ^ 1);
        __syncthreads();
    }

    if (!wave_active)
        return;
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / lt;
    if (!row_ok)
        return;
    const int64_t obase = (q_row0 + my_q) * rs + hoff;
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = dt * 32 + 8 * i + 4 * hh;
            const float v0 = o[dt][4 * i + 0] * inv, v1 = o[dt][4 * i + 1] * inv;
            const float v2 = o[dt][4 * i + 2] * inv, v3 = o[dt][4 * i + 3] * inv;
            if constexpr (F32) {
                *reinterpret_cast<float4 *>(static_cast<float *>(optr) + obase + d) =
                    make_float4(v0, v1, v2, v3);
            } else {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 w;
                w[0] = (__bf16)v0; w[1] = (__bf16)v1; w[2] = (__bf16)v2; w[3] = (__bf16)v3;
                *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(optr) + obase + d) = w;
            }
        }
}

template <int D, bool F32>
hipError_t launch_t(const AttnArgs &a, hipStream_t s)
{
    if (a.items <= 0)
        return hipSuccess;
    if (a.items > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((hier_attn_kernel<D, F32>), dim3((uint32_t)a.items), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int hier_attn_block_rows() { return kBQ; }

hipError_t launch_hier_attn(const AttnArgs &a, int head_dim, int is_f32, hipStream_t s)
{
    if (head_dim == 128)
        return is_f32 ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
    if (head_dim == 64)
        return is_f32 ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace atlas
