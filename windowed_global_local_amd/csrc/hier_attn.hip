// hier_attn.hip -- asymmetric hierarchical (window + global) attention on gfx950.
//
// "Technische Samenvatting: AtlasVid", Methodologie 2, Asymmetrische
// Hierarchische Attention, with the window attention of Methodologie 1, Fase 2:
// a detail query in cube c takes one softmax over the V keys of cube c plus all
// G global keys; a global query takes a softmax over the G global keys only.
// o = softmax(scale * q.K^T) V per head, fp32 accumulation, bf16 matrix cores.
//
// Work decomposition.  One workgroup = 8 waves (two per SIMD) = 256 query rows
// of one head: either a block of one cube window (its key list is [V window
// keys | G global keys], walked as one sequence of 64-key tiles, so one tile
// may straddle the window/global boundary) or a block of global queries (key
// list = the G global keys).  Workgroups are numbered head-major and remapped
// so that each XCD (consecutive workgroup ids round-robin over the 8 XCDs)
// walks a contiguous range of (head, window) items: the concurrent workgroups
// of one XCD then stream the same head's global K/V through that XCD's L2.
//
// Per 64-key tile, K and V (64 x D each) go from global memory straight into
// LDS with buffer loads that carry the LDS flag (no staging registers, no LDS
// store instructions), issued by waves 4-7, two buffers with one barrier per
// tile: tile t + 1 loads into one buffer while tile t is computed from the
// other.  Buffer loads
// take 32-bit offsets from a per-tile base, and rows past the end of the
// window or of the global list come back as zeros from the hardware range
// check.  Rows are stored unpadded with their 16-byte chunks XOR-swizzled, so
// that a wave's 1 KiB load block is whole rows and both read patterns below
// hit all 64 banks.  Each wave owns 32 query rows; two waves per SIMD let one
// wave's softmax overlap the other wave's matrix work.  S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16, K row fragments by 16-byte LDS reads) puts one
// query column in each lane (16 keys per lane and 32-key step), so the row
// max needs one exchange between lane halves (a permlane swap) and the row
// sum none.  P^T (bf16) feeds O^T += V^T P^T straight from the S^T registers:
// the V^T operand of each 16-key MFMA step comes from the V rows by two
// transposing 8-byte LDS reads (ds_read_b64_tr_b16), addressed so that the
// keys arrive in the S^T register order.
// Online softmax in base 2 (scale folded with log2 e) with lazy rescaling:
// the running max only moves when a tile's max exceeds it by more than 32
// (any lane of the wave), so p <= 2^32: the fp32 sums stay below 2^63 for up
// to 2^31 keys, and the final division by the running sum makes this exact.
// A rescale (64 multiplies and a branch) then fires only on large jumps, as
// at rows that meet an outlier key.  The
// running sum adds the bf16-rounded p (the values the P.V product uses) with
// v_dot2_f32_bf16.  Only the last tile of a key list can be partial; it is
// peeled off the loop, so full tiles carry no key masking.
//
// GATHER (the per-window global subset): window c's key list is [its V keys |
// the global rows listed for it].  Tiles wholly inside the window load as
// above; a tile that reaches the listed part reads its window rows from the
// window and each listed row by its index (per-lane buffer offsets; positions
// outside the list, or indices outside [0, G), read as zeros).
#include "atlas_internal.hpp"
#include "mfma_util.hpp"

#include <type_traits>

namespace atlas {

namespace {

using namespace mfma;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBQ = kWaves * 32;        // query rows per workgroup (32 per wave)
constexpr int kKT = 64;                 // keys per tile
constexpr float kLazy = 32.0f;          // log2 headroom before a rescale

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct Tile {
    static constexpr int kCh = D / 8;                           // 16-byte chunks per row
    static constexpr int kElems = kKT * D;                      // one staged 64-row tile
    static constexpr int kStage = 2 * kElems;                   // K rows | V rows
    static constexpr int kKs = D / 16;                          // k-steps of q.k
    static constexpr int kDt = D / 32;                          // 32-row tiles of O^T
    static constexpr int kRC = kKT * kCh / (kThreads / 2);      // chunks per loading thread per tile
};

// Staged rows are unpadded and XOR-swizzled: 16-byte chunk c of row r sits in
// slot c ^ swz(r), so a wave-wide 1 KiB block of whole rows is written by one
// direct-to-LDS buffer load and both the 16-byte row reads and the transposing
// 8-byte reads hit every bank.
template <int D>
__device__ constexpr int swz(int row)
{
    if constexpr (D == 128) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        const int m = (row >> 1) & 7;
        return ((m & 1) << 2) | (m >> 1);
    }
}

template <int D>
__device__ constexpr int soff(int row, int chunk)
{
    return row * D + 8 * (chunk ^ swz<D>(row));
}

template <int N>
__device__ inline void wait_vm()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// transposed MFMA A operand (row d = this lane's l32 within a 32-row block, the
// 16 keys of one group in S^T register order) from a row-major swizzled stage
__device__ __attribute__((always_inline)) bf16x8 tr_frag(const __bf16 *lo, const __bf16 *hi)
{
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lo));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(hi));
    const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
}

template <int D, bool F32, bool GATHER>
__global__ __launch_bounds__(kThreads) void hier_attn_kernel(const AttnArgs a)
{
    using TL = Tile<D>;
    constexpr int kEsize = F32 ? 4 : 2;
    // two tile buffers, declared apart so that reads of one provably do not
    // alias the direct-to-LDS loads in flight into the other
    __shared__ __attribute__((aligned(16))) __bf16 lds0[TL::kStage];
    __shared__ __attribute__((aligned(16))) __bf16 lds1[TL::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;      // MFMA row/column index of this lane
    const int hh = lane >> 5;       // MFMA k-half of this lane

    // ---- XCD-aware item: XCD x (= blockIdx % 8) walks a contiguous item range
    const int64_t item = xcd_item(blockIdx.x, gridDim.x);

    const int64_t head = item / a.items_per_head;
    const int64_t rem = item - head * a.items_per_head;
    const int64_t ndet = a.C * a.qb_win;
    const bool glob = rem >= ndet;
    const int64_t rs = (int64_t)a.heads * D;         // token row stride (elements)
    const uint32_t rb = (uint32_t)(rs * kEsize);     // token row stride (bytes)
    const int64_t hoff = head * D;

    int64_t q_row0, n_q, kw_row0;
    int32_t n_win;
    int32_t n_glob = (int32_t)a.G;   // global keys of this item's list
    int32_t g_first = 0;            // GATHER: position of that list in a.gidx
    const void *qptr;
    void *optr;
    if (!glob) {
        const int64_t c = rem / a.qb_win;
        if constexpr (GATHER) {
            // window c's listed global keys, clamped to the index array
            const int32_t g0 = min(max(a.goff[c], 0), a.n_gidx);
            const int32_t g1 = min(max(a.goff[c + 1], g0), a.n_gidx);
            g_first = g0;
            n_glob = g1 - g0;
        }
        const int64_t qb = rem - c * a.qb_win;
        q_row0 = c * a.V + qb * kBQ;
        n_q = min<int64_t>(kBQ, a.V - qb * kBQ);
        n_win = (int32_t)a.V;
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
    const int32_t nkeys = n_win + n_glob;
    const int ntiles = (nkeys + kKT - 1) / kKT;

    // ---- Q fragments: B operand of S^T = K Q^T (column = query l32, k-half hh)
    const int my_q = wave * 32 + l32;
    const bool wave_active = wave * 32 < n_q;
    const bool row_ok = my_q < n_q;
    bf16x8 qf[TL::kKs];
#pragma unroll
    for (int ks = 0; ks < TL::kKs; ++ks)
        qf[ks] = row_ok ? gload8<F32>(qptr, (q_row0 + my_q) * rs + hoff + ks * 16 + 8 * hh) : zero8();

    // ---- per-lane LDS offsets: K row fragments, transposed V fragments
    int rowo[TL::kKs];
#pragma unroll
    for (int ks = 0; ks < TL::kKs; ++ks)
        rowo[ks] = soff<D>(l32, 2 * ks + hh);      // swz(l32 + 32) == swz(l32)
    int trlo[TL::kDt], trhi[TL::kDt];
    {
        const int g = lane >> 4, i = lane & 15;
        const int r = 4 * (g >> 1) + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < TL::kDt; ++dt) {
            const int col = dt * 32 + 16 * (g & 1) + 4 * (i & 3);
            trlo[dt] = soff<D>(r, col >> 3) + (col & 7);
            trhi[dt] = soff<D>(r + 8, col >> 3) + (col & 7);
        }
    }

    // ---- staging map: LDS slot e (16 bytes) of a tile holds chunk p ^ swz(r) of row r
    uint32_t sgoff[TL::kRC];
    int srow[TL::kRC], sslot[TL::kRC];
#pragma unroll
    for (int u = 0; u < TL::kRC; ++u) {
        const int e = (tid & (kThreads / 2 - 1)) + (kThreads / 2) * u;
        const int r = e / TL::kCh, p = e % TL::kCh;
        srow[u] = r;
        sgoff[u] = (uint32_t)r * rb + (uint32_t)((p ^ swz<D>(r)) * 8 * kEsize);
        sslot[u] = F32 ? e * 8 : ((wave & (kWaves / 2 - 1)) * 64 + (kThreads / 2) * u) * 8;
    }
    // waves 4-7 (the second wave of each SIMD) stage the tiles; measured a
    // little faster than staging by all eight waves or by waves 0-3
    const bool loader = wave >= kWaves / 2;
    auto put = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, __bf16 *stage, int u) __attribute__((always_inline)) {
        if constexpr (F32) {
            *reinterpret_cast<u32x4 *>(stage + sslot[u]) = bload8<true>(r, off);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(stage + sslot[u]), 16, (int)off, 0, 0, 0);
        }
    };

    const char *kwin = static_cast<const char *>(a.kd) + (kw_row0 * rs + hoff) * kEsize;
    const char *vwin = static_cast<const char *>(a.vd) + (kw_row0 * rs + hoff) * kEsize;
    const char *kglb = static_cast<const char *>(a.kg) + hoff * kEsize;
    const char *vglb = static_cast<const char *>(a.vg) + hoff * kEsize;

    // key tile t -> LDS stage Ks (window keys, global keys, or the one tile
    // that straddles the two lists: each row from its own list; rows past a
    // list read as zeros)
    auto stage = [&](int t, __bf16 *Ks) __attribute__((always_inline)) {
        __bf16 *Vs = Ks + TL::kElems;
        const int32_t k0 = t * kKT;
        if constexpr (GATHER) {
            if (!glob && k0 + kKT > n_win) {
                const int32_t r0 = max(0, n_win - k0);
                const int32_t kb0 = min(k0, n_win);
                const __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)kb0 * rb, (uint32_t)r0 * rb);
                const __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)kb0 * rb, (uint32_t)r0 * rb);
                const __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)a.G * rb);
                const __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)a.G * rb);
                const int32_t p0 = k0 - n_win;   // list position of tile row 0
#pragma unroll
                for (int u = 0; u < TL::kRC; ++u) {
                    const int32_t row = srow[u];
                    if (row < r0) {
                        put(rkw, sgoff[u], Ks, u);
                        put(rvw, sgoff[u], Vs, u);
                    } else {
                        const int32_t pos = p0 + row;
                        const uint32_t cho = sgoff[u] - (uint32_t)row * rb;
                        uint32_t off = 0x80000000u;
                        if (pos < n_glob) {
                            const int32_t idx = a.gidx[g_first + pos];
                            if ((uint32_t)idx < (uint32_t)a.G)
                                off = (uint32_t)idx * rb + cho;
                        }
                        put(rkg, off, Ks, u);
                        put(rvg, off, Vs, u);
                    }
                }
                return;
            }
        }
        if (k0 + kKT <= n_win || k0 >= n_win) {
            const bool in_win = k0 < n_win;
            const int32_t g0 = k0 - n_win;
            const int32_t rows = in_win ? kKT : max(0, min(kKT, (int32_t)a.G - g0));
            const char *kb = in_win ? kwin + (int64_t)k0 * rb : kglb + (int64_t)g0 * rb;
            const char *vb = in_win ? vwin + (int64_t)k0 * rb : vglb + (int64_t)g0 * rb;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)rows * rb);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)rows * rb);
#pragma unroll
            for (int u = 0; u < TL::kRC; ++u) {
                put(rk, sgoff[u], Ks, u);
                put(rv, sgoff[u], Vs, u);
            }
        } else {
            const int32_t r0 = n_win - k0;
            const int32_t ng = max(0, min(kKT - r0, (int32_t)a.G));
            const __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            const __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            const __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)ng * rb);
            const __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)ng * rb);
            const uint32_t gs = (uint32_t)r0 * rb;
#pragma unroll
            for (int u = 0; u < TL::kRC; ++u) {
                if (srow[u] < r0) {
                    put(rkw, sgoff[u], Ks, u);
                    put(rvw, sgoff[u], Vs, u);
                } else {
                    put(rkg, sgoff[u] - gs, Ks, u);
                    put(rvg, sgoff[u] - gs, Vs, u);
                }
            }
        }
    };

    f32x16 o[TL::kDt];
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[dt][r] = 0.0f;
    float m_run = -INFINITY;   // running max, log2 domain
    float l_run = 0.0f;        // this lane's half of the running sum
    const float cl = a.c_log2;
    bf16x2 ones;
    ones[0] = (__bf16)1.0f;
    ones[1] = (__bf16)1.0f;

    // one 64-key tile of compute on LDS stage `buf`; kMasked only for the final
    // tile (keys past the end of the list get -inf logits)
    auto tile = [&](const __bf16 *Ks, int t, auto masked_c) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked_c)::value;
        const __bf16 *Vs = Ks + TL::kElems;

        // S^T = K Q^T for the two 32-key halves of the tile.  All K fragments
        // of the tile are requested before the first MFMA, so LDS latency
        // overlaps the MFMA chain instead of stalling each step.
        bf16x8 ka[2][TL::kKs];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < TL::kKs; ++ks)
                ka[kt][ks] = *reinterpret_cast<const bf16x8 *>(Ks + kt * 32 * D + rowo[ks]);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kt][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kt][ks], qf[ks], s[kt], 0, 0, 0);
        // the V^T fragments of P.V are requested now, behind the S^T MFMAs, so
        // they arrive during the softmax
        bf16x8 va[TL::kDt][4];
#pragma unroll
        for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                va[dt][j] = tr_frag(Vs + j * 16 * D + trlo[dt], Vs + j * 16 * D + trhi[dt]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kMasked) {
            const int32_t kbase = t * kKT;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (kbase + key >= nkeys)
                        s[kt][r] = -INFINITY;
                }
        }

        // online softmax over the tile's 64 keys (32 here, 32 in lane ^ 32)
        float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = (kt == 0 ? 1 : 1); r < 16; ++r)
                mx = fmaxf(mx, s[kt][r]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
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
        const float mneg = -m_run;
        bf16x8 p[2][2];
        float ls = l_run;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    p[kt][i2][m] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kt][8 * i2 + m], cl, mneg));
#pragma unroll
                for (int m = 0; m < 8; m += 2) {
                    bf16x2 pp;
                    pp[0] = p[kt][i2][m];
                    pp[1] = p[kt][i2][m + 1];
                    ls = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls, false);
                }
            }
        l_run = ls;

        // O^T += V^T P^T: va[dt][2 kt + i2] holds the keys [kt*32 + i2*16, +16)
        // in the S^T register order that p[kt][i2] uses
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int dt = 0; dt < TL::kDt; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][2 * kt + i2], p[kt][i2], o[dt],
                                                                    0, 0, 0);
    };

    // tile t is computed from one buffer while tile t + 1 loads into the
    // other; each step ends with the wait for that load and a barrier, after
    // which no wave reads tile t's buffer again.  Unrolled by two so that the
    // two buffers stay distinct objects to the compiler.
    if (loader)
        stage(0, lds0);
    wait_vm<0>();
    __syncthreads();
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
        if (loader)
            stage(t + 1, lds1);
        if (wave_active)
            tile(lds0, t, std::false_type{});
        wait_vm<0>();
        __syncthreads();
        if (loader)
            stage(t + 2, lds0);
        if (wave_active)
            tile(lds1, t + 1, std::false_type{});
        wait_vm<0>();
        __syncthreads();
    }
    if (t + 1 < ntiles) {
        if (loader)
            stage(t + 1, lds1);
        if (wave_active)
            tile(lds0, t, std::false_type{});
        wait_vm<0>();
        __syncthreads();
        if (!wave_active)
            return;
        tile(lds1, t + 1, std::true_type{});
    } else {
        if (!wave_active)
            return;
        tile(lds0, t, std::true_type{});
    }

    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / lt;
    if (!row_ok)
        return;
    // log-sum-exp of the scaled logits (natural log), for the backward pass
    float *lse = glob ? a.lse_g : a.lse_d;
    if (lse != nullptr && hh == 0)
        lse[head * (glob ? a.G : a.C * a.V) + q_row0 + my_q] = (m_run + log2f(lt)) * 0.69314718055994531f;
    // output row: the cube-order query row, or (raster epilogue) the raster
    // token it came from
    int64_t orow = q_row0 + my_q;
    if (!glob && a.raster) {
        const int64_t V = (int64_t)a.ct * a.ch * a.cw;
        const int64_t c = orow / V;
        const int32_t o = (int32_t)(orow - c * V);
        const int32_t cubes_per_frame = a.nH * a.nW;
        const int32_t ca = (int32_t)(c / cubes_per_frame);
        const int32_t crem = (int32_t)(c - (int64_t)ca * cubes_per_frame);
        const int32_t cb = crem / a.nW, ce = crem - cb * a.nW;
        const int32_t dt = o / (a.ch * a.cw);
        const int32_t orem = o - dt * (a.ch * a.cw);
        const int32_t dh = orem / a.cw, dw = orem - dh * a.cw;
        orow = ((int64_t)(ca * a.ct + dt) * a.H + (cb * a.ch + dh)) * a.W + (ce * a.cw + dw);
    }
    const int64_t obase = orow * rs + hoff;
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
    if (a.goff != nullptr)
        hipLaunchKernelGGL((hier_attn_kernel<D, F32, true>), dim3((uint32_t)a.items), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((hier_attn_kernel<D, F32, false>), dim3((uint32_t)a.items), dim3(kThreads), 0, s, a);
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
