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
// Per 64-key tile, K (64 x D) and V transposed (D x 64) are staged in LDS,
// double buffered through registers with one barrier per tile.  Staging uses
// buffer loads: 32-bit offsets from a per-tile base, and rows past the end of
// the window or of the global list come back as zeros from the hardware range
// check.  Each wave owns 32 query rows; two waves per SIMD let one wave's
// softmax overlap the other wave's matrix work.  S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16) puts one query column in each lane (16 keys per
// lane and 32-key step), so the row max needs one exchange between lane
// halves and the row sum none.  P^T (bf16) feeds O^T += V^T P^T straight from
// the S^T registers: inside each 16-key MFMA step the key order is permuted to
// match the S^T register layout, and V^T is stored in LDS in that permuted
// order, so every MFMA operand is one 16-byte LDS read.  The LDS issue rate,
// not its byte rate, bounds this kernel (about one LDS instruction per 5.4
// clocks per CU at any width), so the layouts favour 16-byte accesses: K rows
// padded to D+8 elements and V^T rows to 72 make 16 consecutive rows hit 16
// distinct 4-bank groups of the 64 banks, and the transposing V^T stores pair
// two keys per 4-byte store, spread over lanes so that a wave's 64 stores hit
// 64 distinct banks.
// Online softmax in base 2 (scale folded with log2 e) with lazy rescaling:
// the running max only moves when a tile's max exceeds it by more than 8, so
// p <= 256; the final division by the running sum makes this exact.  The
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
constexpr float kLazy = 8.0f;           // log2 headroom before a rescale

template <int D>
struct Tile {
    // K rows padded by 16 bytes (68 dwords for D = 128): 16 consecutive key
    // rows read at one column hit 16 distinct 4-bank groups.  V^T rows hold the
    // 64 keys of a tile padded to 72 elements (36 dwords; 36*d mod 64 is a
    // bijection onto the multiples of 4 for 16 consecutive d).
    static constexpr int kKStr = D + 8;
    static constexpr int kVStr = kKT + 8;
    static constexpr int kKElems = kKT * kKStr;
    static constexpr int kVElems = D * kVStr;
    static constexpr int kStage = kKElems + kVElems;
    static constexpr int kKs = D / 16;                          // k-steps of q.k
    static constexpr int kDt = D / 32;                          // 32-row tiles of O^T
    static constexpr int kChunks = kKT * (D / 8) / kThreads;    // K (and V) chunks / thread
};

template <int D, bool F32, bool GATHER>
__global__ __launch_bounds__(kThreads) void hier_attn_kernel(const AttnArgs a)
{
    using TL = Tile<D>;
    constexpr int kEsize = F32 ? 4 : 2;
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * TL::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    // ---- staging maps
    // K: chunk e = tid + kThreads*u -> key row e / (D/8), 8-element column e % (D/8).
    uint32_t k_goff[TL::kChunks];
    int k_lds[TL::kChunks];
#pragma unroll
    for (int u = 0; u < TL::kChunks; ++u) {
        const int e = tid + kThreads * u;
        const int row = e / (D / 8), ch = e % (D / 8);
        k_goff[u] = (uint32_t)row * rb + (uint32_t)(ch * 8 * kEsize);
        k_lds[u] = row * TL::kKStr + ch * 8;
    }
    // V: lane -> key pair pp = lane % 32 (keys 2pp, 2pp+1) and d-chunk dc (d =
    // 8dc .. 8dc+7).  Its 8 four-byte stores go to V^T rows 8dc+m at the pair's
    // permuted position: a key at offset 8i+4h+j of its 16-key group sits at
    // 8h+4i+j (the S^T register order).  Across a wave the 32 pairs times two
    // d-chunks of opposite parity make the stores hit 64 distinct banks.
    const bool v_on = (D == 128) || wave < 4;
    const int v_pp = lane & 31;
    const int v_dc = 2 * wave + (lane >> 5);
    const int v_key0 = 2 * v_pp;
    const int v_pos0 = tperm(v_key0);
    const uint32_t v_goff = (uint32_t)v_key0 * rb + (uint32_t)(v_dc * 8 * kEsize);
    const int v_lds = (8 * v_dc) * TL::kVStr + v_pos0;

    const char *kwin = static_cast<const char *>(a.kd) + (kw_row0 * rs + hoff) * kEsize;
    const char *vwin = static_cast<const char *>(a.vd) + (kw_row0 * rs + hoff) * kEsize;
    const char *kglb = static_cast<const char *>(a.kg) + hoff * kEsize;
    const char *vglb = static_cast<const char *>(a.vg) + hoff * kEsize;

    u32x4 kst[TL::kChunks], vst[2];

    // GATHER: byte offset of chunk `cho` of global-list position p, or an
    // offset past any buffer (zero fill) when p is outside the list or its
    // index outside [0, G)
    constexpr uint32_t kNoRow = 0x80000000u;
    auto grow = [&](int32_t p, uint32_t cho) -> uint32_t {
        if (p < 0 || p >= n_glob)
            return kNoRow;
        const int32_t idx = a.gidx[g_first + p];
        return (uint32_t)idx < (uint32_t)a.G ? (uint32_t)idx * rb + cho : kNoRow;
    };

    // global -> registers for tile t.  A tile lies in the window block, in the
    // global list, or straddles the boundary (once per item); the source is
    // selected per tile, uniformly, and only the straddling tile merges two.
    auto gload = [&](int t) {
        const int32_t k0 = t * kKT;
        if constexpr (GATHER) {
            if (!glob && k0 + kKT > n_win) {
                // a tile with listed global keys: rows below n_win from the
                // window, the others gathered by index (each read is zero
                // outside its own source)
                const int32_t r0 = max(0, n_win - k0);
                const __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)min(k0, n_win) * rb, (uint32_t)r0 * rb);
                const __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)min(k0, n_win) * rb, (uint32_t)r0 * rb);
                const __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)a.G * rb);
                const __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)a.G * rb);
                const int32_t p0 = k0 - n_win;   // list position of tile row 0
#pragma unroll
                for (int u = 0; u < TL::kChunks; ++u) {
                    const int e = tid + kThreads * u;
                    const int row = e / (D / 8);
                    const uint32_t cho = (uint32_t)((e % (D / 8)) * 8 * kEsize);
                    kst[u] = bload8<F32>(rkw, k_goff[u]) | bload8<F32>(rkg, grow(p0 + row, cho));
                }
                if (v_on) {
                    const uint32_t cho = (uint32_t)(v_dc * 8 * kEsize);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        vst[j] = bload8<F32>(rvw, v_goff + (uint32_t)j * rb) |
                                 bload8<F32>(rvg, grow(p0 + v_key0 + j, cho));
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
            __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)rows * rb);
            __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)rows * rb);
#pragma unroll
            for (int u = 0; u < TL::kChunks; ++u)
                kst[u] = bload8<F32>(rk, k_goff[u]);
            if (v_on) {
                vst[0] = bload8<F32>(rv, v_goff);
                vst[1] = bload8<F32>(rv, v_goff + rb);
            }
        } else {
            // tile rows [0, r0) are window keys k0.., rows [r0, 64) global keys 0..
            const int32_t r0 = n_win - k0;
            const int32_t ng = max(0, min(kKT - r0, (int32_t)a.G));
            __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)ng * rb);
            __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)ng * rb);
            // rows < r0 give offsets that wrap to huge unsigned values in the global
            // buffer (out of range -> 0); rows >= r0 are past the window buffer
            const uint32_t gshift = (uint32_t)r0 * rb;
#pragma unroll
            for (int u = 0; u < TL::kChunks; ++u)
                kst[u] = bload8<F32>(rkw, k_goff[u]) | bload8<F32>(rkg, k_goff[u] - gshift);
            if (v_on) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t off = v_goff + (uint32_t)j * rb;
                    vst[j] = bload8<F32>(rvw, off) | bload8<F32>(rvg, off - gshift);
                }
            }
        }
    };

    // registers -> LDS stage `buf`
    auto lstore = [&](int buf) {
        __bf16 *Ks = lds + buf * TL::kStage;
        __bf16 *Vs = Ks + TL::kKElems;
#pragma unroll
        for (int u = 0; u < TL::kChunks; ++u)
            *reinterpret_cast<u32x4 *>(Ks + k_lds[u]) = kst[u];
        if (v_on) {
            const u32x4 x = vst[0], y = vst[1];
            __bf16 *col = Vs + v_lds;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // (key 2pp, key 2pp+1) at d = 8dc+2m and at d = 8dc+2m+1
                *reinterpret_cast<uint32_t *>(col + (2 * m) * TL::kVStr) =
                    __builtin_amdgcn_perm(y[m], x[m], 0x05040100u);
                *reinterpret_cast<uint32_t *>(col + (2 * m + 1) * TL::kVStr) =
                    __builtin_amdgcn_perm(y[m], x[m], 0x07060302u);
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
    auto tile = [&](int buf, int t, auto masked_c) {
        constexpr bool kMasked = decltype(masked_c)::value;
        const __bf16 *Ks = lds + buf * TL::kStage;
        const __bf16 *Vs = Ks + TL::kKElems;

        // S^T = K Q^T for the two 32-key halves of the tile.  All K fragments
        // of the tile are requested before the first MFMA, so LDS latency
        // overlaps the MFMA chain instead of stalling each step.
        bf16x8 ka[2][TL::kKs];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < TL::kKs; ++ks)
                ka[kt][ks] = *reinterpret_cast<const bf16x8 *>(
                    Ks + (kt * 32 + l32) * TL::kKStr + ks * 16 + 8 * hh);
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
                va[dt][j] = *reinterpret_cast<const bf16x8 *>(
                    Vs + (dt * 32 + l32) * TL::kVStr + 8 * hh + 16 * j);
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

        // O^T += V^T P^T: the V^T fragment for keys [kt*32 + i2*16, +16) in the
        // S^T register order is 8 consecutive stored positions of row d
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int dt = 0; dt < TL::kDt; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][2 * kt + i2], p[kt][i2], o[dt],
                                                                    0, 0, 0);
    };

    gload(0);
    lstore(0);
    __syncthreads();
    // all tiles but the last are full: no key masking inside the loop
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
