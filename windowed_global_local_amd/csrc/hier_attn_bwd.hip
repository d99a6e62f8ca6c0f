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
// Cube mask (every detail query sees all G global keys): three kernels, no
// atomics, every gradient row written once, so the results are bit-for-bit
// reproducible:
//   delta  D_i = dO_i.o_i per (query, head), fp32, into the caller's workspace;
//   dq     one workgroup per 256 queries of one head (a window block or a
//          global block), streaming that query's key list in 64-key tiles, as
//          the forward does: S^T = K Q^T and dP^T = V dO^T put one query in each
//          lane, dS^T = P^T o (dP^T - D) is formed in registers and
//          dq^T += K^T dS^T (K^T read from the K rows by transposing LDS
//          loads, in the permuted key order that matches the S^T registers);
//   dk/dv  one workgroup per 128 keys of one head, streaming every query that
//          sees those keys in 64-query tiles (a window's keys: the window's V
//          queries; a global key block: all N detail and G global queries):
//          S = Q K^T and dP = dO V^T put one key in each lane,
//          dv^T += dO^T P and dk^T += Q^T dS with dO^T and Q^T read by
//          transposing LDS loads.  K and V of the block stay in registers.
// Tiles go from global memory straight into LDS (buffer loads with the LDS
// flag: no staging registers), two buffers, one tile ahead; rows are stored
// unpadded with an XOR swizzle of their 16-byte chunks.  dq runs 8 waves of
// 32 queries, two per SIMD (accumulator, q and dO of its queries and one
// half-tile of operands fit 256 registers), so that each wave's exp / dS work
// and LDS waits overlap the other's MFMAs.  dk/dv runs one wave per SIMD: its
// accumulators (128 fp32 per lane) and K, V of its keys (64) alone take most
// of 256 registers, so it software-pipelines each tile inside the wave.
// Splitting dq from dk/dv recomputes S and dP once more, but a key-major pass
// that also produced dq would have to add every global key block's partial
// dq into every query row (hundreds of partial sums per row), and a
// query-major pass the same for dk/dv of the global keys.
//
// Per-window global subset (SUBSET / GATHER instances): a global key may be
// listed by many windows, so its dk/dv share from detail queries is summed by
// two more kernels: bwd_zero_kernel clears fp32 accumulators in the caller's
// workspace and bwd_listed_kernel (one workgroup per head and window) adds
// each window's contribution to them with fp32 atomic adds; the global key
// blocks of the dk/dv kernel then stream only the G global queries and add
// the accumulators.  The order of those atomic adds varies from run to run,
// so dk_g and dv_g of the subset backward may differ in the last bits
// between runs (graph replays included); every other output is
// deterministic.
//
// All rows outside a list read as zeros (buffer range checks, lse and D
// included): a query past the end of a tile has zero q and dO, so it adds
// nothing to dk or dv; a key past the end of a list has zero K and V, so it
// adds nothing to dq (its P = exp(-lse) is clamped to 1 like every P, so it
// stays finite however negative lse is); keys past the end of a key block
// only fill accumulator columns that are never stored.  Matrix products run on v_mfma_f32_32x32x16_bf16 with bf16
// operands (P and dS rounded to bf16) and fp32 accumulation.
#include "atlas_internal.hpp"
#include "mfma_util.hpp"


namespace atlas {

namespace {

using namespace mfma;

constexpr int kBW = 4;                  // dk/dv: waves per workgroup (one per SIMD)
constexpr int kBThreads = kBW * 64;
constexpr int kBRows = kBW * 32;        // keys per dk/dv workgroup
constexpr int kQW = 8;                  // dq: waves per workgroup (two per SIMD)
constexpr int kQThreads = kQW * 64;
constexpr int kQRows = kQW * 32;        // queries per dq workgroup
constexpr int kT = 64;                  // rows per streamed tile
constexpr float kLog2e = 1.4426950408889634f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct BTile {
    static constexpr int kCh = D / 8;                   // 16-byte chunks per bf16 row
    static constexpr int kElems = kT * D;               // one staged 64-row tile (unpadded)
    static constexpr int kKs = D / 16;                  // k-steps over head_dim
    static constexpr int kDt = D / 32;                  // 32-row tiles of a D x 32 result
};

// Staged rows are unpadded and XOR-swizzled: 16-byte chunk c of row r sits in
// slot c ^ swz(r), so that a wave-wide 1 KiB block of whole rows can be written
// by one direct-to-LDS buffer load (lane i -> bytes 16i .. 16i+15) and both
// read patterns run without bank conflicts:
//  - 16-byte row reads: 16 consecutive rows at one chunk hit 16 distinct
//    4-bank groups (swz is a bijection on 16 rows; for D = 64 two rows share
//    the 64 banks, so swz is one on the 8 row pairs);
//  - transposing 8-byte reads: 32 lanes read 4 consecutive rows x 4 chunks of
//    one aligned 4-chunk block, which must cover all 64 banks, so the 4 rows
//    (D = 128; the 2 row pairs for D = 64) must differ in the upper swizzle
//    bits.  D = 128: swap the two 2-bit fields of r mod 16; D = 64: rotate
//    the 3 bits of the row-pair index.
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

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Pointers into LDS are handed to the LDS-only instructions through plain
// address-space casts (generic -> local), which keep the pointer's origin, so
// alias analysis still tells the two tile buffers apart.
typedef __attribute__((address_space(3))) void lds_void;

// 64 fp32 values (4 bytes per lane) from a buffer straight into LDS at dst
__device__ __attribute__((always_inline)) void dma4(__amdgpu_buffer_rsrc_t r, float *dst, int lane)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst), 4, lane * 4, 0, 0, 0);
}

// Transposed MFMA A operand from a row-major swizzled stage: output row d (this
// lane's l32 within a 32-row block) and the 16 rows of one group in S register
// order (rows 4h .. 4h+3 then 8+4h .. 8+4h+3 of the group, h = lane half).
// ds_read_b64_tr_b16: in each 16-lane group, lane i addresses row base + i/4,
// columns d0 + 4(i%4) .. +3, and receives column d0 + i of the four rows.
__device__ __attribute__((always_inline)) bf16x8 tr_frag(const __bf16 *lo, const __bf16 *hi)
{
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lo));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(hi));
    const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
}

// Per-lane LDS offsets (elements) into a swizzled 64 x D stage.
template <int D>
struct LaneMap {
    using TL = BTile<D>;
    int row[TL::kKs];                // row operand: row l32 (+32 kt), chunk 2ks + hh
    int trlo[TL::kDt], trhi[TL::kDt];  // transposed operand of group 0, per 32-column block

    __device__ LaneMap(int lane)
    {
        const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks)
            row[ks] = soff<D>(l32, 2 * ks + hh);       // swz(l32 + 32kt) == swz(l32)
        const int g = lane >> 4, i = lane & 15;
        const int r = 4 * (g >> 1) + (i >> 2);         // swz(16 grp + r) == swz(r)
#pragma unroll
        for (int dt = 0; dt < TL::kDt; ++dt) {
            const int col = dt * 32 + 16 * (g & 1) + 4 * (i & 3);
            trlo[dt] = soff<D>(r, col >> 3) + (col & 7);
            trhi[dt] = soff<D>(r + 8, col >> 3) + (col & 7);
        }
    }
};

// Staging of one 64-row tile from a buffer resource (rows past its range read
// as zeros).  bf16: direct-to-LDS loads, one per 1 KiB block of the wave; fp32:
// loaded, rounded to bf16 and stored by the thread.
template <int D, bool F32, int NT = kBThreads>
struct Stager {
    using TL = BTile<D>;
    static constexpr int kEsize = F32 ? 4 : 2;
    static constexpr int kRC = kT * TL::kCh / NT;   // chunks per thread per staged tile
    static_assert(kRC * NT == kT * TL::kCh, "threads must divide the tile's chunks");
    uint32_t goff[kRC];   // byte offset of this thread's chunk in the source tile
    int row[kRC];         // its row in the tile
    int slot[kRC];        // element offset of its chunk (fp32) / its wave's block (bf16)

    __device__ Stager(int tid, int wave, int lane, uint32_t rb)
    {
#pragma unroll
        for (int u = 0; u < kRC; ++u) {
            const int e = tid + NT * u;
            const int r = e / TL::kCh, p = e % TL::kCh;
            row[u] = r;
            // LDS slot e holds chunk p ^ swz(r) of row r
            goff[u] = (uint32_t)r * rb + (uint32_t)((p ^ swz<D>(r)) * 8 * kEsize);
            slot[u] = F32 ? e * 8 : (wave * 64 + NT * u) * 8;
            (void)lane;
        }
    }

    __device__ __attribute__((always_inline)) void put(__amdgpu_buffer_rsrc_t r, uint32_t off, __bf16 *stage, int u) const
    {
        if constexpr (F32) {
            *reinterpret_cast<u32x4 *>(stage + slot[u]) = bload8<true>(r, off);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(stage + slot[u]), 16, (int)off, 0, 0, 0);
        }
    }
};

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

// An empty asm statement that takes a value and gives it back: it orders
// the value's producers before, and its users after, the neighbouring
// scheduling barriers, which pure arithmetic is otherwise free to cross.
typedef float pin_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void pin(f32x16 &x)
{
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        pin_f4 c = {x[i], x[i + 1], x[i + 2], x[i + 3]};
        asm volatile("" : "+v"(c));
        x[i] = c[0];
        x[i + 1] = c[1];
        x[i + 2] = c[2];
        x[i + 3] = c[3];
    }
}
__device__ __forceinline__ void pin(bf16x8 &x)
{
    u32x4 u = __builtin_bit_cast(u32x4, x);
    asm volatile("" : "+v"(u));
    x = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void pin(float4 &x)
{
    pin_f4 c = {x.x, x.y, x.z, x.w};
    asm volatile("" : "+v"(c));
    x = make_float4(c[0], c[1], c[2], c[3]);
}

// --------------------------------------------------------------------- dq
// 8 waves of 32 queries, two waves per SIMD: the accumulator (64 fp32 per
// lane), q and dO of the wave's queries (64) and one half-tile of operands fit
// the 256 registers of one of two waves, and the two waves of a SIMD overlap
// each other's exp / dS work and LDS waits with their MFMAs.  A 64-key tile in
// LDS serves all 256 queries of the workgroup.
template <int D, bool F32, bool GATHER>
__global__ __launch_bounds__(kQThreads) void bwd_dq_kernel(const BwdArgs a)
{
    using TL = BTile<D>;
    using ST = Stager<D, F32, kQThreads>;
    constexpr int kEsize = F32 ? 4 : 2;
    constexpr int kStage = 2 * TL::kElems;               // K rows | V rows
    // two tile buffers, declared apart so that reads of one provably do not
    // alias the direct-to-LDS loads in flight into the other
    __shared__ __attribute__((aligned(16))) __bf16 lds0[kStage];
    __shared__ __attribute__((aligned(16))) __bf16 lds1[kStage];

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
    int32_t n_glob = (int32_t)a.G;   // global keys of this item's list
    int32_t g_first = 0;            // GATHER: position of that list in a.gidx
    const void *qptr, *doptr;
    void *dqptr;
    const float *lse, *dl;
    if (!glob) {
        const int64_t c = rem / a.qb_win;
        if constexpr (GATHER) {
            const int32_t g0 = min(max(a.goff[c], 0), a.n_gidx);
            const int32_t g1 = min(max(a.goff[c + 1], g0), a.n_gidx);
            g_first = g0;
            n_glob = g1 - g0;
        }
        const int64_t qb = rem - c * a.qb_win;
        q_row0 = c * a.V + qb * kQRows;
        n_q = min<int64_t>(kQRows, a.V - qb * kQRows);
        n_win = (int32_t)a.V;
        kw_row0 = c * a.V;
        qptr = a.qd;
        doptr = a.dod;
        dqptr = a.dqd;
        lse = a.lse_d + head * a.N;
        dl = a.dl_d + head * a.N;
    } else {
        const int64_t gb = rem - ndet;
        q_row0 = gb * kQRows;
        n_q = min<int64_t>(kQRows, a.G - gb * kQRows);
        n_win = 0;
        kw_row0 = 0;
        qptr = a.qg;
        doptr = a.dog;
        dqptr = a.dqg;
        lse = a.lse_g + head * a.G;
        dl = a.dl_g + head * a.G;
    }
    const int32_t nkeys = n_win + n_glob;
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
    const float nlse2 = row_ok ? -lse[q_row0 + my_q] * kLog2e : 0.0f;
    const float dlt = row_ok ? dl[q_row0 + my_q] : 0.0f;

    const ST st(tid, wave, lane, rb);
    const LaneMap<D> lm(lane);
    const char *kwin = static_cast<const char *>(a.kd) + (kw_row0 * rs + hoff) * kEsize;
    const char *vwin = static_cast<const char *>(a.vd) + (kw_row0 * rs + hoff) * kEsize;
    const char *kglb = static_cast<const char *>(a.kg) + hoff * kEsize;
    const char *vglb = static_cast<const char *>(a.vg) + hoff * kEsize;

    // key tile t -> LDS buffer Ks (window keys, global keys, or the one tile
    // that straddles the two lists: each row from its own list)
    auto stage = [=](int t, __bf16 *Ks) __attribute__((always_inline)) {
        __bf16 *Vs = Ks + TL::kElems;
        const int32_t k0 = t * kT;
        if constexpr (GATHER) {
            if (!glob && k0 + kT > n_win) {
                // a tile with listed global keys: rows below n_win from the
                // window, the others gathered by index (byte offset past the
                // global rows, i.e. zeros, outside the list or for an index
                // outside [0, G))
                const int32_t r0 = max(0, n_win - k0);
                const int32_t kb0 = min(k0, n_win);
                const __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)kb0 * rb, (uint32_t)r0 * rb);
                const __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)kb0 * rb, (uint32_t)r0 * rb);
                const __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)a.G * rb);
                const __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)a.G * rb);
                const int32_t p0 = k0 - n_win;          // list position of tile row 0
#pragma unroll
                for (int u = 0; u < ST::kRC; ++u) {
                    const int32_t row = st.row[u];
                    if (row < r0) {
                        st.put(rkw, st.goff[u], Ks, u);
                        st.put(rvw, st.goff[u], Vs, u);
                    } else {
                        const int32_t pos = p0 + row;
                        const uint32_t cho = st.goff[u] - (uint32_t)row * rb;
                        uint32_t off = 0x80000000u;
                        if (pos < n_glob) {
                            const int32_t idx = a.gidx[g_first + pos];
                            if ((uint32_t)idx < (uint32_t)a.G)
                                off = (uint32_t)idx * rb + cho;
                        }
                        st.put(rkg, off, Ks, u);
                        st.put(rvg, off, Vs, u);
                    }
                }
                return;
            }
        }
        if (k0 + kT <= n_win || k0 >= n_win) {
            const bool in_win = k0 < n_win;
            const int32_t g0 = k0 - n_win;
            const int32_t rows = in_win ? kT : max(0, min(kT, (int32_t)a.G - g0));
            const char *kb = in_win ? kwin + (int64_t)k0 * rb : kglb + (int64_t)g0 * rb;
            const char *vb = in_win ? vwin + (int64_t)k0 * rb : vglb + (int64_t)g0 * rb;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)rows * rb);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)rows * rb);
#pragma unroll
            for (int u = 0; u < ST::kRC; ++u) {
                st.put(rk, st.goff[u], Ks, u);
                st.put(rv, st.goff[u], Vs, u);
            }
        } else {
            const int32_t r0 = n_win - k0;
            const int32_t ng = max(0, min(kT - r0, (int32_t)a.G));
            const __amdgpu_buffer_rsrc_t rkw = make_rsrc(kwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            const __amdgpu_buffer_rsrc_t rvw = make_rsrc(vwin + (int64_t)k0 * rb, (uint32_t)r0 * rb);
            const __amdgpu_buffer_rsrc_t rkg = make_rsrc(kglb, (uint32_t)ng * rb);
            const __amdgpu_buffer_rsrc_t rvg = make_rsrc(vglb, (uint32_t)ng * rb);
            const uint32_t gs = (uint32_t)r0 * rb;
#pragma unroll
            for (int u = 0; u < ST::kRC; ++u) {
                if (st.row[u] < r0) {
                    st.put(rkw, st.goff[u], Ks, u);
                    st.put(rvw, st.goff[u], Vs, u);
                } else {
                    st.put(rkg, st.goff[u] - gs, Ks, u);
                    st.put(rvg, st.goff[u] - gs, Vs, u);
                }
            }
        }
    };

    f32x16 dq[TL::kDt];
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dq[dt][r] = 0.0f;
    const float cl = a.c_log2;

    // One 64-key tile in two 32-key halves: S^T, dP^T (K and V row fragments
    // from LDS), dS^T = P^T o (dP^T - D) with P^T = exp2(S^T cl - lse2) in
    // bf16, then dq^T += K^T dS^T (K^T by transposing LDS reads).  Keys past
    // the end of the list need no mask: their K rows read as zeros, so
    // whatever their (finite) dS, they add nothing to dq.
    auto tile = [&](const __bf16 *Ks) __attribute__((always_inline)) {
        const __bf16 *Vs = Ks + TL::kElems;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.0f;
                dp[r] = 0.0f;
            }
#pragma unroll
            for (int ks = 0; ks < TL::kKs; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(Ks + kt * 32 * D + lm.row[ks]);
                const bf16x8 va = *reinterpret_cast<const bf16x8 *>(Vs + kt * 32 * D + lm.row[ks]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp, 0, 0, 0);
            }
            bf16x8 ds[2];
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int r = 8 * i2 + m;
                    // P <= 1 for every allowed key; the clamp (free on the
                    // exp) keeps a key past the list finite for any lse
                    const float p = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(fmaf(s[r], cl, nlse2)), 0.0f, 1.0f);
                    ds[i2][m] = (__bf16)(p * (dp[r] - dlt));
                }
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                for (int dt = 0; dt < TL::kDt; ++dt) {
                    const int grp = 2 * kt + i2;
                    const bf16x8 ktf = tr_frag(Ks + grp * 16 * D + lm.trlo[dt], Ks + grp * 16 * D + lm.trhi[dt]);
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf, ds[i2], dq[dt], 0, 0, 0);
                }
        }
    };

    // tile t is computed from one buffer while tile t + 1 loads into the other;
    // each step ends with the wait for that load and a barrier
    stage(0, lds0);
    wait_vm<0>();
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles)
            stage(t + 1, lds1);
        if (wave_active)
            tile(lds0);
        if (t + 1 >= ntiles)
            break;
        wait_vm<0>();
        __syncthreads();
        if (t + 2 < ntiles)
            stage(t + 2, lds0);
        if (wave_active)
            tile(lds1);
        if (t + 2 >= ntiles)
            break;
        wait_vm<0>();
        __syncthreads();
    }
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
template <int D, bool F32, bool SUBSET>
__global__ __launch_bounds__(kBThreads) void bwd_dkdv_kernel(const BwdArgs a)
{
    using TL = BTile<D>;
    constexpr int kEsize = F32 ? 4 : 2;
    constexpr int kStage = 2 * TL::kElems;               // Q rows | dO rows
    // two tile buffers (rows, then [lse | D][row]), declared apart so that
    // reads of one provably do not alias the loads in flight into the other
    __shared__ __attribute__((aligned(16))) __bf16 lds0[kStage];
    __shared__ __attribute__((aligned(16))) __bf16 lds1[kStage];
    __shared__ __attribute__((aligned(16))) float lsd0[2][kT];
    __shared__ __attribute__((aligned(16))) float lsd1[2][kT];

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
    // query segments: [q0, q0 + nq) of (q, dO, lse, D)
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
        if constexpr (SUBSET) {
            // with a subset the detail queries' share arrives through acc_k /
            // acc_v (added in the epilogue): stream the global queries only
            qp0 = a.qg; dop0 = a.dog; ls0 = a.lse_g + head * a.G; dl0 = a.dl_g + head * a.G;
            q00 = 0; nq0 = a.G;
            qp1 = nullptr; dop1 = nullptr; ls1 = nullptr; dl1 = nullptr;
            nq1 = 0;
        } else {
            qp0 = a.qd; dop0 = a.dod; ls0 = a.lse_d + head * a.N; dl0 = a.dl_d + head * a.N;
            q00 = 0; nq0 = a.N;
            qp1 = a.qg; dop1 = a.dog; ls1 = a.lse_g + head * a.G; dl1 = a.dl_g + head * a.G;
            nq1 = a.G;
        }
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

    const Stager<D, F32> st(tid, wave, lane, rb);
    const LaneMap<D> lm(lane);

    // query tile -> LDS buffer (Qs, Ls): q rows, dO rows, and lse (even waves)
    // or D (odd waves) of the 64 rows by a 4-byte direct-to-LDS load per lane.
    // Rows past the list read as zeros: their q and dO rows are zero, so they
    // add nothing to dk or dv whatever their P.
    auto stage = [=](const char *qb, const char *ob, const float *lb, int32_t rows, __bf16 *Qs,
                     float (*Ls)[kT]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)rows * rb);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(ob, (uint32_t)rows * rb);
        __bf16 *Os = Qs + TL::kElems;
#pragma unroll
        for (int u = 0; u < Stager<D, F32>::kRC; ++u) {
            st.put(rq, st.goff[u], Qs, u);
            st.put(ro, st.goff[u], Os, u);
        }
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(lb, (uint32_t)rows * 4u);
        dma4(rl, &Ls[wave & 1][0], lane);
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

    // One 64-query tile, software-pipelined by 32-query halves so that the
    // VALU work of one half (P, dS) issues between the MFMAs of the other:
    //   S, dP of half 0 | S, dP of half 1 + P, dS of half 0
    //   | dv, dk of half 0 + P, dS of half 1 | dv, dk of half 1.
    // The last phase needs registers only: it runs after the barrier that
    // hands over the next tile, while that tile's row fragments and lse / D
    // values are read, so that a tile starts with its operands in registers.
    bf16x8 qa[2][TL::kKs], oa[2][TL::kKs];     // q, dO row fragments (A operands)
    float4 Lq[2][4], Dq[2][4];                 // lse, D of this lane's query rows
    f32x16 s[2], dp[2];
    bf16x8 pb[2][2], db[2][2];                 // P, dS in bf16 (B operands)
    bf16x8 oT[2][2][TL::kDt], qT[2][2][TL::kDt];   // dO^T, Q^T fragments per half

    // row fragments of one half of the tile in Qs
    auto frag_load = [&](const __bf16 *Qs, int qt) __attribute__((always_inline)) {
        const __bf16 *Os = Qs + TL::kElems;
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks) {
            qa[qt][ks] = *reinterpret_cast<const bf16x8 *>(Qs + qt * 32 * D + lm.row[ks]);
            oa[qt][ks] = *reinterpret_cast<const bf16x8 *>(Os + qt * 32 * D + lm.row[ks]);
        }
    };
    // lse and D of this lane's query rows of the tile
    auto ld_load = [&](const float (*Ls)[kT]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                Lq[qt][g] = *reinterpret_cast<const float4 *>(&Ls[0][qt * 32 + 8 * g + 4 * hh]);
                Dq[qt][g] = *reinterpret_cast<const float4 *>(&Ls[1][qt * 32 + 8 * g + 4 * hh]);
            }
    };
    // S = Q K^T and dP = dO V^T of one half
    auto sdp = [&](int qt) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks) {
            s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[qt][ks], kf[ks], s[qt], 0, 0, 0);
            dp[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[qt][ks], vf[ks], dp[qt], 0, 0, 0);
        }
    };
    auto pin_half = [&](int qt) __attribute__((always_inline)) {
        pin(s[qt]);
        pin(dp[qt]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            pin(Lq[qt][g]);
            pin(Dq[qt][g]);
        }
    };
    auto pin_pd = [&](int qt) __attribute__((always_inline)) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
            pin(pb[qt][i2]);
            pin(db[qt][i2]);
        }
    };
    // P = exp2(S cl - lse2) and dS = P o (dP - D) of one half, in bf16;
    // rows = queries of this lane's registers (8i + 4hh + j)
    auto softmax_grad = [&](int qt) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 L = Lq[qt][g];
            const float4 Dv = Dq[qt][g];
            const float lv[4] = {L.x, L.y, L.z, L.w};
            const float dv[4] = {Dv.x, Dv.y, Dv.z, Dv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g + j;
                const float p = __builtin_amdgcn_exp2f(fmaf(s[qt][r], cl, -lv[j] * kLog2e));
                pb[qt][g >> 1][4 * (g & 1) + j] = (__bf16)p;
                db[qt][g >> 1][4 * (g & 1) + j] = (__bf16)(p * (dp[qt][r] - dv[j]));
            }
        }
    };
    // dO^T, Q^T fragments of one half (query groups 2qt, 2qt + 1)
    auto tr_load = [&](const __bf16 *Qs, int qt) __attribute__((always_inline)) {
        const __bf16 *Os = Qs + TL::kElems;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int dt = 0; dt < TL::kDt; ++dt) {
                const int grp = 2 * qt + i2;
                oT[qt][i2][dt] = tr_frag(Os + grp * 16 * D + lm.trlo[dt], Os + grp * 16 * D + lm.trhi[dt]);
                qT[qt][i2][dt] = tr_frag(Qs + grp * 16 * D + lm.trlo[dt], Qs + grp * 16 * D + lm.trhi[dt]);
            }
    };
    // dv^T += dO^T P and dk^T += Q^T dS of one half
    auto dvdk = [&](int qt) __attribute__((always_inline)) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int dt = 0; dt < TL::kDt; ++dt) {
                dvT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oT[qt][i2][dt], pb[qt][i2], dvT[dt], 0, 0, 0);
                dkT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT[qt][i2][dt], db[qt][i2], dkT[dt], 0, 0, 0);
            }
    };
    constexpr int kM = 2 * TL::kKs;            // MFMAs of one S, dP half = of one dv, dk half
    constexpr int kTailLds = (2 * TL::kKs + 16) / kM;   // operand reads per MFMA of the last phase
    // phases 1-3 of the tile in Qs (half 0's operands already in registers)
    auto tile_main = [&](const __bf16 *Qs) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[qt][r] = 0.0f;
                dp[qt][r] = 0.0f;
            }
        // phase 1: S, dP of half 0 while half 1's row fragments arrive
        sdp(0);
        frag_load(Qs, 1);
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // phase 2: S, dP of half 1 with P, dS of half 0.  The empty asm
        // statements keep each half's work inside its phase: pure arithmetic
        // is otherwise free to drift across the scheduling barriers.
        pin(qa[1][0]);
        pin(oa[1][0]);
        pin_half(0);
        sdp(1);
        softmax_grad(0);
        tr_load(Qs, 0);
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);   // then VALU
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // then LDS reads
        }
        pin_pd(0);
        __builtin_amdgcn_sched_barrier(0);
        // phase 3: dv, dk of half 0 with P, dS of half 1
        pin_pd(0);
        pin_half(1);
        dvdk(0);
        softmax_grad(1);
        tr_load(Qs, 1);
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        pin_pd(1);
        __builtin_amdgcn_sched_barrier(0);
    };
    // phase 4 (dv, dk of half 1) with the next tile's first operand reads
    auto tile_tail = [&](const __bf16 *Qn, const float (*Ln)[kT]) __attribute__((always_inline)) {
        pin_pd(1);
        dvdk(1);
        frag_load(Qn, 0);
        ld_load(Ln);
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, kTailLds, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // the query lists (global key block: all detail rows, then all global
    // rows; window key block: the window's rows).  Within a list, tile t + 1
    // loads into one buffer while tile t is computed from the other.  After
    // phase 3 of tile t, a wait for that load and a barrier: tile t + 1 is
    // then in LDS and no wave reads tile t's buffer again, so tile t + 2
    // starts loading into it.  Past the last tile, the operand reads of the
    // tail fetch unused values from the idle buffer.
    const int nseg = nq1 > 0 ? 2 : 1;
    for (int sg = 0; sg < nseg; ++sg) {
        const int64_t q0 = sg ? 0 : q00;
        const int64_t nq = sg ? nq1 : nq0;
        const char *qbase = static_cast<const char *>(sg ? qp1 : qp0) + (q0 * rs + hoff) * kEsize;
        const char *obase = static_cast<const char *>(sg ? dop1 : dop0) + (q0 * rs + hoff) * kEsize;
        const float *lbase = ((wave & 1) ? (sg ? dl1 : dl0) : (sg ? ls1 : ls0)) + q0;
        const int nt = (int)((nq + kT - 1) / kT);
        auto put = [=](int t, __bf16 *Qs, float (*Ls)[kT]) __attribute__((always_inline)) {
            const int64_t r0 = (int64_t)t * kT;
            stage(qbase + r0 * rb, obase + r0 * rb, lbase + r0, (int32_t)min<int64_t>(kT, nq - r0), Qs, Ls);
        };
        if (sg)
            __syncthreads();      // every wave is done with both buffers
        put(0, lds0, lsd0);
        wait_vm<0>();
        __syncthreads();
        if (nt > 1)
            put(1, lds1, lsd1);
        if (wave_active) {
            frag_load(lds0, 0);
            ld_load(lsd0);
        }
        for (int t = 0; t < nt; t += 2) {
            if (wave_active)
                tile_main(lds0);
            wait_vm<0>();
            __syncthreads();
            if (t + 2 < nt)
                put(t + 2, lds0, lsd0);
            if (wave_active)
                tile_tail(lds1, lsd1);
            if (t + 1 >= nt)
                break;
            if (wave_active)
                tile_main(lds1);
            wait_vm<0>();
            __syncthreads();
            if (t + 3 < nt)
                put(t + 3, lds1, lsd1);
            if (wave_active)
                tile_tail(lds0, lsd0);
        }
    }
    if (!key_ok)
        return;

    const float sc = a.scale;
    const int64_t obase = (k_row0 + my_k) * rs + hoff;
#pragma unroll
    for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = dt * 32 + 8 * i + 4 * hh;
            float k4[4], v4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                k4[j] = dkT[dt][4 * i + j] * sc;
                v4[j] = dvT[dt][4 * i + j];
            }
            if constexpr (SUBSET) {
                if (glob) {
                    const float4 ak = *reinterpret_cast<const float4 *>(a.acc_k + obase + d);
                    const float4 av = *reinterpret_cast<const float4 *>(a.acc_v + obase + d);
                    k4[0] += ak.x; k4[1] += ak.y; k4[2] += ak.z; k4[3] += ak.w;
                    v4[0] += av.x; v4[1] += av.y; v4[2] += av.z; v4[3] += av.w;
                }
            }
            store4<F32>(dkptr, obase + d, k4[0], k4[1], k4[2], k4[3]);
            store4<F32>(dvptr, obase + d, v4[0], v4[1], v4[2], v4[3]);
        }
}

// ------------------------------------------------- per-window subset: listed keys
// The detail queries' share of dk/dv of the global keys a window lists: one
// workgroup per (head, window), its listed keys in blocks of 128 (32 per
// wave, gathered by index), each block streaming the window's V queries in
// 64-row tiles like a window key block of bwd_dkdv_kernel (plain order: S and
// dP, then P and dS, then dv and dk).  The sums go into fp32 acc_k / acc_v
// with atomic adds, since a key may be listed by several windows; the global
// key blocks of bwd_dkdv_kernel add them to the global queries' share.  Keys
// past the list or with an index outside [0, G) have zero K and V rows and
// store nothing.
template <int D, bool F32>
__global__ __launch_bounds__(kBThreads) void bwd_listed_kernel(const BwdArgs a)
{
    using TL = BTile<D>;
    using ST = Stager<D, F32>;
    constexpr int kEsize = F32 ? 4 : 2;
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * TL::kElems];   // q rows | dO rows
    __shared__ __attribute__((aligned(16))) float lsd[2][kT];             // lse | D

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int64_t item = xcd_item(blockIdx.x, gridDim.x);     // head * C + window
    const int64_t head = item / a.C;
    const int64_t c = item - head * a.C;
    const int32_t g0 = min(max(a.goff[c], 0), a.n_gidx);
    const int32_t g1 = min(max(a.goff[c + 1], g0), a.n_gidx);
    const int32_t n_list = g1 - g0;
    const int64_t rs = (int64_t)a.heads * D;
    const uint32_t rb = (uint32_t)(rs * kEsize);
    const int64_t hoff = head * D;
    const ST st(tid, wave, lane, rb);
    const LaneMap<D> lm(lane);
    const int64_t q0 = c * a.V;
    const char *qbase = static_cast<const char *>(a.qd) + (q0 * rs + hoff) * kEsize;
    const char *obase = static_cast<const char *>(a.dod) + (q0 * rs + hoff) * kEsize;
    const float *lbase = ((wave & 1) ? a.dl_d : a.lse_d) + head * a.N + q0;
    const int nt = (int)((a.V + kT - 1) / kT);
    const float cl = a.c_log2;
    const __bf16 *Qs = lds;
    const __bf16 *Os = lds + TL::kElems;

    for (int32_t k0 = 0; k0 < n_list; k0 += kBRows) {     // uniform over the workgroup
        const int32_t pos = k0 + wave * 32 + l32;
        int32_t idx = -1;
        if (pos < n_list) {
            const int32_t v = a.gidx[g0 + pos];
            idx = (uint32_t)v < (uint32_t)a.G ? v : -1;
        }
        const bool wave_active = k0 + wave * 32 < n_list;
        bf16x8 kf[TL::kKs], vf[TL::kKs];
        const int64_t koff = (int64_t)max(idx, 0) * rs + hoff + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < TL::kKs; ++ks) {
            kf[ks] = idx >= 0 ? gload8<F32>(a.kg, koff + ks * 16) : zero8();
            vf[ks] = idx >= 0 ? gload8<F32>(a.vg, koff + ks * 16) : zero8();
        }
        f32x16 dkT[TL::kDt], dvT[TL::kDt];
#pragma unroll
        for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dkT[dt][r] = 0.0f;
                dvT[dt][r] = 0.0f;
            }
        for (int t = 0; t < nt; ++t) {
            __syncthreads();        // every wave is done with the previous tile
            const int64_t r0 = (int64_t)t * kT;
            const uint32_t rows = (uint32_t)min<int64_t>(kT, a.V - r0);
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase + r0 * rb, rows * rb);
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase + r0 * rb, rows * rb);
#pragma unroll
            for (int u = 0; u < ST::kRC; ++u) {
                st.put(rq, st.goff[u], lds, u);
                st.put(ro, st.goff[u], lds + TL::kElems, u);
            }
            dma4(make_rsrc(lbase + r0, rows * 4u), &lsd[wave & 1][0], lane);
            wait_vm<0>();
            __syncthreads();
            if (!wave_active)
                continue;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                f32x16 s, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[r] = 0.0f;
                    dp[r] = 0.0f;
                }
#pragma unroll
                for (int ks = 0; ks < TL::kKs; ++ks) {
                    const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(Qs + qt * 32 * D + lm.row[ks]);
                    const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(Os + qt * 32 * D + lm.row[ks]);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[ks], dp, 0, 0, 0);
                }
                // P = exp2(S cl - lse2) (<= 1 for every listed key) and dS = P o (dP - D)
                bf16x8 pb[2], db[2];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 L = *reinterpret_cast<const float4 *>(&lsd[0][qt * 32 + 8 * g + 4 * hh]);
                    const float4 Dv = *reinterpret_cast<const float4 *>(&lsd[1][qt * 32 + 8 * g + 4 * hh]);
                    const float lv[4] = {L.x, L.y, L.z, L.w};
                    const float dv[4] = {Dv.x, Dv.y, Dv.z, Dv.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * g + j;
                        const float p = __builtin_amdgcn_fmed3f(
                            __builtin_amdgcn_exp2f(fmaf(s[r], cl, -lv[j] * kLog2e)), 0.0f, 1.0f);
                        pb[g >> 1][4 * (g & 1) + j] = (__bf16)p;
                        db[g >> 1][4 * (g & 1) + j] = (__bf16)(p * (dp[r] - dv[j]));
                    }
                }
                // dv^T += dO^T P and dk^T += Q^T dS (query groups 2qt, 2qt + 1)
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                    for (int dt = 0; dt < TL::kDt; ++dt) {
                        const int grp = 2 * qt + i2;
                        const bf16x8 oT = tr_frag(Os + grp * 16 * D + lm.trlo[dt], Os + grp * 16 * D + lm.trhi[dt]);
                        const bf16x8 qT = tr_frag(Qs + grp * 16 * D + lm.trlo[dt], Qs + grp * 16 * D + lm.trhi[dt]);
                        dvT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oT, pb[i2], dvT[dt], 0, 0, 0);
                        dkT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT, db[i2], dkT[dt], 0, 0, 0);
                    }
            }
        }
        if (idx >= 0) {
            const float sc = a.scale;
            const int64_t abase = (int64_t)idx * rs + hoff;
#pragma unroll
            for (int dt = 0; dt < TL::kDt; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = dt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    unsafeAtomicAdd(a.acc_k + abase + d, dkT[dt][r] * sc);
                    unsafeAtomicAdd(a.acc_v + abase + d, dvT[dt][r]);
                }
        }
    }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float *x, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        x[i] = 0.0f;
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
    if (a.goff != nullptr)
        hipLaunchKernelGGL((bwd_dq_kernel<D, F32, true>), dim3((uint32_t)a.dq_items), dim3(kQThreads), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<D, F32, false>), dim3((uint32_t)a.dq_items), dim3(kQThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (a.goff != nullptr && a.G > 0) {
        // detail queries' share of the listed global keys into acc_k / acc_v
        const int64_t n = 2 * a.G * a.heads * D;          // acc_k and acc_v, contiguous
        const int64_t zb = (n + 255) / 256;
        const int64_t items = (int64_t)a.heads * a.C;
        if (zb > 0x7fffffffLL || items > 0x7fffffffLL)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((uint32_t)zb), dim3(256), 0, s, a.acc_k, n);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL((bwd_listed_kernel<D, F32>), dim3((uint32_t)items), dim3(kBThreads), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (a.goff != nullptr)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, true>), dim3((uint32_t)a.kv_items), dim3(kBThreads), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, false>), dim3((uint32_t)a.kv_items), dim3(kBThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int hier_attn_bwd_block_rows() { return kBRows; }
int hier_attn_bwd_dq_rows() { return kQRows; }

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
