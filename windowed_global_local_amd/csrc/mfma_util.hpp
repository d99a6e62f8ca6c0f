// mfma_util.hpp -- device helpers shared by the gfx950 attention kernels
// (forward and backward): vector types, buffer resources, 8-element loads and
// the XCD-aware workgroup numbering.  Internal; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atlas {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int32_t kRsrcWord3 = 0x00020000;   // raw buffer, gfx9 family

// Buffer resource for a wave-uniform base and size (made provably uniform, so
// the loads need no per-lane descriptor loop).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// 8 consecutive elements at byte offset off of a buffer, as bf16 (fp32 inputs
// are rounded to nearest even); out-of-range offsets read as zeros.
template <bool F32>
__device__ inline u32x4 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (F32) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, 0);
        bf16x8 b;
        b[0] = (__bf16)__uint_as_float(x.x); b[1] = (__bf16)__uint_as_float(x.y);
        b[2] = (__bf16)__uint_as_float(x.z); b[3] = (__bf16)__uint_as_float(x.w);
        b[4] = (__bf16)__uint_as_float(y.x); b[5] = (__bf16)__uint_as_float(y.y);
        b[6] = (__bf16)__uint_as_float(y.z); b[7] = (__bf16)__uint_as_float(y.w);
        return __builtin_bit_cast(u32x4, b);
    } else {
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    }
}

// 8 consecutive elements at element offset elem_off of a tensor, as bf16.
template <bool F32>
__device__ inline bf16x8 gload8(const void *base, int64_t elem_off)
{
    if constexpr (F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem_off);
        const float4 x = p[0], y = p[1];
        bf16x8 r;
        r[0] = (__bf16)x.x; r[1] = (__bf16)x.y; r[2] = (__bf16)x.z; r[3] = (__bf16)x.w;
        r[4] = (__bf16)y.x; r[5] = (__bf16)y.y; r[6] = (__bf16)y.z; r[7] = (__bf16)y.w;
        return r;
    } else {
        return *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(base) + elem_off);
    }
}

__device__ inline bf16x8 zero8()
{
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Consecutive workgroup ids go round-robin over the 8 XCDs; this renumbers
// them so that XCD x (= bid % 8) walks one contiguous range of item numbers.
__device__ inline int64_t xcd_item(uint32_t bid, uint32_t nb)
{
    const uint32_t xcd = bid & 7u, jx = bid >> 3, q8 = nb >> 3, r8 = nb & 7u;
    return (xcd < r8) ? (int64_t)xcd * (q8 + 1) + jx
                      : (int64_t)r8 * (q8 + 1) + (int64_t)(xcd - r8) * q8 + jx;
}

// Position of row r (0..63) of a 64-row tile inside a transposed operand
// stage.  The C/D registers of v_mfma_f32_32x32x16_bf16 hold rows
// 8i + 4h + j (register 4i + j, lane half h); a row at offset 8i + 4h + j of
// its 16-row group is stored at 8h + 4i + j, so that the 8 registers that
// form one B operand (k = 8h .. 8h + 7 of a 16-step) meet their A operand in
// 8 consecutive stored positions.
__device__ constexpr int tperm(int r)
{
    return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

}  // namespace mfma
}  // namespace atlas
