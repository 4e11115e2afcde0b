// device_common.hpp -- small gfx950 device helpers shared by the GDN kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;  // CDNA4 wavefront width (single target: gfx950)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
// Streaming (non-temporal) 128-bit load / store.
__device__ __forceinline__ f32x4 ld4_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st4_nt(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// Workgroup barrier for data written to LDS with ds_write: waits for this
// wavefront's LDS operations only, so that outstanding global and
// direct-to-LDS loads and global stores stay in flight across it.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// bfloat16 bits -> float32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Unpack the two bf16 values of a 32-bit word (low half first).
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
}

// Load N consecutive elements (float32 or bf16) as float32.  The first
// element must be aligned to the vector width used (16 bytes for float32 and
// for 8 bf16 values, 8 bytes for 4 bf16 values).
template <int N, bool BF16>
__device__ __forceinline__ void load_vec(const void* base, size_t offset, float (&out)[N]) {
    if constexpr (BF16 && N % 8 == 0) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + offset);
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            uint4 w = p[i];
            unpack_bf16x2(w.x, out[8 * i + 0], out[8 * i + 1]);
            unpack_bf16x2(w.y, out[8 * i + 2], out[8 * i + 3]);
            unpack_bf16x2(w.z, out[8 * i + 4], out[8 * i + 5]);
            unpack_bf16x2(w.w, out[8 * i + 6], out[8 * i + 7]);
        }
    } else if constexpr (BF16) {
        static_assert(N % 4 == 0, "bf16 vector loads move 4 or 8 values at a time");
        const uint2* p = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + offset);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            uint2 w = p[i];
            unpack_bf16x2(w.x, out[4 * i + 0], out[4 * i + 1]);
            unpack_bf16x2(w.y, out[4 * i + 2], out[4 * i + 3]);
        }
    } else {
        static_assert(N % 4 == 0, "float32 vector loads move 4 values at a time");
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + offset);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            float4 w = p[i];
            out[4 * i + 0] = w.x;
            out[4 * i + 1] = w.y;
            out[4 * i + 2] = w.z;
            out[4 * i + 3] = w.w;
        }
    }
}

// Load 4 consecutive elements (float32 or bf16) as float32.
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, size_t offset) {
    if constexpr (BF16) {
        uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + offset);
        float a, b, c, d;
        unpack_bf16x2(w.x, a, b);
        unpack_bf16x2(w.y, c, d);
        return f32x4{a, b, c, d};
    } else {
        return ld4(static_cast<const float*>(base) + offset);
    }
}

// ---------------------------------------------------------------------------
// Butterfly sums across lane groups of a wave64.  Each step adds a value to
// its partner's copy; IEEE addition is commutative, so every lane of a group
// ends with the bit-identical total.
//   xor 8  : DPP row_ror:8 inside each 16-lane row
//   xor 16 : v_permlane16_swap (odd rows <-> even rows)
//   xor 32 : v_permlane32_swap (upper half <-> lower half)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float add_xor8(float x) {
    int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128 /* row_ror:8 */, 0xf, 0xf, false);
    return x + __int_as_float(y);
}

__device__ __forceinline__ float add_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float add_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two butterflies in one swap: the swap exchanges a's upper (odd) lanes with
// b's lower (even) ones, so the sum holds a's total where a's group sits in
// the lower half (even 16-lane rows) and b's total in the upper half (odd
// rows).  No register copy is needed, unlike a swap of a value with itself.
//   add_xor32_pair: lanes 0..31 <- a over (l, l^32); lanes 32..63 <- b over the same
//   add_xor16_pair: rows 0 and 2 <- a over (l, l^16); rows 1 and 3 <- b over the same
__device__ __forceinline__ float add_xor32_pair(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float add_xor16_pair(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

//   xor 4  : ds_swizzle in bitmask mode (and 0x1f, xor 4) inside 32 lanes
__device__ __forceinline__ float add_xor4(float x) {
    int y = __builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1f | (4 << 10));
    return x + __int_as_float(y);
}

// Sum over the lanes that share lane % FROM, i.e. the butterfly over lane
// bits log2(FROM)..5.  FROM is 4 or 8.
template <int FROM>
__device__ __forceinline__ float sum_lanes_from(float x) {
    static_assert(FROM == 4 || FROM == 8, "row-group stride");
    if constexpr (FROM == 4) x = add_xor4(x);
    return add_xor32(add_xor16(add_xor8(x)));
}

}  // namespace gdn
