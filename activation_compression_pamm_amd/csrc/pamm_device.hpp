// pamm_device.hpp -- device helpers shared by the PAMM kernels (gfx950).
//
// Wave64 everywhere.  MFMA operand layouts used below (checked on gfx950):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + 0..7] and
//       B^T[l%16][8*(l/16) + 0..7]; result element i of lane l is
//       D[4*(l/16) + i][l%16].
//   v_mfma_f32_16x16x4f32:   lane l holds A[l%16][l/16], B^T[l%16][l/16];
//       result as above.
//   v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32) + 0..7] and
//       B[8*(l/32) + 0..7][l%32]; result element i of lane l is
//       D[8*(i/4) + 4*(l/32) + i%4][l%32].
//   v_mfma_f32_32x32x2f32:   lane l holds A[l%32][l/32], B[l/32][l%32];
//       result as above.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pamm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum : int { DT_F32 = 0, DT_BF16 = 1 };

// Elements of a dtype held by one 16-byte vector.
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int size = 4; static constexpr int per16 = 4; };
template <> struct Elem<DT_BF16> { static constexpr int size = 2; static constexpr int per16 = 8; };

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Unpack a 16-byte vector of stored elements to floats (8 for bf16, 4 for fp32).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float* out) {
    if constexpr (DT == DT_BF16) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            out[2 * q] = __uint_as_float(w[q] << 16);
            out[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    } else {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
}

// Load the 16-byte group of row-element `col` (a multiple of per16) from a
// row that holds `len` valid elements; missing elements read as zero.  The
// full-vector path needs a 16-byte aligned address.
template <int DT>
__device__ __forceinline__ uint4 load16_tail(const char* row, int64_t col, int64_t len) {
    constexpr int P = Elem<DT>::per16;
    if (col + P <= len) return *reinterpret_cast<const uint4*>(row + col * Elem<DT>::size);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col >= len) return v;
    uint32_t w[4] = {0, 0, 0, 0};
    if constexpr (DT == DT_BF16) {
        const uint16_t* r = reinterpret_cast<const uint16_t*>(row);
        for (int e = 0; e < P; ++e)
            if (col + e < len) w[e >> 1] |= (uint32_t)r[col + e] << (16 * (e & 1));
    } else {
        const uint32_t* r = reinterpret_cast<const uint32_t*>(row);
        for (int e = 0; e < P; ++e)
            if (col + e < len) w[e] = r[col + e];
    }
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    return v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint (streamed data that is not reused).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, 64); }

}  // namespace pamm
