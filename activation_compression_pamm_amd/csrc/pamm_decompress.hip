// pamm_decompress.hip -- reconstruction X~_i = alpha_i * C_f(i) on gfx950.
//
// The approximation of a row by its generator from "QKV Projections Require
// a Fraction of Their Memory", section 2 "Metodologia", sub-part "Algoritmo
// in Due Fasi"; dropped rows (f outside [0, k)) reconstruct to zero.  The
// product is an fp32 multiply rounded once more to the storage dtype.  One
// thread per 16 bytes of output, coalesced along each row.
#include "pamm_device.hpp"
#include "pamm_kernels.hpp"

namespace pamm {

template <int DT>
__global__ __launch_bounds__(256) void decompress_kernel(DecompressArgs a, int64_t row_chunks) {
    constexpr int PE = Elem<DT>::per16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.n * row_chunks) return;
    const int64_t i = idx / row_chunks;
    const int64_t col = (idx % row_chunks) * PE;
    const int fi = a.f[i];
    const bool valid = fi >= 0 && fi < a.k;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (valid) {
        const float al = a.alpha[i];
        const uint4 c = load16_tail<DT>(reinterpret_cast<const char*>(a.C) + (int64_t)fi * a.d * Elem<DT>::size, col,
                                        a.d);
        float v[PE];
        unpack16<DT>(c, v);
        uint32_t w[4];
        if constexpr (DT == DT_BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = f32_to_bf16(al * v[2 * q]) | (f32_to_bf16(al * v[2 * q + 1]) << 16);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = __float_as_uint(al * v[q]);
        }
        out = make_uint4(w[0], w[1], w[2], w[3]);
    }
    char* dst = reinterpret_cast<char*>(a.Xt) + i * a.ldxt_bytes + col * Elem<DT>::size;
    if (col + PE <= a.d) {
        *reinterpret_cast<uint4*>(dst) = out;
    } else {
        const uint32_t w[4] = {out.x, out.y, out.z, out.w};
        for (int e = 0; e < PE && col + e < a.d; ++e) {
            if constexpr (DT == DT_BF16)
                reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            else
                reinterpret_cast<uint32_t*>(dst)[e] = w[e];
        }
    }
}

hipError_t run_decompress(const DecompressArgs& a, int dtype, hipStream_t st) {
    const int per = dtype == DT_BF16 ? 8 : 4;
    const int64_t row_chunks = (a.d + per - 1) / per;
    const int64_t total = a.n * row_chunks;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(decompress_kernel<DT_BF16>, grid, dim3(256), 0, st, a, row_chunks);
    else
        hipLaunchKernelGGL(decompress_kernel<DT_F32>, grid, dim3(256), 0, st, a, row_chunks);
    return hipGetLastError();
}

}  // namespace pamm
