// pamm_api.hip -- the extern "C" boundary of the PAMM library (declared in
// include/pamm.h): argument validation, workspace carve-up, launches.
// Nothing here allocates device memory, synchronises, or keeps state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "pamm.h"
#include "pamm_kernels.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int elem_size(int dtype) { return dtype == PAMM_BF16 ? 2 : 4; }
int per16(int dtype) { return 16 / elem_size(dtype); }
bool dtype_ok(int dtype) { return dtype == PAMM_F32 || dtype == PAMM_BF16; }

constexpr int64_t kMaxRows = 2147483647LL;
// Largest span of a matrix, (rows - 1) * ld + row length, in elements: far
// beyond any device's memory, and small enough that no byte offset overflows.
constexpr int64_t kMaxSpan = (int64_t)1 << 40;
bool span_ok(int64_t rows, int64_t ld, int64_t len) {
    return rows <= 0 || (ld <= kMaxSpan && rows - 1 <= (kMaxSpan - len) / ld);
}

// SplitMix64 generator (Steele, Lea, Flood 2014): a Weyl sequence with
// increment 0x9E3779B97F4A7C15 passed through a two-round multiply/xorshift
// finaliser.
struct SplitMix64 {
    uint64_t s;
    uint64_t next() {
        s += 0x9E3779B97F4A7C15ULL;
        uint64_t z = s;
        z ^= z >> 30;
        z *= 0xBF58476D1CE4E5B9ULL;
        z ^= z >> 27;
        z *= 0x94D049BB133111EBULL;
        z ^= z >> 31;
        return z;
    }
    // uniform in [0, m): high word of the 128-bit product
    uint64_t below(uint64_t m) { return (uint64_t)(((unsigned __int128)next() * m) >> 64); }
};

int num_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    return cus;
}

}  // namespace

namespace pamm {

// Argument checks of pamm_wgrad, everything except the workspace.
int wgrad_check(const void* C, const int32_t* f, const float* alpha, int64_t n, int64_t k, int64_t d, const void* dY,
                int64_t d_out, int64_t lddy, int dtype, const float* dW, int64_t lddw, int transpose_out) {
    if (!dtype_ok(dtype)) return PAMM_ERR_DTYPE;
    if (n < 0 || n > kMaxRows || k < 0 || k > n || k > PAMM_MAX_K || d < 1 || d > kMaxRows || d_out < 1 ||
        d_out > kMaxRows || (n > 0 && lddy < d_out) || lddw < (transpose_out ? d : d_out))
        return PAMM_ERR_SHAPE;
    if (!span_ok(n, lddy, d_out) || !span_ok(transpose_out ? d_out : d, lddw, transpose_out ? d : d_out))
        return PAMM_ERR_SHAPE;
    if (!dW || (n > 0 && (!f || !alpha || !dY)) || (k > 0 && !C)) return PAMM_ERR_NULL;
    if (!aligned(dW, 16) || lddw % 4 != 0) return PAMM_ERR_ALIGN;
    if (n > 0 && (!aligned(f, 4) || !aligned(alpha, 4) || !aligned(dY, 16) || lddy % per16(dtype) != 0))
        return PAMM_ERR_ALIGN;
    if (k > 0 && !aligned(C, 16)) return PAMM_ERR_ALIGN;
    return PAMM_OK;
}

}  // namespace pamm

extern "C" {

int pamm_abi_version(void) { return PAMM_ABI_VERSION; }

const char* pamm_status_string(int status) {
    switch (status) {
        case PAMM_OK: return "ok";
        case PAMM_ERR_NULL: return "a required pointer is NULL";
        case PAMM_ERR_SHAPE: return "a size or leading dimension is out of range";
        case PAMM_ERR_DTYPE: return "unknown dtype";
        case PAMM_ERR_ALIGN: return "a pointer or leading dimension is not aligned";
        case PAMM_ERR_WORKSPACE: return "workspace missing or too small";
        case PAMM_ERR_UNSUPPORTED: return "unsupported request";
        case PAMM_ERR_HIP: return "HIP runtime error at launch";
        case PAMM_ERR_VALUE: return "a scalar argument is out of range";
        case PAMM_ERR_TOO_LARGE: return "the problem needs more memory than is available (the fixed no-allocation scratch array, or host memory for sampling)";
        default: return "unknown status";
    }
}

int pamm_sample_generators(int64_t n, int64_t k, uint64_t seed, int32_t* gen_idx_host) {
    if (n < 0 || n > kMaxRows || k < 0 || k > n) return PAMM_ERR_SHAPE;
    if (k == 0) return PAMM_OK;
    if (!gen_idx_host) return PAMM_ERR_NULL;
    // Floyd: for j = n-k .. n-1 draw t in [0, j]; keep t if new, else keep j.
    // The taken set is a bitmap of n bits; an allocation failure is a status,
    // not an exception that would cross the C interface.
    std::vector<uint64_t> taken;
    try {
        taken.assign((size_t)((n + 63) / 64), 0);
    } catch (...) {
        return PAMM_ERR_TOO_LARGE;
    }
    SplitMix64 rng{seed};
    int64_t m = 0;
    for (int64_t j = n - k; j < n; ++j) {
        const int64_t t = (int64_t)rng.below((uint64_t)j + 1);
        const bool seen = (taken[(size_t)t >> 6] >> (t & 63)) & 1u;
        const int64_t pick = seen ? j : t;
        taken[(size_t)pick >> 6] |= 1ull << (pick & 63);
        gen_idx_host[m++] = (int32_t)pick;
    }
    std::sort(gen_idx_host, gen_idx_host + k);
    return PAMM_OK;
}

// Workspace of pamm_compress, 256-byte aligned parts:
//   k > 256:                per-tile winners [ntiles x n] and |x|^2 [n]
//   bf16 with k > 128:      |c_j|^2 [k] (the GEMM-shaped path)
namespace {
struct CompressLayout {
    size_t off_partial, off_xn2, off_cn2, total;
    bool has_partial, has_cn2;
};
size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }
CompressLayout compress_layout(int64_t n, int64_t k, int dtype) {
    CompressLayout L{0, 0, 0, 0, false, false};
    if (n <= 0) return L;
    size_t off = 0;
    if (k > pamm::kMaxTileGens) {
        const int64_t ntiles = (k + pamm::kMaxTileGens - 1) / pamm::kMaxTileGens;
        L.has_partial = true;
        L.off_partial = off;
        off += up256(sizeof(pamm::PartialBest) * (size_t)(ntiles * n));
        L.off_xn2 = off;
        off += up256(sizeof(float) * (size_t)n);
    }
    if (dtype == PAMM_BF16 && k > pamm::kMaxTileGens / 2) {
        L.has_cn2 = true;
        L.off_cn2 = off;
        off += up256(sizeof(float) * (size_t)k);
    }
    L.total = off;
    return L;
}
}  // namespace

size_t pamm_compress_workspace_size(int64_t n, int64_t d, int64_t k, int dtype) {
    (void)d;
    return compress_layout(n, k, dtype).total;
}

int pamm_compress(const void* X, int64_t n, int64_t d, int64_t ldx, int dtype, const int32_t* gen_idx, int64_t k,
                  float eps, void* C, int32_t* f, float* alpha, void* ws, size_t ws_bytes, void* stream) {
    if (!dtype_ok(dtype)) return PAMM_ERR_DTYPE;
    if (n < 0 || n > kMaxRows || k < 0 || k > n || k > PAMM_MAX_K || d < 1 || d > kMaxRows || ldx < d ||
        !span_ok(n, ldx, d))
        return PAMM_ERR_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return PAMM_ERR_VALUE;
    if (n == 0) return PAMM_OK;
    if (!X || !f || !alpha || (k > 0 && (!gen_idx || !C))) return PAMM_ERR_NULL;
    if (!aligned(X, 16) || ldx % per16(dtype) != 0 || !aligned(f, 4) || !aligned(alpha, 4) ||
        (k > 0 && (!aligned(gen_idx, 4) || !aligned(C, 16))))
        return PAMM_ERR_ALIGN;
    const size_t need = pamm_compress_workspace_size(n, d, k, dtype);
    if (need > 0 && (!ws || ws_bytes < need)) return PAMM_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 256)) return PAMM_ERR_ALIGN;

    pamm::CompressArgs a;
    memset(&a, 0, sizeof a);
    a.X = X;
    a.n = n;
    a.d = d;
    a.ldx_bytes = ldx * elem_size(dtype);
    a.row_bytes = d * elem_size(dtype);
    a.gen_idx = gen_idx;
    a.k = (int)k;
    a.eps = eps;
    a.C = C;
    a.c_vec_ok = (d * elem_size(dtype)) % 16 == 0;
    a.f = f;
    a.alpha = alpha;
    a.num_cus = num_cus();
    const CompressLayout L = compress_layout(n, k, dtype);
    char* w = reinterpret_cast<char*>(ws);
    if (L.has_partial) {
        a.partial = reinterpret_cast<pamm::PartialBest*>(w + L.off_partial);
        a.xn2 = reinterpret_cast<float*>(w + L.off_xn2);
    }
    if (L.has_cn2) a.cn2 = reinterpret_cast<float*>(w + L.off_cn2);
    const hipError_t e = pamm::run_compress(a, dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PAMM_OK : PAMM_ERR_HIP;
}

// Workspace of pamm_forward_compress: |c_j|^2 [k] always, plus per-tile
// winners and |x|^2 when k > 256.
namespace {
struct ForwardLayout {
    size_t off_partial, off_xn2, off_cn2, total;
};
ForwardLayout forward_layout(int64_t n, int64_t k) {
    ForwardLayout L{0, 0, 0, 0};
    size_t off = 0;
    if (k > pamm::kMaxTileGens) {
        const int64_t ntiles = (k + pamm::kMaxTileGens - 1) / pamm::kMaxTileGens;
        L.off_partial = off;
        off += up256(sizeof(pamm::PartialBest) * (size_t)(ntiles * n));
        L.off_xn2 = off;
        off += up256(sizeof(float) * (size_t)n);
    }
    L.off_cn2 = off;
    off += up256(sizeof(float) * (size_t)(k > 0 ? k : 1));
    L.total = off;
    return L;
}
}  // namespace

size_t pamm_forward_compress_workspace_size(int64_t n, int64_t d, int64_t k, int dtype) {
    (void)d;
    (void)dtype;
    if (n < 0 || k < 0) return 0;
    return forward_layout(n, k).total;
}

int pamm_forward_compress(const void* X, int64_t n, int64_t d, int64_t ldx, int dtype, const void* W, int64_t d_out,
                          int64_t ldw, const void* bias, void* Y, int64_t ldy, const int32_t* gen_idx, int64_t k,
                          float eps, void* C, int32_t* f, float* alpha, void* ws, size_t ws_bytes, void* stream) {
    if (!dtype_ok(dtype)) return PAMM_ERR_DTYPE;
    if (n < 0 || n > kMaxRows || k < 0 || k > n || k > PAMM_MAX_K || d < 1 || d > kMaxRows || ldx < d ||
        d_out < 1 || d_out > kMaxRows || ldw < d || ldy < d_out || !span_ok(n, ldx, d) || !span_ok(d_out, ldw, d) ||
        !span_ok(n, ldy, d_out))
        return PAMM_ERR_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return PAMM_ERR_VALUE;
    if (dtype != PAMM_BF16) return PAMM_ERR_UNSUPPORTED;
    if (n == 0) return PAMM_OK;
    if (!X || !W || !Y || !f || !alpha || (k > 0 && (!gen_idx || !C))) return PAMM_ERR_NULL;
    if (!aligned(X, 16) || ldx % 8 != 0 || !aligned(W, 16) || ldw % 8 != 0 || !aligned(Y, 16) || ldy % 8 != 0 ||
        (bias && !aligned(bias, 2)) || !aligned(f, 4) || !aligned(alpha, 4) ||
        (k > 0 && (!aligned(gen_idx, 4) || !aligned(C, 16))))
        return PAMM_ERR_ALIGN;
    // the kernel addresses X and W with 32-bit offsets from a base
    if ((uint64_t)n * (uint64_t)ldx * 2u + 256u > 0xffffffffull ||
        (uint64_t)d_out * (uint64_t)ldw * 2u + 256u > 0xffffffffull)
        return PAMM_ERR_UNSUPPORTED;
    const ForwardLayout L = forward_layout(n, k);
    if (!ws || ws_bytes < L.total) return PAMM_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return PAMM_ERR_ALIGN;

    pamm::CompressArgs a;
    memset(&a, 0, sizeof a);
    a.X = X;
    a.n = n;
    a.d = d;
    a.ldx_bytes = ldx * 2;
    a.row_bytes = d * 2;
    a.gen_idx = gen_idx;
    a.k = (int)k;
    a.eps = eps;
    a.C = C;
    a.c_vec_ok = (d * 2) % 16 == 0;
    a.f = f;
    a.alpha = alpha;
    a.num_cus = num_cus();
    char* w = reinterpret_cast<char*>(ws);
    if (k > pamm::kMaxTileGens) {
        a.partial = reinterpret_cast<pamm::PartialBest*>(w + L.off_partial);
        a.xn2 = reinterpret_cast<float*>(w + L.off_xn2);
    }
    a.cn2 = reinterpret_cast<float*>(w + L.off_cn2);
    a.W = W;
    a.ldw_bytes = ldw * 2;
    a.d_out = d_out;
    a.Y = Y;
    a.ldy_bytes = ldy * 2;
    a.bias = bias;
    const hipError_t e = pamm::run_forward_compress(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PAMM_OK : PAMM_ERR_HIP;
}

size_t pamm_wgrad_workspace_size(int64_t n, int64_t k, int64_t d, int64_t d_out, int dtype) {
    (void)dtype;
    if (n < 0 || k < 0 || d < 1 || d_out < 1) return 0;
    return pamm::wgrad_layout(n, k, d, d_out).total;
}

int pamm_wgrad(const void* C, const int32_t* f, const float* alpha, int64_t n, int64_t k, int64_t d, const void* dY,
               int64_t d_out, int64_t lddy, int dtype, float* dW, int64_t lddw, int accumulate, int transpose_out,
               void* ws, size_t ws_bytes, void* stream) {
    const int st = pamm::wgrad_check(C, f, alpha, n, k, d, dY, d_out, lddy, dtype, dW, lddw, transpose_out);
    if (st != PAMM_OK) return st;
    const pamm::WgradLayout L = pamm::wgrad_layout(n, k, d, d_out);
    if (!ws || ws_bytes < L.total) return PAMM_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return PAMM_ERR_ALIGN;

    pamm::WgradArgs a;
    memset(&a, 0, sizeof a);
    a.C = C;
    a.f = f;
    a.alpha = alpha;
    a.n = n;
    a.k = (int)k;
    a.d = d;
    a.dY = dY;
    a.d_out = d_out;
    a.lddy_bytes = lddy * elem_size(dtype);
    a.dW = dW;
    a.lddw = lddw;
    a.accumulate = accumulate ? 1 : 0;
    a.transpose_out = transpose_out ? 1 : 0;
    a.ws = reinterpret_cast<char*>(ws);
    a.L = L;
    a.num_cus = num_cus();
    const hipError_t e = pamm::run_wgrad(a, dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PAMM_OK : PAMM_ERR_HIP;
}

int pamm_decompress(const void* C, const int32_t* f, const float* alpha, int64_t n, int64_t k, int64_t d, int dtype,
                    void* Xt, int64_t ldxt, void* stream) {
    if (!dtype_ok(dtype)) return PAMM_ERR_DTYPE;
    if (n < 0 || n > kMaxRows || k < 0 || k > n || k > PAMM_MAX_K || d < 1 || d > kMaxRows || ldxt < d ||
        !span_ok(n, ldxt, d))
        return PAMM_ERR_SHAPE;
    if (n == 0) return PAMM_OK;
    if (!f || !alpha || !Xt || (k > 0 && !C)) return PAMM_ERR_NULL;
    if (!aligned(f, 4) || !aligned(alpha, 4) || !aligned(Xt, 16) || ldxt % per16(dtype) != 0 ||
        (k > 0 && !aligned(C, 16)))
        return PAMM_ERR_ALIGN;
    pamm::DecompressArgs a;
    a.C = C;
    a.f = f;
    a.alpha = alpha;
    a.n = n;
    a.k = (int)k;
    a.d = d;
    a.Xt = Xt;
    a.ldxt_bytes = ldxt * elem_size(dtype);
    const hipError_t e = pamm::run_decompress(a, dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PAMM_OK : PAMM_ERR_HIP;
}

}  // extern "C"
