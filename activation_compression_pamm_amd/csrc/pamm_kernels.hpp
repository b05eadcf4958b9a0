// pamm_kernels.hpp -- argument blocks and launchers of the PAMM kernels.
// Host code validates everything before calling a launcher; launchers only
// enqueue work on the given stream and report hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pamm {

// Generators handled by one compress workgroup; larger k is split into tiles
// whose winners are merged.
constexpr int kMaxTileGens = 256;
// Rows of one chunk of a generator's row list in the wgrad scatter-reduce:
// kMaxChunkRows, halved down to kMinChunkRows while the upper bound on
// (chunk, 64-column slab) items stays below kFillItems (the waves a full
// device holds), so that small problems still spread over the device.
constexpr int kMaxChunkRows = 256;
constexpr int kMinChunkRows = 64;
constexpr int64_t kFillItems = 8192;
// Rows handled by one block of the wgrad counting sort.
constexpr int kSortBlockRows = 1024;
// Above this many histogram entries (sort blocks x generators) the histogram
// is prefixed once instead of being summed by every sort block.
constexpr int64_t kSortPrefixEntries = 8192;

struct PartialBest {
    float score;  // best |<x,c>|/|c| in the tile, -1 if none
    int32_t gen;  // its generator slot, -1 if none
    float alpha;  // <x,c>/|c|^2 for it
};

struct CompressArgs {
    const void* X;
    int64_t n, d;
    int64_t ldx_bytes;  // leading dimension of X in bytes
    int64_t row_bytes;  // d * element size
    const int32_t* gen_idx;
    int k;
    float eps;
    void* C;       // [k x d] output (may be null: not written)
    int c_vec_ok;  // C rows are 16-byte aligned
    int32_t* f;
    float* alpha;
    PartialBest* partial;  // [ntiles x n] when k > kMaxTileGens
    float* xn2;            // [n] when k > kMaxTileGens
    float* cn2;            // [k] |c_j|^2, bf16 with k > kMaxTileGens / 2 (the GEMM-shaped path)
    int ntiles;            // generator tiles (set by the launcher)
    int num_cus;           // compute units of the device
    // the forward projection computed in the same pass (pamm_forward_compress;
    // all zero for pamm_compress): Y [n x d_out] = X W^T (+ bias), bf16
    const void* W;         // [d_out x d], rows ldw_bytes apart
    int64_t ldw_bytes;
    int64_t d_out;
    void* Y;               // [n x d_out], rows ldy_bytes apart
    int64_t ldy_bytes;
    const void* bias;      // [d_out] or null
    int tiles_w;           // 256-column tiles of Y
};

hipError_t run_compress(const CompressArgs& a, int dtype, hipStream_t st);
// Y = X W^T (+ bias) and the compression of X in one pass (bf16 only).
hipError_t run_forward_compress(const CompressArgs& a, hipStream_t st);

// Workspace carve-up of pamm_wgrad (all offsets 256-byte aligned).
struct WgradLayout {
    int64_t nb;         // sort blocks
    int chunk_rows;     // rows per chunk (a generator's last chunk may hold fewer)
    int64_t max_chunks; // upper bound on row chunks
    size_t off_hist, off_tot, off_nchunks, off_chunk_gen, off_chunk_begin, off_chunk_count;
    size_t off_perm, off_palpha, off_AT, off_BT;
    int64_t ks_cap;     // 16-chunk contraction steps the product operands hold
    size_t total;
};

WgradLayout wgrad_layout(int64_t n, int64_t k, int64_t d, int64_t d_out);

struct WgradArgs {
    const void* C;
    const int32_t* f;
    const float* alpha;
    int64_t n;
    int k;
    int64_t d;
    const void* dY;
    int64_t d_out;
    int64_t lddy_bytes;
    float* dW;              // [d x d_out], or [d_out x d] when transpose_out
    int64_t lddw;
    int accumulate;
    int transpose_out;
    char* ws;
    WgradLayout L;
    int num_cus;
};

hipError_t run_wgrad(const WgradArgs& a, int dtype, hipStream_t st);

// Argument checks of pamm_wgrad apart from the workspace (a pamm_status_t).
int wgrad_check(const void* C, const int32_t* f, const float* alpha, int64_t n, int64_t k, int64_t d, const void* dY,
                int64_t d_out, int64_t lddy, int dtype, const float* dW, int64_t lddw, int transpose_out);

struct DecompressArgs {
    const void* C;
    const int32_t* f;
    const float* alpha;
    int64_t n;
    int k;
    int64_t d;
    void* Xt;
    int64_t ldxt_bytes;
};

hipError_t run_decompress(const DecompressArgs& a, int dtype, hipStream_t st);

}  // namespace pamm
