// pamm_wgrad.hip -- PAMM approximate weight gradient on gfx950.
//
// Implements the backward-pass phase of "QKV Projections Require a Fraction
// of Their Memory", section 2 "Metodologia", sub-part "Algoritmo in Due
// Fasi" (gradient approximation): the output-gradient rows of the tokens of
// each generator are summed with their alpha weights into a k x m matrix B~,
// and the weight gradient is approximated by C^T B~.
//
// Kernels, in stream order:
//   1. sort_hist       per block of 1024 rows: count of rows per generator.
//   2. sort_scatter    stable counting sort of the kept rows by generator:
//                      every block rebuilds the global segment offsets from
//                      the histograms (a few KB, L2-resident), ranks its rows
//                      with wave ballots and writes (row, alpha) in generator
//                      order; block 0 also cuts each generator's rows into
//                      chunks of at most kChunkRows rows.
//   3. scatter_reduce  one wave per (chunk, 128-byte column slab): sums
//                      alpha_i * dY[i, slab] over the chunk's rows, reading
//                      only kept rows, each 128-byte row piece by 8 lanes;
//                      writes the chunk's partial row P[chunk, slab] (fp32).
//                      Fixed summation order, no atomics: deterministic.
//   4. gen_gemm        dW = sum over chunks of c_gen(chunk) (x) P[chunk],
//                      i.e. C^T B~ with B~ split into its chunk partials.
//                      MFMA 32x32 tiles fed from LDS panels that are stored
//                      transposed (contraction index contiguous); bf16 uses
//                      a hi/lo bf16 split of P, fp32 uses fp32 MFMA.
// Dropped rows (f outside [0, k)) are never sorted, so their dY rows are not
// read at all.
#include <type_traits>

#include "pamm_device.hpp"
#include "pamm_kernels.hpp"

namespace pamm {

namespace {

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << __lane_id()) - 1ull; }

// Lanes of this wave whose value `v` equals this lane's (valid lanes only),
// by bit-slicing v over `nbits` ballots.
__device__ __forceinline__ uint64_t match_lanes(int v, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (v >> b) & 1;
        const uint64_t bm = __ballot(valid && bit);
        m &= bit ? bm : ~bm;
    }
    return m;
}

// Exclusive prefix sum over s[0..len) in LDS with a 256-thread block; returns
// the total.  `tmp` needs 256 ints of LDS.
__device__ int block_exclusive_scan(int* s, int len, int* tmp) {
    const int t = threadIdx.x;
    const int per = (len + 255) / 256;
    const int b = t * per, e = min(len, b + per);
    int sum = 0;
    for (int j = b; j < e; ++j) sum += s[j];
    tmp[t] = sum;
    __syncthreads();
    // Hillis-Steele over the 256 partial sums
    for (int off = 1; off < 256; off <<= 1) {
        const int v = t >= off ? tmp[t - off] : 0;
        __syncthreads();
        tmp[t] += v;
        __syncthreads();
    }
    const int total = tmp[255];
    int run = t > 0 ? tmp[t - 1] : 0;
    __syncthreads();
    for (int j = b; j < e; ++j) {
        const int v = s[j];
        s[j] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. per-block histogram of f
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sort_hist_kernel(const int32_t* __restrict__ f, int64_t n, int k,
                                                        int32_t* __restrict__ hist) {
    extern __shared__ int s_dyn[];
    int* cnt = s_dyn;
    for (int j = threadIdx.x; j < k; j += 256) cnt[j] = 0;
    __syncthreads();
    const int64_t r0 = (int64_t)blockIdx.x * kSortBlockRows;
    for (int r = threadIdx.x; r < kSortBlockRows; r += 256) {
        const int64_t i = r0 + r;
        if (i < n) {
            const int fi = f[i];
            if (fi >= 0 && fi < k) atomicAdd(&cnt[fi], 1);
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += 256) hist[(int64_t)blockIdx.x * k + j] = cnt[j];
}

// ---------------------------------------------------------------------------
// 2. stable counting-sort scatter (+ segment offsets and chunk list)
// ---------------------------------------------------------------------------
struct SortScatterArgs {
    const int32_t* f;
    const float* alpha;
    int64_t n;
    int k;
    int nbits;
    int64_t nb;
    const int32_t* hist;
    int32_t* seg_start;    // [k + 1]
    int32_t* nchunks;      // [1]
    int32_t* chunk_gen;    // [max_chunks]
    int32_t* chunk_begin;  // [max_chunks]
    int32_t* chunk_count;  // [max_chunks]
    int32_t* perm;         // [n]
    float* palpha;         // [n]
};

__global__ __launch_bounds__(256) void sort_scatter_kernel(SortScatterArgs a) {
    extern __shared__ int s_dyn[];
    const int k = a.k;
    int* s_tot = s_dyn;          // [k]   segment sizes, then segment starts
    int* s_base = s_dyn + k;     // [k]   rows of this generator in earlier blocks, then start of this block
    int* s_w = s_dyn + 2 * k;    // [4][k] per-wave counts, then per-wave running positions
    int* s_tmp = s_dyn + 6 * k;  // [256] scan scratch
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int64_t b = blockIdx.x;

    // segment sizes and the rows of each generator that precede this block
    for (int j = t; j < k; j += 256) {
        int tot = 0, pre = 0;
        for (int64_t bb = 0; bb < a.nb; ++bb) {
            const int h = a.hist[bb * k + j];
            tot += h;
            if (bb < b) pre += h;
        }
        s_tot[j] = tot;
        s_base[j] = pre;
    }
    for (int j = t; j < 4 * k; j += 256) s_w[j] = 0;
    __syncthreads();

    // block 0 cuts every generator's rows into chunks (before s_tot becomes starts)
    if (b == 0) {
        int* s_nch = s_w;  // reuse: per-generator chunk count -> chunk offset
        for (int j = t; j < k; j += 256) s_nch[j] = (s_tot[j] + kChunkRows - 1) / kChunkRows;
        __syncthreads();
        const int total_chunks = block_exclusive_scan(s_nch, k, s_tmp);
        if (t == 0) *a.nchunks = total_chunks;
        __syncthreads();
        // chunk rows are laid out after the segment starts, computed below;
        // stash the offsets in s_tmp-free form: keep s_nch until starts are known
    }

    const int total_rows = block_exclusive_scan(s_tot, k, s_tmp);  // s_tot := segment starts
    if (b == 0) {
        for (int j = t; j < k; j += 256) a.seg_start[j] = s_tot[j];
        if (t == 0) a.seg_start[k] = total_rows;
        const int* s_nch = s_w;
        for (int j = t; j < k; j += 256) {
            const int start = s_tot[j];
            const int size = (j + 1 < k ? s_tot[j + 1] : total_rows) - start;
            const int c0 = s_nch[j];
            for (int c = 0; c * kChunkRows < size; ++c) {
                a.chunk_gen[c0 + c] = j;
                a.chunk_begin[c0 + c] = start + c * kChunkRows;
                a.chunk_count[c0 + c] = min(kChunkRows, size - c * kChunkRows);
            }
        }
        __syncthreads();
        for (int j = t; j < 4 * k; j += 256) s_w[j] = 0;
        __syncthreads();
    }
    for (int j = t; j < k; j += 256) s_base[j] += s_tot[j];  // first position of this block's rows
    __syncthreads();

    // per-wave counts over the wave's 256 rows
    const int64_t r0 = b * kSortBlockRows + wave * 256;
    int fv[4];
    bool ok[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
        const int64_t i = r0 + sub * 64 + lane;
        const int fi = i < a.n ? a.f[i] : -1;
        ok[sub] = fi >= 0 && fi < k;
        fv[sub] = ok[sub] ? fi : 0;
        if (ok[sub]) atomicAdd(&s_w[wave * k + fi], 1);
    }
    __syncthreads();
    // running position of each wave := block start + counts of earlier waves
    for (int j = t; j < k; j += 256) {
        int run = s_base[j];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int c = s_w[w * k + j];
            s_w[w * k + j] = run;
            run += c;
        }
    }
    __syncthreads();
    // rank rows within the wave in row order and scatter
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
        const int64_t i = r0 + sub * 64 + lane;
        const uint64_t m = match_lanes(fv[sub], ok[sub], a.nbits);
        if (ok[sub]) {
            const int rank = __popcll(m & lanemask_lt());
            const int pos = s_w[wave * k + fv[sub]] + rank;
            a.perm[pos] = (int32_t)i;
            a.palpha[pos] = a.alpha[i];
        }
        // all lanes have read the running position; the lowest lane of each
        // group advances it (LDS accesses of one wave stay in program order)
        if (ok[sub] && (m & lanemask_lt()) == 0) s_w[wave * k + fv[sub]] += __popcll(m);
    }
}

// ---------------------------------------------------------------------------
// 3. alpha-weighted segmented reduction over kept rows
// ---------------------------------------------------------------------------
struct ScatterArgs {
    const char* dY;
    int64_t lddy_bytes;
    int64_t d_out;
    int64_t nslab;  // column slabs of 128 bytes
    const int32_t* nchunks;
    const int32_t* chunk_begin;
    const int32_t* chunk_count;
    const int32_t* perm;
    const float* palpha;
    float* P;
    int64_t ldp;
};

template <int DT>
__global__ __launch_bounds__(256) void scatter_reduce_kernel(ScatterArgs a) {
    constexpr int PE = Elem<DT>::per16;   // elements per lane
    constexpr int SC = 8 * PE;            // columns per slab (128 bytes)
    constexpr int U = 8;                  // rows in flight per lane group
    const int lane = threadIdx.x & 63;
    const int g = lane >> 3, l8 = lane & 7;
    const int64_t nitems = (int64_t)(*a.nchunks) * a.nslab;
    const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); item < nitems;
         item += wstride) {
        const int64_t ch = item / a.nslab;
        const int64_t col = (item % a.nslab) * SC + l8 * PE;
        const int begin = a.chunk_begin[ch];
        const int cnt = a.chunk_count[ch];
        float acc[PE];
#pragma unroll
        for (int e = 0; e < PE; ++e) acc[e] = 0.f;
        for (int t0 = g; t0 < cnt; t0 += 8 * U) {
            int ii[U];
            float aa[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tt = t0 + 8 * u;
                ii[u] = tt < cnt ? a.perm[begin + tt] : -1;
                aa[u] = tt < cnt ? a.palpha[begin + tt] : 0.f;
            }
            uint4 vv[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                vv[u] = ii[u] >= 0 ? load16_tail<DT>(a.dY + (int64_t)ii[u] * a.lddy_bytes, col, a.d_out)
                                   : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float v[PE];
                unpack16<DT>(vv[u], v);
#pragma unroll
                for (int e = 0; e < PE; ++e) acc[e] = __builtin_fmaf(aa[u], v[e], acc[e]);
            }
        }
        // fixed-order combine of the 8 row groups
#pragma unroll
        for (int m = 8; m < 64; m <<= 1)
#pragma unroll
            for (int e = 0; e < PE; ++e) acc[e] += shfl_xor(acc[e], m);
        if (g == 0) {
            float* dst = a.P + ch * a.ldp + col;
            if (col + PE <= a.d_out) {
#pragma unroll
                for (int e = 0; e < PE; e += 4)
                    *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
            } else {
                for (int e = 0; e < PE; ++e)
                    if (col + e < a.d_out) dst[e] = acc[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 4. generator product dW = sum_chunk c_gen(chunk) (x) P[chunk]
// ---------------------------------------------------------------------------
struct GemmArgs {
    const void* C;  // [k x d]
    int64_t d;
    int64_t d_out;
    const int32_t* nchunks;
    const int32_t* chunk_gen;
    const float* P;
    int64_t ldp;
    float* dW;
    int64_t lddw;
    int accumulate;
};

namespace {
constexpr int kGBM = 128;  // dW rows (d) per workgroup
constexpr int kGBN = 128;  // dW columns (d_out) per workgroup
constexpr int kGKP = 32;   // chunks per LDS panel
}  // namespace

template <int DT>
__global__ __launch_bounds__(256) void gen_gemm_kernel(GemmArgs a) {
    // LDS panels stored transposed: [row of the tile][chunk], chunk contiguous.
    constexpr int KPAD = DT == DT_BF16 ? kGKP + 8 : kGKP + 4;  // padded row length (elements)
    typedef typename std::conditional<DT == DT_BF16, uint16_t, float>::type T;
    __shared__ __align__(16) T sA[kGBM * KPAD];
    __shared__ __align__(16) T sBh[kGBN * KPAD];
    __shared__ __align__(16) T sBl[DT == DT_BF16 ? kGBN * KPAD : 8];

    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int64_t m0 = (int64_t)blockIdx.y * kGBM;
    const int64_t n0 = (int64_t)blockIdx.x * kGBN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int nch = *a.nchunks;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    for (int kp = 0; kp < nch; kp += kGKP) {
        __syncthreads();
        // ---- A panel: sA[m][kk] = C[gen(kp+kk)][m0+m]
        {
            constexpr int PE = Elem<DT>::per16;
            constexpr int MCH = kGBM / PE;        // 16-byte pieces per panel row of C
            for (int c = t; c < kGKP * MCH; c += 256) {
                const int kk = c % kGKP, mc = c / kGKP;
                const int64_t m = m0 + mc * PE;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (kp + kk < nch && m < a.d) {
                    const int gj = a.chunk_gen[kp + kk];
                    v = load16_tail<DT>(reinterpret_cast<const char*>(a.C) + (int64_t)gj * a.d * Elem<DT>::size, m,
                                        a.d);
                }
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < PE; ++e) {
                    if constexpr (DT == DT_BF16)
                        sA[(mc * PE + e) * KPAD + kk] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    else
                        sA[(mc * PE + e) * KPAD + kk] = __uint_as_float(w[e]);
                }
            }
        }
        // ---- B panel: P[kp+kk][n0+n] -> sBh/sBl[n][kk]
        {
            constexpr int NCH = kGBN / 4;
            for (int c = t; c < kGKP * NCH; c += 256) {
                const int kk = c % kGKP, nc = c / kGKP;
                const int64_t nn = n0 + nc * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (kp + kk < nch && nn < a.d_out) {
                    const float* src = a.P + (int64_t)(kp + kk) * a.ldp + nn;
                    if (nn + 4 <= a.d_out) {
                        v = *reinterpret_cast<const float4*>(src);
                    } else {
                        float tmp[4] = {0.f, 0.f, 0.f, 0.f};
                        for (int e = 0; e < 4; ++e)
                            if (nn + e < a.d_out) tmp[e] = src[e];
                        v = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
                    }
                }
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (DT == DT_BF16) {
                        const uint32_t hi = f32_to_bf16(vv[e]);
                        const uint32_t lo = f32_to_bf16(vv[e] - __uint_as_float(hi << 16));
                        sBh[(nc * 4 + e) * KPAD + kk] = (uint16_t)hi;
                        sBl[(nc * 4 + e) * KPAD + kk] = (uint16_t)lo;
                    } else {
                        sBh[(nc * 4 + e) * KPAD + kk] = vv[e];
                    }
                }
            }
        }
        __syncthreads();
        // ---- MFMA over the panel
#pragma unroll
        for (int ks = 0; ks < kGKP; ks += 16) {
            if constexpr (DT == DT_BF16) {
                const int kq = ks + (lane >> 5) * 8;
                bf16x8 af[2], bh[2], bl[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    af[i] = *reinterpret_cast<const bf16x8*>(&sA[(wm + i * 32 + (lane & 31)) * KPAD + kq]);
                    bh[i] = *reinterpret_cast<const bf16x8*>(&sBh[(wn + i * 32 + (lane & 31)) * KPAD + kq]);
                    bl[i] = *reinterpret_cast<const bf16x8*>(&sBl[(wn + i * 32 + (lane & 31)) * KPAD + kq]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bh[j], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bl[j], acc[i][j], 0, 0, 0);
                    }
            } else {
                // lane group (lane/32) holds chunks ks + 8*(lane/32) + 0..7; MFMA s uses element s
                const int kq = ks + (lane >> 5) * 8;
                float4 af[2][2], bf[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        af[i][h] = *reinterpret_cast<const float4*>(&sA[(wm + i * 32 + (lane & 31)) * KPAD + kq + 4 * h]);
                        bf[i][h] = *reinterpret_cast<const float4*>(&sBh[(wn + i * 32 + (lane & 31)) * KPAD + kq + 4 * h]);
                    }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][h].x, bf[j][h].x, acc[i][j], 0, 0, 0);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][h].y, bf[j][h].y, acc[i][j], 0, 0, 0);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][h].z, bf[j][h].z, acc[i][j], 0, 0, 0);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][h].w, bf[j][h].w, acc[i][j], 0, 0, 0);
                        }
            }
        }
    }

    // ---- store: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32 of a 32x32 tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < a.d && col < a.d_out) {
                    float* p = a.dW + row * a.lddw + col;
                    const float v = acc[i][j][e];
                    if (a.accumulate) *p = *p + v;
                    else __builtin_nontemporal_store(v, p);
                }
            }
        }
}

__global__ void zero_count_kernel(int32_t* c) {
    if (threadIdx.x == 0) *c = 0;
}

// ---------------------------------------------------------------------------
// host-side launcher
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WgradLayout wgrad_layout(int64_t n, int64_t k, int64_t d_out) {
    WgradLayout L;
    L.nb = (n + kSortBlockRows - 1) / kSortBlockRows;
    if (L.nb < 1) L.nb = 1;
    L.max_chunks = (n + kChunkRows - 1) / kChunkRows + k;
    L.ldp = (d_out + 7) & ~(int64_t)7;
    size_t off = 0;
    L.off_hist = off; off = align256(off + sizeof(int32_t) * (size_t)(L.nb * (k > 0 ? k : 1)));
    L.off_seg = off; off = align256(off + sizeof(int32_t) * (size_t)(k + 1));
    L.off_nchunks = off; off = align256(off + sizeof(int32_t));
    L.off_chunk_gen = off; off = align256(off + sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_chunk_begin = off; off = align256(off + sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_chunk_count = off; off = align256(off + sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_perm = off; off = align256(off + sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    L.off_palpha = off; off = align256(off + sizeof(float) * (size_t)(n > 0 ? n : 1));
    L.off_P = off; off = align256(off + sizeof(float) * (size_t)(L.max_chunks * L.ldp));
    L.total = off;
    return L;
}

template <int DT>
static hipError_t wgrad_impl(const WgradArgs& a, hipStream_t st) {
    const WgradLayout& L = a.L;
    char* ws = a.ws;
    int32_t* hist = reinterpret_cast<int32_t*>(ws + L.off_hist);
    int32_t* seg = reinterpret_cast<int32_t*>(ws + L.off_seg);
    int32_t* nchunks = reinterpret_cast<int32_t*>(ws + L.off_nchunks);
    int32_t* cgen = reinterpret_cast<int32_t*>(ws + L.off_chunk_gen);
    int32_t* cbeg = reinterpret_cast<int32_t*>(ws + L.off_chunk_begin);
    int32_t* ccnt = reinterpret_cast<int32_t*>(ws + L.off_chunk_count);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.off_perm);
    float* palpha = reinterpret_cast<float*>(ws + L.off_palpha);
    float* P = reinterpret_cast<float*>(ws + L.off_P);
    const int k = a.k;

    if (k > 0 && a.n > 0) {
        hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)L.nb), dim3(256), sizeof(int) * k, st, a.f, a.n, k, hist);
        SortScatterArgs s;
        s.f = a.f; s.alpha = a.alpha; s.n = a.n; s.k = k;
        int nbits = 0;
        while ((1 << nbits) < k) ++nbits;
        s.nbits = nbits;
        s.nb = L.nb; s.hist = hist; s.seg_start = seg; s.nchunks = nchunks;
        s.chunk_gen = cgen; s.chunk_begin = cbeg; s.chunk_count = ccnt; s.perm = perm; s.palpha = palpha;
        const size_t lds = sizeof(int) * (6 * (size_t)k + 256);
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sort_scatter_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)L.nb), dim3(256), lds, st, s);

        ScatterArgs r;
        r.dY = reinterpret_cast<const char*>(a.dY);
        r.lddy_bytes = a.lddy_bytes;
        r.d_out = a.d_out;
        constexpr int SC = 8 * Elem<DT>::per16;
        r.nslab = (a.d_out + SC - 1) / SC;
        r.nchunks = nchunks; r.chunk_begin = cbeg; r.chunk_count = ccnt; r.perm = perm; r.palpha = palpha;
        r.P = P; r.ldp = L.ldp;
        const int64_t max_items = L.max_chunks * r.nslab;
        int64_t grid = (max_items + 3) / 4;
        const int64_t cap = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * 8;
        if (grid > cap) grid = cap;
        if (grid < 1) grid = 1;
        hipLaunchKernelGGL(scatter_reduce_kernel<DT>, dim3((unsigned)grid), dim3(256), 0, st, r);
    } else {
        // no generators or no rows: no chunks, dW = 0 (or unchanged when accumulating)
        hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, st, nchunks);
    }

    GemmArgs g;
    g.C = a.C; g.d = a.d; g.d_out = a.d_out; g.nchunks = nchunks; g.chunk_gen = cgen; g.P = P; g.ldp = L.ldp;
    g.dW = a.dW; g.lddw = a.lddw; g.accumulate = a.accumulate;
    dim3 grid((unsigned)((a.d_out + kGBN - 1) / kGBN), (unsigned)((a.d + kGBM - 1) / kGBM));
    hipLaunchKernelGGL(gen_gemm_kernel<DT>, grid, dim3(256), 0, st, g);
    return hipGetLastError();
}

hipError_t run_wgrad(const WgradArgs& a, int dtype, hipStream_t st) {
    return dtype == DT_BF16 ? wgrad_impl<DT_BF16>(a, st) : wgrad_impl<DT_F32>(a, st);
}

}  // namespace pamm
