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
//   1'. sort_prefix    only when the histogram is large (blocks x generators
//                      above kSortPrefixEntries): turns it in place into
//                      per-block prefixes along the blocks plus segment sizes.
//   2. sort_scatter    stable counting sort of the kept rows by generator:
//                      every block rebuilds the global segment offsets from
//                      the histograms (a few KB, L2-resident) or reads its
//                      prefixes, ranks its rows with wave ballots and writes
//                      (row, alpha) in generator order; block 0 also cuts
//                      each generator's rows into chunks of at most
//                      chunk_rows rows (chosen with the workspace layout).
//   3. scatter_reduce  gathers the product's A operand (each chunk's
//                      generator row of C, in MFMA fragment order), then
//                      one wave per (chunk, 128-byte column slab): sums
//                      alpha_i * dY[i, slab] over the chunk's rows, reading
//                      only kept rows, each 128-byte row piece by 8 lanes,
//                      and writes the chunk's partial row P[chunk, slab]
//                      (fp32) straight into the product's B operand.
//                      With few rows per generator a wave item is a pair
//                      of chunks, one per half of the row groups.
//                      Fixed summation order, no atomics: deterministic.
//   4. gen_gemm        dW = sum over chunks of c_gen(chunk) (x) P[chunk],
//                      i.e. C^T B~ with B~ split into its chunk partials.
//                      MFMA 32x32 tiles fed by contiguous fragment loads,
//                      no LDS; bf16 uses a hi/lo bf16 split of P, fp32 uses
//                      fp32 MFMA.
// Dropped rows (f outside [0, k)) are never sorted, so their dY rows are not
// read at all.
#include <type_traits>

#include "pamm_device.hpp"
#include "pamm_kernels.hpp"

// segmented reduction: lanes per row piece, rows in flight per row group
#ifndef PAMM_SR_LPR
#define PAMM_SR_LPR 8
#endif
#ifndef PAMM_SR_U
#define PAMM_SR_U 8
#endif
// with full-length chunks, generators averaging at most this many rows (n / k,
// as if every row were kept) get paired reduction items: two chunks per item
#ifndef PAMM_SR_PAIR_ROWS
#define PAMM_SR_PAIR_ROWS 128
#endif
// dW tile of one wave: 32*TM rows x 32*TN columns (32*TN_WIDE columns from
// kWideProductK generators on)
#ifndef PAMM_GEMM_TM
#define PAMM_GEMM_TM 2
#endif
#ifndef PAMM_GEMM_TN
#define PAMM_GEMM_TN 1
#endif
#ifndef PAMM_GEMM_TN_WIDE
#define PAMM_GEMM_TN_WIDE 2
#endif

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

// Compiler-only memory barrier: loads issued before it stay before it (the
// compiler would otherwise sink a prefetch into the iteration that uses it);
// it emits no instruction and no wait.
__device__ __forceinline__ void pin_issued_loads() { asm volatile("" ::: "memory"); }

// Exclusive prefix sum over s[0..len) in LDS with a 256-thread block; returns
// the total.  Each thread sums a run of `per` entries; the 256 run sums are
// scanned with shuffles inside each wave and across the four wave totals.
// `tmp` needs 4 ints of LDS.
__device__ int block_exclusive_scan(int* s, int len, int* tmp) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int per = (len + 255) / 256;
    const int b = min(len, t * per), e = min(len, b + per);
    int sum = 0;
    for (int j = b; j < e; ++j) sum += s[j];
    int inc = sum;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
    }
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    int run = inc - sum, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int x = tmp[w];
        if (w < wave) run += x;
        total += x;
    }
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
    // all of this thread's rows are loaded first: their latency overlaps the
    // clearing of the bins, and none is counted before all have arrived
    const int64_t r0 = (int64_t)blockIdx.x * kSortBlockRows;
    int fv[kSortBlockRows / 256];
#pragma unroll
    for (int u = 0; u < kSortBlockRows / 256; ++u) {
        const int64_t i = r0 + u * 256 + threadIdx.x;
        fv[u] = i < n ? f[i] : -1;
    }
    for (int j = threadIdx.x; j < k; j += 256) cnt[j] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSortBlockRows / 256; ++u)
        if (fv[u] >= 0 && fv[u] < k) atomicAdd(&cnt[fv[u]], 1);
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += 256) hist[(int64_t)blockIdx.x * k + j] = cnt[j];
}

// 1'. when the histogram is large (many blocks x many generators): turn it,
// in place, into per-block exclusive prefixes along the blocks, and write the
// segment sizes, so that each sort block reads 2k numbers instead of nb*k.
// 64 generators per workgroup, the blocks split into 4 ranges, one per wave.
__global__ __launch_bounds__(256) void sort_prefix_kernel(int32_t* __restrict__ hist, int64_t nb, int k,
                                                          int32_t* __restrict__ totals) {
    constexpr int B = 16;  // histogram rows loaded together
    __shared__ int s_sum[4][64];
    const int c = threadIdx.x & 63, seg = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + c;
    const int64_t len = (nb + 3) / 4, r0 = min(nb, seg * len), r1 = min(nb, r0 + len);
    const int jj = min(j, k - 1);  // lanes past k read a valid column, write nothing
    int sum = 0;
    for (int64_t b0 = r0; b0 < r1; b0 += B) {
        int h[B];
#pragma unroll
        for (int u = 0; u < B; ++u) h[u] = b0 + u < r1 ? hist[(b0 + u) * k + jj] : 0;
#pragma unroll
        for (int u = 0; u < B; ++u) sum += h[u];
    }
    s_sum[seg][c] = sum;
    __syncthreads();
    int run = 0;
    for (int w = 0; w < seg; ++w) run += s_sum[w][c];
    if (seg == 3 && j < k) totals[j] = run + sum;
    for (int64_t b0 = r0; b0 < r1; b0 += B) {
        int h[B];
#pragma unroll
        for (int u = 0; u < B; ++u) h[u] = b0 + u < r1 ? hist[(b0 + u) * k + jj] : 0;
#pragma unroll
        for (int u = 0; u < B; ++u) {
            if (b0 + u < r1 && j < k) hist[(b0 + u) * k + j] = run;
            run += h[u];
        }
    }
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
    int chunk_rows;
    int64_t nb;
    const int32_t* hist;   // [nb][k] per-block counts, or (PREFIXED) exclusive prefixes along the blocks
    const int32_t* totals; // [k] segment sizes (PREFIXED only)
    int32_t* nchunks;      // [1]
    int32_t* chunk_gen;    // [max_chunks]
    int32_t* chunk_begin;  // [max_chunks]
    int32_t* chunk_count;  // [max_chunks]
    int32_t* perm;         // [n]
    float* palpha;         // [n]
};

template <bool PREFIXED>
__global__ __launch_bounds__(256) void sort_scatter_kernel(SortScatterArgs a) {
    extern __shared__ int s_dyn[];
    const int k = a.k;
    int* s_tot = s_dyn;          // [k]   segment sizes, then segment starts
    int* s_base = s_dyn + k;     // [k]   rows of this generator in earlier blocks
    int* s_w = s_dyn + 2 * k;    // [4][k] per-wave counts, then per-wave running positions
    int* s_tmp = s_dyn + 6 * k;  // [256] scan scratch
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int64_t b = blockIdx.x;

    // this thread's rows: issue their f and alpha loads first so they overlap
    // the histogram reads below
    const int64_t r0 = b * kSortBlockRows + wave * 256;
    int fv[4];
    float av[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
        const int64_t i = r0 + sub * 64 + lane;
        fv[sub] = i < a.n ? a.f[i] : -1;
        av[sub] = i < a.n ? a.alpha[i] : 0.f;
    }

    // segment sizes and the rows of each generator that precede this block:
    // read from the prefixed histogram, or, for a small histogram, summed
    // here from all of it with coalesced, independent loads and LDS integer
    // atomics (exact, so the order does not matter)
    if constexpr (PREFIXED) {
        for (int j = t; j < 4 * k; j += 256) s_w[j] = 0;
        for (int j = t; j < k; j += 256) {
            s_tot[j] = a.totals[j];
            s_base[j] = a.hist[b * k + j];
        }
        __syncthreads();
    } else {
        // column sums of the histogram: R threads share a generator column
        // (R = 256 / k for k < 256, else 1), thread t summing the blocks
        // t / k, t / k + R, ... with HB loads issued before any add; the R
        // partial sums meet in LDS integer atomics (exact, in any order)
        constexpr int HB = 16;
        const int R = k >= 256 ? 1 : 256 / k;
        const int r = k >= 256 ? 0 : t / k;
        for (int j = t; j < 4 * k; j += 256) s_w[j] = 0;
        for (int j = t; j < k; j += 256) { s_tot[j] = 0; s_base[j] = 0; }
        __syncthreads();
        if (r < R) {
            for (int j = k >= 256 ? t : t % k; j < k; j += 256) {
                int tot = 0, pre = 0;
                for (int64_t b0 = r; b0 < a.nb; b0 += (int64_t)R * HB) {
                    int hv[HB];
#pragma unroll
                    for (int u = 0; u < HB; ++u) {
                        const int64_t bb = b0 + (int64_t)u * R;
                        hv[u] = bb < a.nb ? a.hist[bb * k + j] : 0;
                    }
#pragma unroll
                    for (int u = 0; u < HB; ++u) {
                        tot += hv[u];
                        if (b0 + (int64_t)u * R < b) pre += hv[u];
                    }
                }
                if (tot) atomicAdd(&s_tot[j], tot);
                if (pre) atomicAdd(&s_base[j], pre);
            }
        }
        __syncthreads();
    }

    // block 0 cuts every generator's rows into chunks (before s_tot becomes starts)
    if (b == 0) {
        int* s_nch = s_w;  // reuse: per-generator chunk count -> first chunk
        for (int j = t; j < k; j += 256) s_nch[j] = (s_tot[j] + a.chunk_rows - 1) / a.chunk_rows;
        __syncthreads();
        const int total_chunks = block_exclusive_scan(s_nch, k, s_tmp);
        if (t == 0) *a.nchunks = total_chunks;
        __syncthreads();
    }

    const int total_rows = block_exclusive_scan(s_tot, k, s_tmp);  // s_tot := segment starts
    if (b == 0) {
        const int* s_nch = s_w;
        for (int j = t; j < k; j += 256) {
            const int start = s_tot[j];
            const int size = (j + 1 < k ? s_tot[j + 1] : total_rows) - start;
            const int c0 = s_nch[j];
            for (int c = 0; c * a.chunk_rows < size; ++c) {
                a.chunk_gen[c0 + c] = j;
                a.chunk_begin[c0 + c] = start + c * a.chunk_rows;
                a.chunk_count[c0 + c] = min(a.chunk_rows, size - c * a.chunk_rows);
            }
        }
        __syncthreads();
        for (int j = t; j < 4 * k; j += 256) s_w[j] = 0;
        __syncthreads();
    }
    // per-wave counts over the wave's 256 rows
    bool ok[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
        const int fi = fv[sub];
        ok[sub] = fi >= 0 && fi < k;
        fv[sub] = ok[sub] ? fi : 0;
        if (ok[sub]) atomicAdd(&s_w[wave * k + fi], 1);
    }
    __syncthreads();
    // running position of each wave := segment start + rows of earlier
    // blocks + counts of earlier waves
    for (int j = t; j < k; j += 256) {
        int run = s_tot[j] + s_base[j];
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
            a.palpha[pos] = av[sub];
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
    const int32_t* chunk_gen;
    const void* C;    // [k x d]
    int64_t d;
    void* AF;         // product operand A, MFMA-fragment order
    void* BF;         // product operand B, MFMA-fragment order
    int64_t ks_cap;   // contraction steps BF holds
    int64_t ncols;    // columns BF holds: d_out rounded up to 32
};

// The product's operands are stored in MFMA-fragment order, so that every
// fragment a wave of gen_gemm needs is one contiguous 1 KB (64 lanes x 16
// bytes) load.  For 32-row block mb (rows of dW, i.e. d) or 32-column block
// nb (d_out) and contraction step ks (16 chunks):
//   bf16: lane l, piece 0:  A[32mb + l%32][16ks + 8(l/32) + 0..7]
//   fp32: lane l, piece h:  A[32mb + l%32][16ks + 8h + 4(l/32) + 0..3]
// with A[m][kk] = C[gen(kk)][m] and B[n][kk] = P[kk][n] (bf16: P split into
// hi + lo bf16 terms, B holding all hi blocks, then all lo blocks); entries
// past d or the chunk count are zero.
//
// One A slot (1 KB) per wave: lane l gathers its 16 bytes from C.
template <int DT>
__device__ __forceinline__ void write_a_slot(const ScatterArgs& a, int64_t slot, int ks_used, int nch, int lane) {
    constexpr int PIECES = DT == DT_BF16 ? 1 : 2;
    typedef typename std::conditional<DT == DT_BF16, uint16_t, float>::type T;
    constexpr int PE = 16 / (int)sizeof(T);
    const int piece = (int)(slot % PIECES);
    const int64_t ks = (slot / PIECES) % ks_used;
    const int64_t mb = (slot / PIECES) / ks_used;
    const int64_t m = mb * 32 + (lane & 31);
    const int kk0 = (int)(ks * 16) + (DT == DT_BF16 ? 8 * (lane >> 5) : 8 * piece + 4 * (lane >> 5));
    const T* C = reinterpret_cast<const T*>(a.C);
    T v[PE];
#pragma unroll
    for (int e = 0; e < PE; ++e) {
        const int kk = kk0 + e;
        v[e] = (kk < nch && m < a.d) ? C[(int64_t)a.chunk_gen[kk] * a.d + m] : T(0);
    }
    reinterpret_cast<uint4*>(a.AF)[((mb * a.ks_cap + ks) * PIECES + piece) * 64 + lane] =
        *reinterpret_cast<uint4*>(v);
}

// Items: first the A slots, then one per (chunk, column slab).  For the
// latter LPR lanes cover one row piece of 16*LPR bytes (whole 128-byte
// lines), 64/LPR row groups walk the chunk's rows, U rows per group in
// flight.  PAIR (for short chunks): an item is a pair of consecutive chunks
// at one slab, each half of the wave's row groups walking one of them, so
// that an item still gathers up to 64 rows at once.
template <int DT, int LPR, int U, bool PAIR>
__global__ __launch_bounds__(256) void scatter_reduce_kernel(ScatterArgs a) {
    constexpr int PE = Elem<DT>::per16;   // elements per lane
    constexpr int SC = LPR * PE;          // columns per slab
    constexpr int RG = 64 / LPR;          // row groups per wave
    constexpr int HALVES = PAIR ? 2 : 1;  // chunks per item
    constexpr int RGH = RG / HALVES;      // row groups per chunk
    constexpr int BR = RGH * U;           // rows of a chunk per batch
    const int lane = threadIdx.x & 63;
    const int g = lane / LPR, lq = lane % LPR;
    const int h = g / RGH, gh = g % RGH;  // chunk of the item, row group in it
    // chunks up to the next multiple of 16 are written too (as zeros), so
    // the product's last contraction step holds no stale workspace
    const int nch = *a.nchunks;
    const int ks_used = (nch + 15) >> 4;
    const int64_t a_slots = (a.d + 31) / 32 * ks_used * (DT == DT_BF16 ? 1 : 2);
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t slot = wave; slot < a_slots; slot += wstride) write_a_slot<DT>(a, slot, ks_used, nch, lane);

    // one batch is the 64 rows the wave's row groups take together
    static_assert(RG * U == 64, "a batch is 64 rows");
    static_assert(!PAIR || (RG == 8 && PE >= 4), "paired items: 8 row groups, 4 or 8 columns per lane");
    const int64_t nitems = (int64_t)ks_used * (16 / HALVES) * a.nslab;
    auto meta = [&](int64_t it, int& bg, int& cn) {
        const int64_t c = it / a.nslab * HALVES + h;
        bg = c < nch ? a.chunk_begin[c] : 0;
        cn = c < nch ? a.chunk_count[c] : 0;
    };
    auto row_ids = [&](int bg, int cn, int t0, int* ii) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t0 + RGH * u;
            ii[u] = tt < cn ? a.perm[bg + tt] : -1;
        }
    };
    auto row_alphas = [&](int bg, int cn, int t0, float* aa) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t0 + RGH * u;
            aa[u] = tt < cn ? a.palpha[bg + tt] : 0.f;
        }
    };
    // dY pieces of rows ii at the item's column slab (read once: non-temporal
    // loads of whole 16-byte groups)
    auto fetch = [&](int64_t it, const int* ii, uint4* vv) __attribute__((always_inline)) {
        const int64_t col = (it % a.nslab) * SC + lq * PE;
#pragma unroll
        for (int u = 0; u < U; ++u)
            vv[u] = ii[u] < 0 ? make_uint4(0, 0, 0, 0)
                    : (col + PE <= a.d_out
                           ? load16_nt(a.dY + (int64_t)ii[u] * a.lddy_bytes + col * Elem<DT>::size)
                           : load16_tail<DT>(a.dY + (int64_t)ii[u] * a.lddy_bytes, col, a.d_out));
    };
    auto accumulate = [&](const uint4* vv, const float* aa, float* acc) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[PE];
            unpack16<DT>(vv[u], v);
#pragma unroll
            for (int e = 0; e < PE; ++e) acc[e] = __builtin_fmaf(aa[u], v[e], acc[e]);
        }
    };
    // Software pipeline over the wave's items (stride wstride): while item i
    // is combined and stored, the dY pieces of item i+1's first batch are in
    // flight, the row ids of item i+2's first batch are being fetched and
    // the chunk list entry of item i+3.  Later batches of a long chunk are
    // fetched in turn.
    int b0 = 0, c0 = 0, b1 = 0, c1 = 0, b2 = 0, c2 = 0;
    int jj[U];
    float aa[U];
    uint4 vv[U];
    if (wave < nitems) {
        meta(wave, b0, c0);
        int ii[U];
        row_ids(b0, c0, gh, ii);
        row_alphas(b0, c0, gh, aa);
        fetch(wave, ii, vv);
    }
    if (wave + wstride < nitems) {
        meta(wave + wstride, b1, c1);
        row_ids(b1, c1, gh, jj);
    }
    if (wave + 2 * wstride < nitems) meta(wave + 2 * wstride, b2, c2);
    for (int64_t item = wave; item < nitems; item += wstride) {
        const int64_t ch = item / a.nslab * HALVES + h;
        const int64_t col = (item % a.nslab) * SC + lq * PE;
        float acc[PE];
#pragma unroll
        for (int e = 0; e < PE; ++e) acc[e] = 0.f;
        accumulate(vv, aa, acc);  // first batch, fetched ahead
        const int nbatch = (c0 + BR - 1) / BR;
        for (int bt = 1; bt < nbatch; ++bt) {
            int ii[U];
            row_ids(b0, c0, gh + BR * bt, ii);
            row_alphas(b0, c0, gh + BR * bt, aa);
            fetch(item, ii, vv);
            accumulate(vv, aa, acc);
        }
        const int64_t n1 = item + wstride, n2 = n1 + wstride, n3 = n2 + wstride;
        if (n1 < nitems) {
            fetch(n1, jj, vv);
            row_alphas(b1, c1, gh, aa);
        }
        if (n2 < nitems) row_ids(b2, c2, gh, jj);
        int b3 = 0, c3 = 0;
        if (n3 < nitems) meta(n3, b3, c3);
        b0 = b1; c0 = c1;
        b1 = b2; c1 = c2;
        b2 = b3; c2 = c3;
        // lane stores of column n of this item's chunk straight into the B
        // fragments (B[n][kk] = P[kk][n]): bf16 lane l, piece 0 holds
        // B[32nb + l%32][16ks + 8(l/32) + 0..7], split into a hi and a lo
        // bf16 term (lo blocks after all hi blocks); fp32 lane l, piece h
        // holds B[32nb + l%32][16ks + 8h + 4(l/32) + 0..3]
        auto store = [&](int64_t n, float v) __attribute__((always_inline)) {
            if (n >= a.ncols) return;
            const int64_t nb = n >> 5, ks = ch >> 4;
            const int nl = (int)(n & 31), c16 = (int)(ch & 15);
            if constexpr (DT == DT_BF16) {
                const int64_t idx = ((nb * a.ks_cap + ks) * 64 + nl + 32 * (c16 >> 3)) * 8 + (c16 & 7);
                const uint32_t hi = f32_to_bf16(v);
                const uint32_t lo = f32_to_bf16(v - __uint_as_float(hi << 16));
                uint16_t* bf = reinterpret_cast<uint16_t*>(a.BF);
                bf[idx] = (uint16_t)hi;
                bf[idx + (a.ncols >> 5) * a.ks_cap * 64 * 8] = (uint16_t)lo;
            } else {
                const int64_t idx =
                    (((nb * a.ks_cap + ks) * 2 + (c16 >> 3)) * 64 + nl + 32 * ((c16 >> 2) & 1)) * 4 + (c16 & 3);
                reinterpret_cast<float*>(a.BF)[idx] = v;
            }
        };
        // fixed-order combine of the row groups of a chunk.  With as many
        // groups as columns (bf16) the combine is a reduce-scatter: at each
        // step a lane keeps half of its columns and adds the partner's sums
        // for them (7 exchanges instead of 24), and lane g of each group
        // stores column g; otherwise every lane sums all columns.  Paired
        // items reduce-scatter over the 4 groups of each half (lanes 8 and
        // 16 apart), leaving PE/4 columns per lane.
        if constexpr (PAIR) {
            constexpr int HALF = PE / 2, Q = PE / 4;
            const bool b1 = gh & 2, b0 = gh & 1;
            float r[HALF], q[Q];
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                const float keep = b1 ? acc[HALF + j] : acc[j];
                r[j] = keep + shfl_xor(b1 ? acc[j] : acc[HALF + j], 16);
            }
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const float keep = b0 ? r[Q + j] : r[j];
                q[j] = keep + shfl_xor(b0 ? r[j] : r[Q + j], 8);
            }
#pragma unroll
            for (int j = 0; j < Q; ++j) store(col + Q * gh + j, q[j]);
        } else {
            float v;
            if constexpr (PE == 8 && RG == 8) {
                const bool h4 = g & 4, h2 = g & 2, h1 = g & 1;
                float r4[4], r2[2];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float keep = h4 ? acc[4 + j] : acc[j];
                    r4[j] = keep + shfl_xor(h4 ? acc[j] : acc[4 + j], 32);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float keep = h2 ? r4[2 + j] : r4[j];
                    r2[j] = keep + shfl_xor(h2 ? r4[j] : r4[2 + j], 16);
                }
                // lanes l and l^8 share a row of 16 lanes: a DPP rotation by 8
                const float send = h1 ? r2[0] : r2[1];
                const int sx = __builtin_bit_cast(int, send);
                v = (h1 ? r2[1] : r2[0]) +
                    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(sx, sx, 0x128, 0xf, 0xf, false));
            } else {
#pragma unroll
                for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
                    for (int e = 0; e < PE; ++e) acc[e] += shfl_xor(acc[e], m);
                v = acc[0];
#pragma unroll
                for (int e = 1; e < PE; ++e) v = g == e ? acc[e] : v;
            }
            if (g < PE) store(col + g, v);
        }
    }
}

// ---------------------------------------------------------------------------
// 4. generator product dW = sum_chunk c_gen(chunk) (x) P[chunk]
// ---------------------------------------------------------------------------
// 4. dW tile per wave: 32*TM rows (d) x 32*TN columns (d_out), 32x32 MFMA
// tiles fed by contiguous fragment loads (L2-resident), no LDS and no
// barriers; results stored (non-temporal) as full 128-byte row pieces.
struct GemmArgs {
    const void* AF;
    const void* BF;
    int64_t ks_cap;
    int64_t d;
    int64_t d_out;
    const int32_t* nchunks;
    float* dW;
    int64_t lddw;
};

// TRANS writes dW^T [d_out x d] instead: the two operands swap places in
// every MFMA (their fragments share one lane layout), so each 32x32 result
// is a tile of dW^T and the stores are still whole 128-byte row pieces.
template <int DT, int TM, int TN, bool ACC, bool TRANS>
__global__ __launch_bounds__(256) void gen_gemm_kernel(GemmArgs a) {
    constexpr int PIECES = DT == DT_BF16 ? 1 : 2;
    const int lane = threadIdx.x & 63;
    // consecutive waves take consecutive tiles along the output's rows, so
    // a workgroup's stores extend the same rows: along d_out for dW, along d
    // for dW^T
    const int64_t tiles_m = (a.d + 32 * TM - 1) / (32 * TM);
    const int64_t tiles_n = (a.d_out + 32 * TN - 1) / (32 * TN);
    const int64_t wt = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t tm = TRANS ? wt % tiles_m : wt / tiles_n;
    const int64_t tn = TRANS ? wt / tiles_m : wt % tiles_n;
    const int64_t m0 = tm * 32 * TM, n0 = tn * 32 * TN;
    if (m0 >= a.d || n0 >= a.d_out) return;
    const int ks_used = (*a.nchunks + 15) >> 4;
    const int64_t mblk = (a.d + 31) / 32, nblk = (a.d_out + 31) / 32;
    const uint4* AF = reinterpret_cast<const uint4*>(a.AF);
    const uint4* BF = reinterpret_cast<const uint4*>(a.BF);
    // 1 KB slot of (block, step 0, piece 0) for each fragment row block (clamped
    // blocks past the edge are read but never stored)
    const uint4* ab[TM];
    const uint4* bb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) ab[i] = AF + min(m0 / 32 + i, mblk - 1) * a.ks_cap * PIECES * 64 + lane;
#pragma unroll
    for (int j = 0; j < TN; ++j) bb[j] = BF + min(n0 / 32 + j, nblk - 1) * a.ks_cap * PIECES * 64 + lane;
    const int64_t lo_off = nblk * a.ks_cap * 64;  // bf16: lo blocks follow the hi blocks

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // software pipeline over contraction steps with two register sets used
    // in turn: the fragments of step s+1 are in flight while step s runs its
    // MFMAs (past the last step the last one is re-read, never used)
    const int last = ks_used - 1;
    if constexpr (DT == DT_BF16) {
        uint4 a0[TM], h0[TN], l0[TN], a1[TM], h1[TN], l1[TN];
        auto fetch = [&](int ks, uint4* fa, uint4* fh, uint4* fl) {
            const int64_t o = (int64_t)ks * 64;
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = ab[i][o];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                fh[j] = bb[j][o];
                fl[j] = bb[j][o + lo_off];
            }
            pin_issued_loads();
        };
        auto step = [&](const uint4* fa, const uint4* fh, const uint4* fl) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const bf16x8 x = __builtin_bit_cast(bf16x8, fa[i]);
                    const bf16x8 h = __builtin_bit_cast(bf16x8, fh[j]), l = __builtin_bit_cast(bf16x8, fl[j]);
                    if constexpr (TRANS) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h, x, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l, x, acc[i][j], 0, 0, 0);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, h, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, l, acc[i][j], 0, 0, 0);
                    }
                }
        };
        if (ks_used > 0) fetch(0, a0, h0, l0);
        for (int ks = 0; ks < ks_used; ks += 2) {
            fetch(min(ks + 1, last), a1, h1, l1);
            step(a0, h0, l0);
            fetch(min(ks + 2, last), a0, h0, l0);
            if (ks + 1 < ks_used) step(a1, h1, l1);
        }
    } else {
        // piece h of lane group g holds chunks 16ks + 8h + 4g + 0..3;
        // MFMA (h, e) takes element e: chunks 16ks + 8h + e and + 4
        float4 a0[TM][2], b0[TN][2], a1[TM][2], b1[TN][2];
        auto fetch = [&](int ks, float4 (*fa)[2], float4 (*fb)[2]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t o = ((int64_t)ks * 2 + h) * 64;
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[i][h] = __builtin_bit_cast(float4, ab[i][o]);
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[j][h] = __builtin_bit_cast(float4, bb[j][o]);
            }
            pin_issued_loads();
        };
        auto step = [&](const float4 (*fa)[2], const float4 (*fb)[2]) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float4 x = TRANS ? fb[j][h] : fa[i][h], y = TRANS ? fa[i][h] : fb[j][h];
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y.x, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y.y, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y.z, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y.w, acc[i][j], 0, 0, 0);
                    }
        };
        if (ks_used > 0) fetch(0, a0, b0);
        for (int ks = 0; ks < ks_used; ks += 2) {
            fetch(min(ks + 1, last), a1, b1);
            step(a0, b0);
            fetch(min(ks + 2, last), a0, b0);
            if (ks + 1 < ks_used) step(a1, b1);
        }
    }

    // element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32 of a
    // 32x32 tile: rows in d and columns in d_out, or the other way round
    // for TRANS (rows in d_out, columns in d)
    const bool interior = m0 + 32 * TM <= a.d && n0 + 32 * TN <= a.d_out;
    const int64_t nrows = TRANS ? a.d_out : a.d, ncols = TRANS ? a.d : a.d_out;
    // The wide tile (many contraction steps, k >= kWideProductK): each 32x32
    // tile goes through this wave's slice of LDS (rows 40 floats apart: the
    // two half-waves of a staging write fall 32 banks apart) and leaves as
    // 16-byte pieces, 8 lanes per 128-byte row piece and 8 rows per store
    // instruction: fewer, wider stores than the result layout's 4 bytes per
    // lane.  A wave's LDS accesses complete in order, so the slice needs no
    // barrier between tiles (dW and its leading dimension are 16-byte
    // aligned, which the interface requires).  With few steps, as at 7B, the
    // product is bound by its stores and the staging delays them: the narrow
    // tile keeps the direct stores.
    if constexpr (TN >= 2) {
        constexpr int TP = 40;
        __shared__ __align__(16) float s_tile[4][32 * TP];
        float* tb = s_tile[threadIdx.x >> 6];
        const int sr = lane >> 3, sc = 4 * (lane & 7);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int e = 0; e < 16; ++e) tb[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * TP + (lane & 31)] = acc[i][j][e];
                const int64_t row0 = TRANS ? n0 + 32 * j : m0 + 32 * i;
                const int64_t col = (TRANS ? m0 + 32 * i : n0 + 32 * j) + sc;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int r = 8 * it + sr;
                    f32x4 v = *reinterpret_cast<const f32x4*>(tb + r * TP + sc);
                    float* p = a.dW + (row0 + r) * a.lddw + col;
                    if (interior || (row0 + r < nrows && col + 4 <= ncols)) {
                        // non-temporal: see below
                        if constexpr (ACC) v += *reinterpret_cast<const f32x4*>(p);
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
                    } else if (row0 + r < nrows) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (col + c < ncols) __builtin_nontemporal_store(ACC ? p[c] + v[c] : v[c], p + c);
                    }
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t row0 = TRANS ? n0 + 32 * j : m0 + 32 * i;
            const int64_t col = (TRANS ? m0 + 32 * i : n0 + 32 * j) + (lane & 31);
            float* base = a.dW + (row0 + 4 * (lane >> 5)) * a.lddw + col;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 8 * (e >> 2) + (e & 3);
                float* p = base + r * a.lddw;
                if (interior || (row0 + 4 * (lane >> 5) + r < nrows && col < ncols)) {
                    // non-temporal: dW goes straight to HBM instead of parking
                    // ~200 MB of dirty lines in the memory-side cache, whose
                    // write-back would otherwise slow the next kernel
                    const float v = ACC ? *p + acc[i][j][e] : acc[i][j][e];
                    __builtin_nontemporal_store(v, p);
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

WgradLayout wgrad_layout(int64_t n, int64_t k, int64_t d, int64_t d_out) {
    WgradLayout L;
    L.nb = (n + kSortBlockRows - 1) / kSortBlockRows;
    if (L.nb < 1) L.nb = 1;
    // chunk length: halved while even the most chunks it allows would give
    // fewer (chunk, 64-column slab) items than a full device has waves
    const int64_t slabs = (d_out + 63) / 64;
    int cr = kMaxChunkRows;
    while (cr > kMinChunkRows && ((n + cr - 1) / cr + k) * slabs < kFillItems) cr /= 2;
    L.chunk_rows = cr;
    L.max_chunks = (n + cr - 1) / cr + k;
    size_t off = 0;
    L.off_hist = off; off = align256(off + sizeof(int32_t) * (size_t)(L.nb * (k > 0 ? k : 1)));
    L.off_tot = off; off = align256(off + sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    L.off_nchunks = off; off = align256(off + sizeof(int32_t));
    L.off_chunk_gen = off; off = align256(off + sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_chunk_begin = off; off = align256(off + sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_chunk_count = off; off = align256(off + sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_perm = off; off = align256(off + sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    L.off_palpha = off; off = align256(off + sizeof(float) * (size_t)(n > 0 ? n : 1));
    // fragment-ordered product operands: 1 KB per (32-row block, 16-chunk
    // step) for bf16 (2 KB for fp32); B holds hi and lo halves for bf16
    L.ks_cap = (L.max_chunks + 15) / 16;
    L.off_AT = off; off = align256(off + 2048 * (size_t)(((d + 31) / 32) * L.ks_cap));
    L.off_BT = off; off = align256(off + 2048 * (size_t)(((d_out + 31) / 32) * L.ks_cap));
    L.total = off;
    return L;
}

// Generator counts from which the product uses the wider wave tile.
constexpr int kWideProductK = 256;

template <int DT, int TM, int TN>
static void launch_gen_gemm(const GemmArgs& g, const WgradArgs& a, hipStream_t st) {
    const int64_t waves = ((a.d + 32 * TM - 1) / (32 * TM)) * ((a.d_out + 32 * TN - 1) / (32 * TN));
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (a.transpose_out) {
        if (a.accumulate)
            hipLaunchKernelGGL((gen_gemm_kernel<DT, TM, TN, true, true>), grid, dim3(256), 0, st, g);
        else
            hipLaunchKernelGGL((gen_gemm_kernel<DT, TM, TN, false, true>), grid, dim3(256), 0, st, g);
    } else {
        if (a.accumulate)
            hipLaunchKernelGGL((gen_gemm_kernel<DT, TM, TN, true, false>), grid, dim3(256), 0, st, g);
        else
            hipLaunchKernelGGL((gen_gemm_kernel<DT, TM, TN, false, false>), grid, dim3(256), 0, st, g);
    }
}

template <int DT>
static hipError_t wgrad_impl(const WgradArgs& a, hipStream_t st) {
    const WgradLayout& L = a.L;
    char* ws = a.ws;
    int32_t* hist = reinterpret_cast<int32_t*>(ws + L.off_hist);
    int32_t* tot = reinterpret_cast<int32_t*>(ws + L.off_tot);
    int32_t* nchunks = reinterpret_cast<int32_t*>(ws + L.off_nchunks);
    int32_t* cgen = reinterpret_cast<int32_t*>(ws + L.off_chunk_gen);
    int32_t* cbeg = reinterpret_cast<int32_t*>(ws + L.off_chunk_begin);
    int32_t* ccnt = reinterpret_cast<int32_t*>(ws + L.off_chunk_count);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.off_perm);
    float* palpha = reinterpret_cast<float*>(ws + L.off_palpha);
    const int k = a.k;

    if (k > 0 && a.n > 0) {
        hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)L.nb), dim3(256), sizeof(int) * k, st, a.f, a.n, k, hist);
        SortScatterArgs s;
        s.f = a.f; s.alpha = a.alpha; s.n = a.n; s.k = k;
        int nbits = 0;
        while ((1 << nbits) < k) ++nbits;
        s.nbits = nbits;
        s.chunk_rows = L.chunk_rows;
        s.nb = L.nb; s.hist = hist; s.totals = tot; s.nchunks = nchunks;
        s.chunk_gen = cgen; s.chunk_begin = cbeg; s.chunk_count = ccnt; s.perm = perm; s.palpha = palpha;
        const size_t lds = sizeof(int) * (6 * (size_t)k + 256);
        const bool prefixed = L.nb * k > kSortPrefixEntries;
        const void* fn = prefixed ? reinterpret_cast<const void*>(&sort_scatter_kernel<true>)
                                  : reinterpret_cast<const void*>(&sort_scatter_kernel<false>);
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        if (prefixed) {
            hipLaunchKernelGGL(sort_prefix_kernel, dim3((unsigned)((k + 63) / 64)), dim3(256), 0, st, hist, L.nb, k,
                               tot);
            hipLaunchKernelGGL(sort_scatter_kernel<true>, dim3((unsigned)L.nb), dim3(256), lds, st, s);
        } else {
            hipLaunchKernelGGL(sort_scatter_kernel<false>, dim3((unsigned)L.nb), dim3(256), lds, st, s);
        }

        ScatterArgs r;
        r.dY = reinterpret_cast<const char*>(a.dY);
        r.lddy_bytes = a.lddy_bytes;
        r.d_out = a.d_out;
        constexpr int SC = PAMM_SR_LPR * Elem<DT>::per16;
        r.nslab = (a.d_out + SC - 1) / SC;
        r.nchunks = nchunks; r.chunk_begin = cbeg; r.chunk_count = ccnt; r.perm = perm; r.palpha = palpha;
        r.chunk_gen = cgen; r.C = a.C; r.d = a.d; r.AF = ws + L.off_AT;
        r.BF = ws + L.off_BT; r.ks_cap = L.ks_cap; r.ncols = (a.d_out + 31) & ~(int64_t)31;
        const int64_t max_items = (a.d + 31) / 32 * L.ks_cap * 2 + L.ks_cap * 16 * r.nslab;
        int64_t grid = (max_items + 3) / 4;
        const int64_t cap = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * 8;
        if (grid > cap) grid = cap;
        if (grid < 1) grid = 1;
        if (L.chunk_rows == kMaxChunkRows && a.n <= (int64_t)PAMM_SR_PAIR_ROWS * a.k)
            hipLaunchKernelGGL((scatter_reduce_kernel<DT, PAMM_SR_LPR, PAMM_SR_U, true>), dim3((unsigned)grid), dim3(256),
                               0, st, r);
        else
            hipLaunchKernelGGL((scatter_reduce_kernel<DT, PAMM_SR_LPR, PAMM_SR_U, false>), dim3((unsigned)grid), dim3(256),
                               0, st, r);
    } else {
        // no generators or no rows: no chunks, dW = 0 (or unchanged when accumulating)
        hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, st, nchunks);
    }

    GemmArgs g;
    g.AF = ws + L.off_AT; g.BF = ws + L.off_BT; g.ks_cap = L.ks_cap; g.d = a.d; g.d_out = a.d_out; g.nchunks = nchunks;
    g.dW = a.dW; g.lddw = a.lddw;
    // With k >= kWideProductK the contraction has at least as many chunk
    // steps and the product reads its operands from L2 many times over: a
    // wider wave tile (64 x 64) halves that traffic.  With few steps the
    // product is bound by the dW write, and the narrower tile (64 x 32)
    // spreads the stores over more waves.
    if (a.k >= kWideProductK)
        launch_gen_gemm<DT, PAMM_GEMM_TM, PAMM_GEMM_TN_WIDE>(g, a, st);
    else
        launch_gen_gemm<DT, PAMM_GEMM_TM, PAMM_GEMM_TN>(g, a, st);
    return hipGetLastError();
}

hipError_t run_wgrad(const WgradArgs& a, int dtype, hipStream_t st) {
    return dtype == DT_BF16 ? wgrad_impl<DT_BF16>(a, st) : wgrad_impl<DT_F32>(a, st);
}

}  // namespace pamm
