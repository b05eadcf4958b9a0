// pamm_compress.hip -- PAMM compression on gfx950.
//
// Implements the forward-pass phase of "QKV Projections Require a Fraction
// of Their Memory", section 2 "Metodologia", sub-part "Algoritmo in Due
// Fasi" (compression): every activation row is matched to the generator of
// largest |cosine|, given the least-squares scale onto that generator's line,
// and dropped when the cosine falls below eps.
//
// One kernel does the whole step.  A workgroup owns BM rows of X and a tile
// of up to KN generators:
//   * X and C (= rows gen_idx of X) are fetched from HBM into VGPRs as full
//     128-byte lines (8 lanes per row, the pattern HBM serves fastest; rows
//     fetched in MFMA-fragment order, 64 bytes per row per instruction, ran
//     at about 70% of that rate), PD stages ahead in a register ring, then
//     written to a double-buffered LDS tile, XOR-swizzled so MFMA fragment
//     reads avoid bank clashes.  Every load lands in registers, so the
//     compiler tracks every wait; each trip issues the same loads.
//   * Workgroups walk the d stages in a rotated order: rows are a leading
//     dimension apart, and in lock-step all workgroups would read the same
//     column range and crowd the same memory channels.
//   * S = X C^T accumulates in MFMA registers (bf16 16x16x32, or fp32
//     16x16x4); it is never written to memory.
//   * |c_j|^2 comes from extra MFMAs of the C fragments with themselves, the
//     same arithmetic as a dot product, so a row that is a power-of-two
//     multiple of a generator gets an exact alpha.
//   * |x_i|^2 is summed in fp32 from the X fragments the wave already holds.
//   * Epilogue: per-row argmax of |S_ij| / |c_j| across the 16 lanes of a row
//     (lowest index on ties, NaN never wins), cosine test against eps, alpha =
//     S_if / |c_f|^2.
// When k exceeds one generator tile the per-tile winners go to a small
// workspace and compress_merge_kernel picks the overall winner.  The tiles of
// one row block then take consecutive workgroup slots of one XCD and walk the
// stages in the same order, so the row block's X lines come from HBM about
// once and are re-read from that XCD's L2.
#include <type_traits>

#include "pamm_device.hpp"
#include "pamm_kernels.hpp"

#ifndef PAMM_COMPRESS_ROTATE
#define PAMM_COMPRESS_ROTATE 1
#endif

namespace pamm {

namespace {


// Workgroup barrier for the staged tiles.  Each wave has already waited for
// its own LDS stores (wait_lds), so the barrier needs no memory fence; the
// fence of __syncthreads() would also wait for every outstanding global
// load, i.e. drain the register prefetch.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14)); }


template <int DT>
__device__ __forceinline__ void mma16(const uint4& a, const uint4& b, f32x4& acc) {
    if constexpr (DT == DT_BF16) {
        bf16x8 av = __builtin_bit_cast(bf16x8, a);
        bf16x8 bv = __builtin_bit_cast(bf16x8, b);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
}

template <int DT>
__device__ __forceinline__ float sumsq16(const uint4& v) {
    float e[Elem<DT>::per16];
    unpack16<DT>(v, e);
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Elem<DT>::per16; ++q) s = __builtin_fmaf(e[q], e[q], s);
    return s;
}

// Byte offset in a staged tile (RB bytes per row) of 16-byte chunk `q` of
// tile row `r`: chunks are XOR-swizzled by the row so that the 16 rows of an
// MFMA fragment read fall into different LDS banks.
template <int RB>
__device__ __forceinline__ int swz(int r, int q) {
    return r * RB + ((q ^ (r & (RB / 16 - 1))) << 4);
}

// Call f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace

// Per-row winner among a generator tile, then the eps test and alpha.
// acc[mt][nt][i] holds S for row 16*mt + 4*(lane/16) + i of the wave and
// generator 16*nt + lane%16 of the tile; xn2r[mt] holds |x|^2 of row
// 16*mt + lane%16.  The 16 lanes of a row reduce (score desc, index asc);
// a NaN score never wins.
template <int MT, int NTL>
__device__ __forceinline__ void epilogue_rows(const CompressArgs& a, const f32x4 (&acc)[MT][NTL],
                                              const float (&xn2r)[MT], const float* s_cn2, const float* s_rinv,
                                              int64_t row_base, int tile, int gen0, int ktile, int lane) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rloc = mt * 16 + 4 * (lane >> 4) + i;
            float bs = -1.0f, bd = 0.f;
            int bg = 0x7fffffff;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const int jl = nt * 16 + (lane & 15);
                if (jl < ktile) {
                    const float dot = acc[mt][nt][i];
                    const float cn = s_cn2[jl];
                    const float sc = cn > 0.f ? fabsf(dot) * s_rinv[jl] : 0.f;
                    if (sc > bs) { bs = sc; bg = gen0 + jl; bd = dot; }
                }
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
                const float os = shfl_xor(bs, m);
                const int og = shfl_xor(bg, m);
                const float od = shfl_xor(bd, m);
                if (os > bs || (os == bs && og < bg)) { bs = os; bg = og; bd = od; }
            }
            const float xn2 = __shfl(xn2r[mt], 4 * (lane >> 4) + i, 64);
            const int64_t row = row_base + rloc;
            if ((lane & 15) == i && row < a.n) {
                const bool found = bg != 0x7fffffff;
                float al = 0.f;
                if (found) {
                    const float cn = s_cn2[bg - gen0];
                    al = cn > 0.f ? bd / cn : 0.f;
                }
                if (a.partial) {
                    PartialBest pb;
                    pb.score = found ? bs : -1.0f;
                    pb.gen = found ? bg : -1;
                    pb.alpha = al;
                    a.partial[(int64_t)tile * a.n + row] = pb;
                    if (tile == 0) a.xn2[row] = xn2;
                } else {
                    // cosine of the winner; 0 for a zero row, NaN (never kept) for a NaN row
                    const float cs = xn2 == 0.f ? 0.f : bs / sqrtf(xn2);
                    const bool keep = found && cs >= a.eps;
                    a.f[row] = keep ? bg : -1;
                    a.alpha[row] = keep ? al : 0.f;
                }
            }
        }
    }
}

// The compress kernel (see the file comment).  WM rows per wave, NW waves,
// KN generators per tile, PD stages of register prefetch.
template <int DT, int WM, int NW, int KN, int PD, int RB>
__global__ __launch_bounds__(64 * NW) void compress_rs_kernel(CompressArgs a) {
    constexpr int SUBS = RB / 64;                     // MFMA K sub-steps per stage
    constexpr int CH = RB / 16;                       // 16-byte chunks per staged row
    constexpr int RPI = 64 / CH;                      // rows per wave-wide load
    constexpr int BM = WM * NW;
    constexpr int MT = WM / 16;
    constexpr int NTL = KN / 16;
    constexpr int NDG = (NTL + NW - 1) / NW;
    constexpr int XPT = BM / (RPI * NW);              // X chunks per lane per stage
    constexpr int CPT = (KN + RPI * NW - 1) / (RPI * NW);
    constexpr int CROWS = CPT * NW * RPI;
    constexpr int E = RB / Elem<DT>::size;
    constexpr int P = Elem<DT>::per16;
    static_assert(BM % (RPI * NW) == 0 && PD % 2 == 0 && PD >= 2, "tile shape");
    static_assert(RB == 128 || RB == 256 || RB == 512, "stage width");

    __shared__ __align__(16) char s_x0[BM * RB];
    __shared__ __align__(16) char s_x1[BM * RB];
    __shared__ __align__(16) char s_c0[CROWS * RB];
    __shared__ __align__(16) char s_c1[CROWS * RB];
    __shared__ float s_cn2[KN];
    __shared__ float s_rinv[KN];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    // workgroup -> (row block, generator tile).  With several tiles, the
    // tiles of one row block take consecutive workgroup slots of one XCD
    // (slots go round-robin over the 8 XCDs) and walk the stages in the same
    // order, so the row block's X lines come from HBM about once and are
    // re-read from that XCD's L2 by the other tiles.
    int64_t rb = blockIdx.x;
    int tile = 0;
    if (a.ntiles > 1) {
        const int64_t grp = blockIdx.x / (8 * a.ntiles), rem = blockIdx.x % (8 * a.ntiles);
        tile = (int)(rem / 8);
        rb = grp * 8 + rem % 8;
    }
    const int64_t m0 = rb * BM;
    const int gen0 = tile * KN;
    const int ktile = min(KN, a.k - gen0);
    const int nst = (int)((a.d + E - 1) / E);
    const int last = nst - 1;
    const char* __restrict__ X = reinterpret_cast<const char*>(a.X);

    // ---- copy out the generator rows C = X[gen_idx] (spread over all workgroups)
    if (a.C) {
        const int64_t row_chunks = (a.d + P - 1) / P;
        const int64_t total = (int64_t)a.k * row_chunks;
        const int64_t nwg = gridDim.x;
        const int64_t wg = blockIdx.x;
        for (int64_t c = wg * (64 * NW) + tid; c < total; c += nwg * (64 * NW)) {
            const int64_t j = c / row_chunks, col = (c % row_chunks) * P;
            int64_t r = a.gen_idx[j];
            r = r < 0 ? 0 : (r >= a.n ? a.n - 1 : r);
            const uint4 v = load16_tail<DT>(X + r * a.ldx_bytes, col, a.d);
            char* dst = reinterpret_cast<char*>(a.C) + (j * a.d + col) * Elem<DT>::size;
            if (a.c_vec_ok && col + P <= a.d) {
                *reinterpret_cast<uint4*>(dst) = v;
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                for (int e = 0; e < P && col + e < a.d; ++e) {
                    if constexpr (DT == DT_BF16)
                        reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    else
                        reinterpret_cast<uint32_t*>(dst)[e] = w[e];
                }
            }
        }
    }

    if (m0 >= a.n) return;  // slot past the last row block (whole workgroup)

    // ---- rows this lane fetches: load i covers tile rows RPI*(wave + NW*i) + lane/CH,
    // 16-byte chunk lane%CH of each RB-byte stage
    const int qc = lane % CH;
    const char* xsrc[XPT];
    int xdst[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int r = RPI * (wave + NW * i) + lane / CH;
        int64_t g = m0 + r;
        if (g >= a.n) g = a.n - 1;  // padding rows: any valid row, results unused
        xsrc[i] = X + g * a.ldx_bytes + qc * 16;
        xdst[i] = swz<RB>(r, qc);
    }
    const char* csrc[CPT];
    int cdst[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int r = RPI * (wave + NW * i) + lane / CH;
        const int jj = min(r, max(ktile - 1, 0));  // padding generators: any valid one, masked later
        int64_t g = a.k > 0 ? a.gen_idx[gen0 + jj] : 0;
        g = g < 0 ? 0 : (g >= a.n ? a.n - 1 : g);
        csrc[i] = X + g * a.ldx_bytes + qc * 16;
        cdst[i] = swz<RB>(r, qc);
    }
    // rotated stage order (workgroups start at different column ranges);
    // padding stages past the end map to the last stage and are zeroed
    const int rot = PAMM_COMPRESS_ROTATE ? (int)(((uint64_t)rb * 37u) % (unsigned)nst) : 0;
    auto stage_of = [&](int s) { if (s >= nst) return last; int t = s + rot; return t >= nst ? t - nst : t; };
    const int tail_elems = (int)(a.d - (int64_t)last * E);

    uint4 xr[PD][XPT], cr[PD][CPT];
    auto issue = [&](int s, auto slotc) {
        constexpr int U = decltype(slotc)::value;
        int64_t off = (int64_t)stage_of(s) * RB + qc * 16;
        off = off >= a.row_bytes ? -(int64_t)qc * 16 : (int64_t)stage_of(s) * RB;  // chunk past the row end: chunk 0
#pragma unroll
        for (int i = 0; i < XPT; ++i) xr[U][i] = load16_nt(xsrc[i] + off);  // X is read once: non-temporal
#pragma unroll
        for (int i = 0; i < CPT; ++i) cr[U][i] = *reinterpret_cast<const uint4*>(csrc[i] + off);
    };
    // zero the elements of a chunk starting at stage element e0 that lie at or past `lim`
    auto mask_chunk = [&](uint4& v, int e0, int lim) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < P; ++e) {
            if (e0 + e >= lim) {
                if constexpr (DT == DT_BF16) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                else w[e] = 0;
            }
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    };

    f32x4 acc[MT][NTL];
    f32x4 dacc[NDG];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NDG; ++g) dacc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    float xsq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xsq[mt] = 0.f;

    static_for<0, PD>([&](auto uc) { issue(decltype(uc)::value, uc); });

    for (int s0 = 0; s0 < nst; s0 += PD) {
        static_for<0, PD>([&](auto uc) {
            constexpr int U = decltype(uc)::value;
            const int s = s0 + U;
            char* sx = (U & 1) ? s_x1 : s_x0;
            char* sc = (U & 1) ? s_c1 : s_c0;
            const int lim = s >= nst ? 0 : (stage_of(s) < last ? E : tail_elems);
            uint4 xw[XPT], cw[CPT];
#pragma unroll
            for (int i = 0; i < XPT; ++i) xw[i] = xr[U][i];
#pragma unroll
            for (int i = 0; i < CPT; ++i) cw[i] = cr[U][i];
            if (lim < E) {  // uniform: the last real stage and the padding stages
#pragma unroll
                for (int i = 0; i < XPT; ++i) mask_chunk(xw[i], qc * P, lim);
#pragma unroll
                for (int i = 0; i < CPT; ++i) mask_chunk(cw[i], qc * P, lim);
            }
#pragma unroll
            for (int i = 0; i < XPT; ++i) *reinterpret_cast<uint4*>(sx + xdst[i]) = xw[i];
#pragma unroll
            for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(sc + cdst[i]) = cw[i];
            issue(s + PD, uc);  // register slot U is free again
            wait_lds();
            ring_barrier();
#pragma unroll
            for (int sub = 0; sub < SUBS; ++sub) {
                const int q = sub * 4 + (lane >> 4);
                uint4 xf[MT], cf[NTL], cd[NDG];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    xf[mt] = *reinterpret_cast<const uint4*>(sx + swz<RB>(wave * WM + mt * 16 + (lane & 15), q));
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
                    cf[nt] = *reinterpret_cast<const uint4*>(sc + swz<RB>(nt * 16 + (lane & 15), q));
#pragma unroll
                for (int g = 0; g < NDG; ++g) {
                    const int nt = min(wave + g * NW, NTL - 1);
                    cd[g] = *reinterpret_cast<const uint4*>(sc + swz<RB>(nt * 16 + (lane & 15), q));
                }
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) mma16<DT>(xf[mt], cf[nt], acc[mt][nt]);
#pragma unroll
                for (int g = 0; g < NDG; ++g) mma16<DT>(cd[g], cd[g], dacc[g]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xsq[mt] += sumsq16<DT>(xf[mt]);
            }
        });
    }

    // ---- epilogue: norms
#pragma unroll
    for (int g = 0; g < NDG; ++g) {
        const int nt = wave + g * NW;
        const int c = lane & 15, grp = lane >> 4;
        if (nt < NTL && (c >> 2) == grp) {
            const float v = dacc[g][c & 3];
            s_cn2[nt * 16 + c] = v;
            s_rinv[nt * 16 + c] = v > 0.f ? 1.0f / sqrtf(v) : 0.f;
        }
    }
    float xn2r[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float v = xsq[mt];
        v += shfl_xor(v, 16);
        v += shfl_xor(v, 32);
        xn2r[mt] = v;
    }
    __syncthreads();
    epilogue_rows<MT, NTL>(a, acc, xn2r, s_cn2, s_rinv, m0 + wave * WM, tile, gen0, ktile, lane);
}

// Pick, per row, the best of the per-tile winners (tiles are in increasing
// generator order, so a strict comparison keeps the lowest index on ties) and
// apply the eps test.
__global__ __launch_bounds__(256) void compress_merge_kernel(const PartialBest* __restrict__ part,
                                                             const float* __restrict__ xn2, int64_t n,
                                                             int ntiles, float eps, int32_t* __restrict__ f,
                                                             float* __restrict__ alpha) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= n) return;
    float bs = -1.0f, ba = 0.f;
    int bg = -1;
    for (int t = 0; t < ntiles; ++t) {
        const PartialBest p = part[(int64_t)t * n + row];
        if (p.gen >= 0 && p.score > bs) { bs = p.score; bg = p.gen; ba = p.alpha; }
    }
    const float x2 = xn2[row];
    const float cs = x2 == 0.f ? 0.f : bs / sqrtf(x2);
    const bool keep = bg >= 0 && cs >= eps;
    f[row] = keep ? bg : -1;
    alpha[row] = keep ? ba : 0.f;
}

// Every row is dropped when there are no generators.
__global__ __launch_bounds__(256) void compress_empty_kernel(int64_t n, int32_t* __restrict__ f,
                                                             float* __restrict__ alpha) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row < n) { f[row] = -1; alpha[row] = 0.f; }
}

template <int DT, int WM, int NW, int KN, int PD, int RB>
static hipError_t launch_compress_rs(const CompressArgs& a, int ntiles, hipStream_t st) {
    constexpr int BM = WM * NW;
    const int64_t nrb = (a.n + BM - 1) / BM;
    const dim3 grid((unsigned)(ntiles > 1 ? (nrb + 7) / 8 * 8 * ntiles : nrb));
    hipLaunchKernelGGL((compress_rs_kernel<DT, WM, NW, KN, PD, RB>), grid, dim3(64 * NW), 0, st, a);
    return hipGetLastError();
}

// Tile shapes per generator-tile width: rows per wave, waves, generators,
// register prefetch depth (stages), bytes of each row per stage.  The
// 256-generator tile prefetches two stages: with four, its accumulators,
// fragments and ring exceed the 256 registers a wave of a 512-thread
// workgroup may hold, and the spills cost twice the time.
#ifndef PAMM_COMPRESS_RS16
#define PAMM_COMPRESS_RS16 16, 8, 16, 4, 128
#endif
#ifndef PAMM_COMPRESS_RS32
#define PAMM_COMPRESS_RS32 16, 8, 32, 4, 128
#endif
#ifndef PAMM_COMPRESS_RS64
#define PAMM_COMPRESS_RS64 16, 8, 64, 4, 128
#endif
#ifndef PAMM_COMPRESS_RS128
#define PAMM_COMPRESS_RS128 16, 8, 128, 4, 128
#endif
#ifndef PAMM_COMPRESS_RS256
#define PAMM_COMPRESS_RS256 16, 8, 256, 2, 128
#endif

template <int DT>
static hipError_t compress_dispatch(const CompressArgs& a, int kn, int ntiles, hipStream_t st) {
    switch (kn) {
        case 16: return launch_compress_rs<DT, PAMM_COMPRESS_RS16>(a, ntiles, st);
        case 32: return launch_compress_rs<DT, PAMM_COMPRESS_RS32>(a, ntiles, st);
        case 64: return launch_compress_rs<DT, PAMM_COMPRESS_RS64>(a, ntiles, st);
        case 128: return launch_compress_rs<DT, PAMM_COMPRESS_RS128>(a, ntiles, st);
        default: return launch_compress_rs<DT, PAMM_COMPRESS_RS256>(a, ntiles, st);
    }
}

hipError_t run_compress(const CompressArgs& a, int dtype, hipStream_t st) {
    if (a.k == 0) {
        hipLaunchKernelGGL(compress_empty_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, st, a.n, a.f,
                           a.alpha);
        return hipGetLastError();
    }
    int kn = 16;
    while (kn < a.k && kn < kMaxTileGens) kn *= 2;
    const int ntiles = (int)((a.k + kn - 1) / kn);
    CompressArgs b = a;
    b.ntiles = ntiles;
    if (ntiles == 1) { b.partial = nullptr; b.xn2 = nullptr; }
    hipError_t e = dtype == DT_BF16 ? compress_dispatch<DT_BF16>(b, kn, ntiles, st)
                                    : compress_dispatch<DT_F32>(b, kn, ntiles, st);
    if (e != hipSuccess || ntiles == 1) return e;
    hipLaunchKernelGGL(compress_merge_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, st, a.partial,
                       a.xn2, a.n, ntiles, a.eps, a.f, a.alpha);
    return hipGetLastError();
}

}  // namespace pamm
