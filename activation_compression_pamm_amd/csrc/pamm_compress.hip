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
//     at about 89% of that rate), PD stages ahead in a register ring, then
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
//   * |x_i|^2 likewise: bf16 takes the diagonal of MFMAs of the wave's X
//     fragments with themselves (the matrix cores idle most of the time at
//     small k, the VALU does not); fp32 sums squares on the VALU.
//   * Epilogue: per-row argmax of |S_ij| / |c_j| across the 16 lanes of a row
//     (lowest index on ties, NaN never wins), cosine test against eps, alpha =
//     S_if / |c_f|^2.
// When k exceeds one generator tile the per-tile winners go to a small
// workspace and compress_merge_kernel picks the overall winner.  The tiles of
// one row block then take consecutive workgroup slots of one XCD and walk the
// stages in the same order, so the row block's X lines come from HBM about
// once and are re-read from that XCD's L2.
#include <algorithm>
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

// Swizzle key of the GEMM-shaped kernel's 128-byte rows, whose 32x32x16
// fragment reads take rows l%32 at chunk 2k + l/32.  Chosen by measurement
// (SQ_LDS_BANK_CONFLICT against SQ_LDS_IDX_ACTIVE): with the key r%8 a third
// of that kernel's LDS-active cycles were bank-conflict stalls, with this key
// under 4%.  The 16x16x32 reads of compress_rs_kernel (rows l%16 at chunk
// 4k + l/16) are conflict-free with r%8 and conflict with this key.
__device__ __forceinline__ int gemm_swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Call f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// C = X[gen_idx]: every workgroup of the launch copies its share of the
// generator rows (the launch's workgroups together cover all k rows).
template <int DT>
__device__ __forceinline__ void copy_out_generators(const CompressArgs& a, int nthreads) {
    if (!a.C) return;
    const char* __restrict__ X = reinterpret_cast<const char*>(a.X);
    constexpr int P = Elem<DT>::per16;
    const int tid = threadIdx.x;
    const int64_t row_chunks = (a.d + P - 1) / P;
    const int64_t total = (int64_t)a.k * row_chunks;
    const int64_t nwg = gridDim.x;
    const int64_t wg = blockIdx.x;
    for (int64_t c = wg * nthreads + tid; c < total; c += nwg * nthreads) {
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

}  // namespace

// Value of lane (l + R) mod 16 within each row of 16 lanes (DPP row_ror; a
// VALU move, no LDS round trip).
template <int R, typename T>
__device__ __forceinline__ T row_ror(T v) {
    static_assert(sizeof(T) == 4 && R >= 1 && R <= 15, "32-bit value, rotation 1..15");
    const int x = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(x, x, 0x120 | R, 0xf, 0xf, false));
}

// One all-reduce round of the (score desc, index asc) winner over 16 lanes.
template <int R>
__device__ __forceinline__ void winner_round(float& bs, int& bg, float& bd) {
    const float os = row_ror<R>(bs);
    const int og = row_ror<R>(bg);
    const float od = row_ror<R>(bd);
    if (os > bs || (os == bs && og < bg)) { bs = os; bg = og; bd = od; }
}

// Per-row winner among a generator tile, then the eps test and alpha.
// acc[mt][nt][i] holds S for row 16*mt + 4*(lane/16) + i of the wave and
// generator 16*nt + lane%16 of the tile; xn2r[mt] holds |x|^2 of row
// 16*mt + lane%16.  The 16 lanes of a row reduce (score desc, index asc)
// by DPP rotations; a NaN score never wins.
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
            // the winner is a maximum under a total order (NaN scores never
            // enter), so rotations reduce the 16 lanes as well as a butterfly
            winner_round<8>(bs, bg, bd);
            winner_round<4>(bs, bg, bd);
            winner_round<2>(bs, bg, bd);
            winner_round<1>(bs, bg, bd);
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar, so tests on it are branches
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

    copy_out_generators<DT>(a, 64 * NW);

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
    // |x|^2: bf16 takes the diagonal of an MFMA of the X fragments with
    // themselves (the matrix cores are mostly idle here, the VALU is not);
    // fp32 sums squares on the VALU
    constexpr bool XMFMA = DT == DT_BF16;
    float xsq[MT];
    f32x4 xacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        xsq[mt] = 0.f;
        xacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

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
                    if (wave + g * NW >= NTL) continue;  // no diagonal block left for this wave
                    const int nt = min(wave + g * NW, NTL - 1);
                    cd[g] = *reinterpret_cast<const uint4*>(sc + swz<RB>(nt * 16 + (lane & 15), q));
                }
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) mma16<DT>(xf[mt], cf[nt], acc[mt][nt]);
#pragma unroll
                for (int g = 0; g < NDG; ++g)
                    if (wave + g * NW < NTL) mma16<DT>(cd[g], cd[g], dacc[g]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (XMFMA) mma16<DT>(xf[mt], xf[mt], xacc[mt]);
                    else xsq[mt] += sumsq16<DT>(xf[mt]);
                }
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
        float v;
        if constexpr (XMFMA) {
            // row r of the block sits at element r%4 of lane 16*(r/4) + r
            const int r = lane & 15, e = r & 3;
            const float own = e == 0 ? xacc[mt][0] : e == 1 ? xacc[mt][1] : e == 2 ? xacc[mt][2] : xacc[mt][3];
            v = __shfl(own, 16 * (r >> 2) + r, 64);
        } else {
            v = xsq[mt];
            v += shfl_xor(v, 16);
            v += shfl_xor(v, 32);
        }
        xn2r[mt] = v;
    }
    __syncthreads();
    epilogue_rows<MT, NTL>(a, acc, xn2r, s_cn2, s_rinv, m0 + wave * WM, tile, gen0, ktile, lane);
}

// Requested instruction order for one scheduling region of the GEMM-shaped
// kernel's loop: each LDS read, LDS write and global load is issued right
// after one of the region's MFMAs (NR reads first, then NW writes, then NV
// loads; NM MFMAs left over), so that it issues while the MFMA runs.  Left to
// itself the scheduler clusters them between runs of MFMAs, and the matrix
// core idles while they issue and while the LDS writes wait for their data.
template <int NR, int NW, int NV, int NM>
__device__ __forceinline__ void interleave_region() {
    static_for<0, NR>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); });
    static_for<0, NW>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); });
    static_for<0, NV>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); });
    if constexpr (NM > 0) __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
}
// The same with NR reads first, then NP pairs of (LDS write, global load).
template <int NR, int NP>
__device__ __forceinline__ void interleave_region2() {
    static_for<0, NR>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); });
    static_for<0, NP>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    });
}

// The same for regions with more memory instructions than MFMAs: the NR
// reads, NW writes and NV loads, in that order, are spread evenly over the
// NM MFMAs (MFMA i is followed by instructions NO*i/NM .. NO*(i+1)/NM - 1).
template <int NR, int NW, int NV>
__device__ __forceinline__ constexpr int op_mask(int o) { return o < NR ? 0x100 : (o < NR + NW ? 0x200 : 0x020); }
template <int NR, int NW, int NV, int NM>
__device__ __forceinline__ void interleave_spread() {
    constexpr int NO = NR + NW + NV;
    static_for<0, NM>([&](auto mi) {
        constexpr int i = decltype(mi)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        static_for<NO * i / NM, NO * (i + 1) / NM>([&](auto oi) {
            __builtin_amdgcn_sched_group_barrier(op_mask<NR, NW, NV>(decltype(oi)::value), 1, 0);
        });
    });
}

// Tiles of 256 generators in bf16: the contraction dominates (k >= 256 means
// at least 256 MFMA flops per byte of X), so the workgroup is shaped like a
// GEMM tile: NWR x NWC waves, each holding 32*MT rows x 32*NT generators of
// S in 32x32 MFMA accumulators.  Two shapes of a 256 x 256 tile: 2 x 2 waves
// of 128 x 128 (256 accumulation registers, one wave per SIMD, one LDS
// fragment read per 2 MFMAs) and 2 x 4 waves of 128 x 64 (two waves per
// SIMD, whose memory traffic and MFMAs overlap; a fragment read per 1.33
// MFMAs).
//   * One stage = 64 elements (128 bytes) of every tile row.  X and C lines
//     are fetched as whole 128-byte lines into registers one stage ahead and
//     written to a double-buffered LDS tile, XOR-swizzled with this kernel's
//     own key (gemm_swz_key).  The steady-state loop has no branch: the stage
//     count is padded to an even number, and padding stages and the columns
//     past d are masked to zero on their way into LDS (a second instance
//     without masks serves d a multiple of 64 with an even stage count).
//     Within each scheduling region every memory instruction is issued right
//     after one MFMA (interleave_region).
//   * |x_i|^2 is summed in fp32 with bf16 dot2 instructions from the staged
//     lines by the workgroups of the first generator tile; |c_j|^2 likewise,
//     once per generator, by gen_prep_kernel, which also writes C.  (The
//     smaller-tile kernels take |c_j|^2 from the MFMA instead, which makes
//     alpha exact for a power-of-two multiple of a generator; here no
//     accumulation registers are left for that, so such an alpha is exact to
//     a few fp32 ulps, and its bf16 reconstruction is still exact.)
//   * The MFMA takes the generator fragment as its A operand and the X
//     fragment as B, so each lane's accumulators hold one row of S and 16 of
//     each 32 generators.  Epilogue: each lane scans its generators of a row
//     in registers, meets lane l^32 (the other 16 of each 32), the NWC
//     column winners meet in LDS, and one thread per row merges them (lower
//     column first, so the lowest index wins ties) and writes the result.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sumsq_dot2(const v4u32& v, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // copy the component out first: this compiler bit-casts a vector
        // component expression as if it were component 0
        const uint32_t e = v[w];
        const bf16x2 h = __builtin_bit_cast(bf16x2, e);
        acc = __builtin_amdgcn_fdot2_f32_bf16(h, h, acc, false);
    }
    return acc;
}

// Epilogue of a Y tile (pamm_forward_compress): each wave's 32*MT x 32*NT
// block of X W^T, plus the bias, rounded to bf16 (nearest even), goes to Y
// through LDS in passes of 32 rows (each lane writes four adjacent values at
// a time, then every lane stores whole 16-byte pieces of the staged rows;
// non-temporal: Y is not re-read by this pass).  Rows past n and columns past
// d_out are not written.  The accumulators hold the product transposed (W
// rows as the MFMA's A operand): element i of a 32x32 result lane l is row
// l%32, column 8*(i/4) + 4*(l/32) + i%4.
template <int MT, int NT, int NWR, int NWC>
__device__ __forceinline__ void store_y_tile(const CompressArgs& a, const f32x16 (&acc)[MT][NT], char* ring,
                                             int64_t m0, int64_t n0, int wr, int wc, int lane, int wave) {
    constexpr int WM = 32 * MT, WN = 32 * NT;
    constexpr int PITCH = WN * 2 + 16;     // bytes per staged row: 16 banks apart for rows 4 apart
    constexpr int CH = WN * 2 / 16;        // 16-byte pieces per staged row
    static_assert((64 % CH) == 0, "pieces of a staged row divide the wave");
    constexpr int RPI = 64 / CH;           // rows read per instruction
    static_assert(NWR * NWC * 32 * PITCH <= 2 * (32 * MT * NWR + 32 * NT * NWC) * 128,
                  "the staged Y rows fit in the stage ring");
    char* buf = ring + wave * 32 * PITCH;
    const int frow = lane & 31, fk = lane >> 5;
    const uint16_t* bias = reinterpret_cast<const uint16_t*>(a.bias);
    // bias of the lane's 16 columns of each 32-column block
    float bt[NT][16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t col = n0 + wc * WN + nt * 32 + 8 * (i >> 2) + 4 * fk + (i & 3);
            bt[nt][i] = (bias && col < a.d_out) ? bf16_to_f32(bias[col]) : 0.f;
        }
    const int64_t col0 = n0 + wc * WN;
    char* Y = reinterpret_cast<char*>(a.Y);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        // lane l holds row l%32 and columns 8*(i/4) + 4*(l/32) + i%4 of
        // each 32-column block: four adjacent columns per 8-byte write
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c0 = nt * 32 + 8 * q + 4 * fk;
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(acc[mt][nt][4 * q + e] + bt[nt][4 * q + e]);
                *reinterpret_cast<uint2*>(buf + frow * PITCH + c0 * 2) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        __syncthreads();
        const int q = lane % CH;
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int r = lane / CH + RPI * it;
            const int64_t row = m0 + wr * WM + mt * 32 + r;
            const int64_t col = col0 + q * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(buf + r * PITCH + q * 16);
            if (row < a.n && col < a.d_out) {
                char* dst = Y + row * a.ldy_bytes + col * 2;
                if (col + 8 <= a.d_out) {
                    __builtin_nontemporal_store(v4u32{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u32*>(dst));
                } else {
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                    for (int e = 0; col + e < a.d_out; ++e)
                        reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
        __syncthreads();
    }
}

// MASKED: the tail stage and padding positions exist (d not a multiple of 64,
// or an odd stage count); without them the stash applies no masks.
// FUSED: the forward projection Y = X W^T (+ bias) runs in the same launch.
// Its 256-column tiles are extra column tiles in front of the generator
// tiles: their B operand rows are rows of W instead of generator rows of X,
// the main loop is the same, and their epilogue stores the bf16 tile of Y.
// Workgroups take (row block, column tile) pairs in groups of 4 row blocks x
// 8 column tiles, one group per XCD at a time, so that the 32 workgroups an
// XCD runs together share their X and W panels in its L2.
template <int MT, int NT, int NWR, int NWC, bool MASKED, bool FUSED = false>
__global__ __launch_bounds__(64 * NWR * NWC) void compress_gemm_kernel(CompressArgs a) {
    constexpr int RB = 128;                 // bytes of a row per stage
    constexpr int E = RB / 2;               // elements per stage
    constexpr int NW = NWR * NWC;
    constexpr int NTH = 64 * NW;
    constexpr int WM = 32 * MT, WN = 32 * NT;
    constexpr int BM = WM * NWR, BN = WN * NWC;
    constexpr int XPT = BM * 8 / NTH;       // 16-byte X chunks per lane per stage
    constexpr int CPT = BN * 8 / NTH;
    static_assert(BN <= kMaxTileGens && BN % 64 == 0, "one generator tile per workgroup");
    static_assert((BM * 8) % NTH == 0 && (BN * 8) % NTH == 0, "tile shape");

    // two stage buffers, each the X tile then the C tile
    constexpr int TILE = (BM + BN) * RB;
    __shared__ __align__(16) char s_tile[2 * TILE];
    __shared__ __align__(16) float s_cn2[BN];
    __shared__ __align__(16) float s_rinv[BN];
    __shared__ __align__(16) float s_floor[BN];  // score without a valid |c|^2: -1 (padding) or 0
    __shared__ float s_ms[NWC][BM];
    __shared__ int s_mg[NWC][BM];
    __shared__ float s_md[NWC][BM];
    __shared__ float s_xn2[BM];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wr = wave / NWC, wc = wave % NWC;
    // workgroup -> (row block, generator tile), as in compress_rs_kernel
    int64_t rb = blockIdx.x;
    int tile = 0;
    bool wtile = false;  // FUSED: a column tile of Y (B rows from W)
    int64_t n0 = 0;      // FUSED: first output column of a Y tile
    if constexpr (FUSED) {
        // block b runs on XCD b % 8; the XCD's slots s = b / 8 take groups of
        // 32: group p = (s / 32) * 8 + XCD, inside it 4 row blocks x 8 tiles
        const int64_t b = blockIdx.x, s = b >> 3;
        const int64_t p = (s >> 5) * 8 + (b & 7);
        const int w = (int)(s & 31);
        const int64_t nct = (int64_t)a.tiles_w + a.ntiles, nqc = (nct + 7) / 8;
        rb = (p / nqc) * 4 + (w & 3);
        const int64_t ct = (p % nqc) * 8 + (w >> 2);
        if (ct >= nct) return;  // slot past the last column tile (whole workgroup)
        if (ct < a.tiles_w) {
            wtile = true;
            n0 = ct * BN;
        } else {
            tile = (int)(ct - a.tiles_w);
        }
    } else if (a.ntiles > 1) {
        const int64_t grp = blockIdx.x / (8 * a.ntiles), rem = blockIdx.x % (8 * a.ntiles);
        tile = (int)(rem / 8);
        rb = grp * 8 + rem % 8;
    }
    const int64_t m0 = rb * BM;
    const int gen0 = tile * BN;
    // B operand rows of this tile that exist: generators, or columns of Y
    const int ktile = FUSED && wtile ? (int)min((int64_t)BN, a.d_out - n0) : min(BN, a.k - gen0);
    const int nst = (int)((a.d + E - 1) / E);
    const int npos = (nst + 1) & ~1;        // stage positions, padded to even
    const int last = nst - 1;
    const char* __restrict__ X = reinterpret_cast<const char*>(a.X);

    if (m0 >= a.n) return;  // slot past the last row block (whole workgroup)

    // |c|^2 of the tile's generators (-1 marks a padding generator of a
    // partial tile), fetched now and put in LDS with the first stage, so the
    // epilogue does not wait on it
    constexpr int CNV = (BN + NTH - 1) / NTH;
    float cn2v[CNV];
#pragma unroll
    for (int u = 0; u < CNV; ++u) {
        const int r = tid + u * NTH;
        cn2v[u] = !(FUSED && wtile) && r < ktile ? a.cn2[gen0 + r] : -1.0f;
    }
    int plain_gen = 1;

    // load i of a lane covers tile row (NTH/8)*i + tid/8 (8 lanes per row, one
    // 128-byte line per row and wave-wide load), 16-byte chunk tid%8.  Loads
    // address a wave-uniform base plus a 32-bit per-lane row offset (the
    // launcher only picks this kernel when X spans less than 4 GiB).
    const int qc = tid & 7;
    const int rsub = tid >> 3;
    uint32_t xoff[XPT], coff[CPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        int64_t g = m0 + (NTH / 8) * i + rsub;
        if (g >= a.n) g = a.n - 1;  // padding rows: any valid row, results unused
        xoff[i] = (uint32_t)((g - m0) * a.ldx_bytes);
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int jj = min((NTH / 8) * i + rsub, ktile - 1);  // padding generators: any valid one, masked later
        if (FUSED && wtile) {
            coff[i] = (uint32_t)((n0 + jj) * a.ldw_bytes);  // padding columns of Y: a valid row of W, unused
        } else {
            int64_t g = a.gen_idx[gen0 + jj];
            g = g < 0 ? 0 : (g >= a.n ? a.n - 1 : g);
            coff[i] = (uint32_t)(g * a.ldx_bytes);
        }
    }
    const char* __restrict__ Bsrc = FUSED && wtile ? reinterpret_cast<const char*>(a.W) : X;
    // LDS slot of load i: row (NTH/8)*i + rsub, chunk qc swizzled by the
    // row's key (the same for every i, so slot i is slot 0 plus a constant)
    const int dst0 = rsub * RB + ((qc ^ gemm_swz_key(rsub)) << 4);
    // stage at position p: workgroups start at different column ranges (as
    // above); positions past the last stage re-read it and are zeroed
    const int rot = PAMM_COMPRESS_ROTATE ? (int)(((uint64_t)rb * 37u) % (unsigned)nst) : 0;
    auto stage_of = [&](int p) { if (p >= nst) return last; int t = p + rot; return t >= nst ? t - nst : t; };
    const int tail_elems = (int)(a.d - (int64_t)last * E);
    auto valid_elems = [&](int p) { return p >= nst ? 0 : (stage_of(p) == last ? tail_elems : E); };
    const int64_t row_chunks = (a.row_bytes + 15) / 16;

    // the staged lines of a lane are handled in parts of four chunks: XP
    // parts of X, then CP parts of C
    constexpr int XP = XPT / 4, CP = CPT / 4, NP = XP + CP;
    static_assert(XPT % 4 == 0 && CPT % 4 == 0 && NP >= 2 && NP <= 4, "the stash is split in two to four parts");
    v4u32 xr[XPT], cr[CPT];
    // per-lane partial |x|^2 of the rows this lane fetches (summed by the
    // workgroups of the first generator tile only; |c|^2 comes from the
    // generator pass, gen_prep_kernel)
    float xsq[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) xsq[i] = 0.f;
    // fetch part `part` (four of the lane's 16 chunks: X for parts 0-1, C
    // for parts 2-3) of position p into registers
    auto issue_part = [&](int p, int part) __attribute__((always_inline)) {
        const int st = stage_of(p);
        // chunks past the row end (tail stage) re-read the row's last chunk;
        // without a tail stage the chunk offset is the same every stage
        const uint32_t q16 =
            MASKED ? (uint32_t)min((int64_t)qc, row_chunks - 1 - (int64_t)st * (RB / 16)) * 16u : (uint32_t)qc * 16u;
        if (part < XP) {
            const char* bx = X + m0 * a.ldx_bytes + (int64_t)st * RB;
#pragma unroll
            // non-temporal: the X lines need not stay in the memory-side cache
            // (other generator tiles of the row block re-read them from L2)
            for (int i = 4 * part; i < 4 * part + 4; ++i)
                xr[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(bx + (xoff[i] + q16)));
        } else {
            const char* bc = Bsrc + (int64_t)st * RB;
#pragma unroll
            for (int i = 4 * (part - XP); i < 4 * (part - XP) + 4; ++i)
                cr[i] = *reinterpret_cast<const v4u32*>(bc + (coff[i] + q16));
        }
    };
    auto issue = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int part = 0; part < NP; ++part) issue_part(p, part);
    };
    // registers of position p -> an LDS buffer.  Elements at or past the
    // position's valid count (the tail stage's columns past d, all of a
    // padding position) are cleared with per-lane masks: no branch.
    auto stage_mask = [&](int p) __attribute__((always_inline)) {
        const int lim = valid_elems(p) - qc * 8;  // valid elements of this lane's chunk
        v4u32 m;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            m[w] = (2 * w < lim ? 0x0000ffffu : 0u) | (2 * w + 1 < lim ? 0xffff0000u : 0u);
        return m;
    };
    auto stash_part = [&](const v4u32& m, char* buf, int part, auto wx) __attribute__((always_inline)) {
        if (part < XP) {
#pragma unroll
            for (int i = 4 * part; i < 4 * part + 4; ++i) {
                const v4u32 v = MASKED ? xr[i] & m : xr[i];
                *reinterpret_cast<v4u32*>(buf + dst0 + i * (NTH / 8) * RB) = v;
                if constexpr (decltype(wx)::value) xsq[i] = sumsq_dot2(v, xsq[i]);
            }
        } else {
#pragma unroll
            for (int i = 4 * (part - XP); i < 4 * (part - XP) + 4; ++i)
                *reinterpret_cast<v4u32*>(buf + BM * RB + dst0 + i * (NTH / 8) * RB) = MASKED ? cr[i] & m : cr[i];
        }
    };
    auto stash = [&](int p, char* buf, auto wx) __attribute__((always_inline)) {
        const v4u32 m = stage_mask(p);
#pragma unroll
        for (int part = 0; part < NP; ++part) stash_part(m, buf, part, wx);
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x16{};

    // fragment of 32x32x16: lane l holds row l%32 of the 32-row tile and
    // elements 8*(l/32) .. +7 of the 16-element K step.  Every tile row the
    // lane reads has row%32 = l%32, hence the same swizzle key, so a
    // fragment's LDS address is one base per K step plus compile-time offsets.
    const int frow = lane & 31, fk = lane >> 5;
    int fa[E / 16];
#pragma unroll
    for (int ks = 0; ks < E / 16; ++ks) fa[ks] = frow * RB + (((2 * ks + fk) ^ gemm_swz_key(frow)) << 4);
    const int xw = wr * WM * RB, cw = BM * RB + wc * WN * RB;
    auto load_frags = [&](const char* buf, int ks, v4u32 (&xf)[MT], v4u32 (&cf)[NT]) __attribute__((always_inline)) {
        const char* bx = buf + xw + fa[ks];
        const char* bc = buf + cw + fa[ks];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xf[mt] = *reinterpret_cast<const v4u32*>(bx + mt * 32 * RB);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) cf[nt] = *reinterpret_cast<const v4u32*>(bc + nt * 32 * RB);
    };
    auto mfma_step = [&](const v4u32 (&xf)[MT], const v4u32 (&cf)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, cf[nt]), __builtin_bit_cast(bf16x8, xf[mt]), acc[mt][nt], 0, 0, 0);

    };
    // One stage position: four K steps of 16 with two fragment register sets
    // in turn.  The schedule is skewed across the barrier: the fragments of
    // step 0 of position p+1 are read after the barrier while the MFMAs of
    // step 3 of position p run, so the barrier does not leave the matrix
    // cores waiting on LDS.  The stash of position p+1 and the fetch of
    // position p+2 are spread over the first three K steps' scheduling
    // regions, next to MFMAs of position p.
    // sched_barrier(0) fences keep the compiler from moving work across.
    v4u32 xa[MT], ca[NT], xb[MT], cb[NT];
    auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    // requested orders: one memory instruction per MFMA where there are
    // enough MFMAs, else the instructions spread evenly over them
    constexpr int NMF = MT * NT, NRD = MT + NT, NCS = 4 * (NP - 2);  // NCS: chunks staged in region 3
    auto order_part = [&]() __attribute__((always_inline)) {       // regions 1 and 2
        if constexpr (NMF >= NRD + 8) interleave_region<NRD, 4, 4, NMF - NRD - 8>();
        else interleave_spread<NRD, 4, 4, NMF>();
    };
    auto order_last_parts = [&]() __attribute__((always_inline)) {  // region 3
        if constexpr (NCS == 8 && NMF >= NRD + 8) interleave_region2<NRD, 8>();
        else if constexpr (NMF >= NRD + 2 * NCS) interleave_region<NRD, NCS, NCS, NMF - NRD - 2 * NCS>();
        else interleave_spread<NRD, NCS, NCS, NMF>();
    };
    auto order_reads = [&]() __attribute__((always_inline)) {       // region 4
        if constexpr (NMF >= NRD) interleave_region<NRD, 0, 0, NMF - NRD>();
        else interleave_spread<NRD, 0, 0, NMF>();
    };
    auto body = [&](int p, const char* cur, char* nxt, auto wx) __attribute__((always_inline)) {
        const v4u32 m = stage_mask(p + 1);
        const int pf = min(p + 2, npos - 1);
        load_frags(cur, 1, xb, cb);
        mfma_step(xa, ca);                     // step 0 (read before the last barrier)
        stash_part(m, nxt, 0, wx);
        issue_part(pf, 0);
        order_part();
        fence();
        load_frags(cur, 2, xa, ca);
        mfma_step(xb, cb);                     // step 1
        stash_part(m, nxt, 1, wx);
        issue_part(pf, 1);
        order_part();
        fence();
        load_frags(cur, 3, xb, cb);
        mfma_step(xa, ca);                     // step 2
#pragma unroll
        for (int part = 2; part < NP; ++part) {
            stash_part(m, nxt, part, wx);
            issue_part(pf, part);
        }
        order_last_parts();
        fence();
        wait_lds();
        ring_barrier();
        fence();
        load_frags(nxt, 0, xa, ca);            // step 0 of position p+1
        mfma_step(xb, cb);                     // step 3
        order_reads();
        fence();
    };
    auto tail = [&](const char* cur) __attribute__((always_inline)) {
        load_frags(cur, 1, xb, cb);
        mfma_step(xa, ca);
        fence();
        load_frags(cur, 2, xa, ca);
        mfma_step(xb, cb);
        fence();
        load_frags(cur, 3, xb, cb);
        mfma_step(xa, ca);
        fence();
        mfma_step(xb, cb);
    };
    static_assert(E / 16 == 4, "the skewed schedule is written for four K steps per stage");

    // the main loop, in two versions: with |x|^2 (first generator tile) or
    // without (the other tiles; their |x|^2 would be the same)
    auto run = [&](auto wx) __attribute__((always_inline)) {
        // distinct empty statements with a memory clobber open the two
        // versions: without them the compiler hoists their identical first
        // loads above the branch and spills the staged lines across it
        if constexpr (decltype(wx)::value)
            asm volatile("; norms" ::: "memory");
        else
            asm volatile("; no norms" ::: "memory");
        issue(0);
        stash(0, s_tile, wx);
#pragma unroll
        for (int u = 0; u < CNV; ++u) {
            const int r = tid + u * NTH;
            if (r < BN) {
                const float v = cn2v[u];
                s_cn2[r] = v;
                s_rinv[r] = v > 0.f ? 1.0f / sqrtf(v) : 0.f;
                s_floor[r] = v < 0.f ? -1.0f : 0.f;
                plain_gen &= v > 0.f && v < INFINITY;
            }
        }
        issue(1);
        wait_lds();
        ring_barrier();
        fence();
        load_frags(s_tile, 0, xa, ca);
        int p = 0;
        for (; p + 2 < npos; p += 2) {
            body(p, s_tile, s_tile + TILE, wx);
            body(p + 1, s_tile + TILE, s_tile, wx);
        }
        body(p, s_tile, s_tile + TILE, wx);
        tail(s_tile + TILE);
    };
    if (tile == 0 && !(FUSED && wtile))
        run(std::true_type{});
    else
        run(std::false_type{});

    // ---- epilogue (the stage ring is free now: every wave has passed the
    // last compute, so waves reuse it as scratch after one more barrier)
    __syncthreads();
    if constexpr (FUSED) {
        if (wtile) {
            store_y_tile<MT, NT, NWR, NWC>(a, acc, s_tile, m0, n0, wr, wc, lane, wave);
            return;
        }
    }
    float* ring = reinterpret_cast<float*>(s_tile);
    // norms: each lane's partial |x|^2 of its 8 rows go to LDS, one thread
    // per tile row adds the 8 chunks (zeros outside the first tile, where
    // they are not used); |c|^2 from the generator pass
#pragma unroll
    for (int i = 0; i < XPT; ++i) ring[((NTH / 8) * i + rsub) * 8 + qc] = xsq[i];
    __syncthreads();
    for (int r = tid; r < BM; r += NTH) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) v += ring[r * 8 + q];
        s_xn2[r] = v;
    }
    // tiles whose generators all have a finite, positive |c|^2 (no zero,
    // NaN or infinite norm, no padding) take the shorter scan below
    const bool plain = __syncthreads_and(plain_gen);
    // winners straight from the accumulators: element i of lane l in
    // acc[mt][nt] is S for row mt*32 + l%32 of the wave's rows and
    // generator nt*32 + 8*(i/4) + 4*(l/32) + i%4 of its generators, so a
    // lane scans its 16*NT generators of one row per mt in increasing
    // order (one chain per nt, merged in nt order: lowest index on ties,
    // NaN never wins), then meets lane l^32, which holds the others.
    const int jb = wc * WN + 4 * fk;  // tile index of the lane's generator for nt = i = 0
    auto gen_of = [](int nt, int i) { return nt * 32 + 8 * (i >> 2) + (i & 3); };
    auto publish = [&](int mt, float bs, int bg, float bd) __attribute__((always_inline)) {
        const float os = shfl_xor(bs, 32);
        const int og = shfl_xor(bg, 32);
        const float od = shfl_xor(bd, 32);
        const bool take = os > bs || (os == bs && og < bg);
        if (fk == 0) {
            const int rloc = wr * WM + mt * 32 + frow;
            s_ms[wc][rloc] = take ? os : bs;
            s_mg[wc][rloc] = take ? og : bg;
            s_md[wc][rloc] = take ? od : bd;
        }
    };
    if (plain) {
        // score = |S| / |c| with 1/|c| of the lane's generators in registers
        float w[NT][16];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 rv = *reinterpret_cast<const f32x4*>(s_rinv + jb + gen_of(nt, 4 * q));
#pragma unroll
                for (int e = 0; e < 4; ++e) w[nt][4 * q + e] = rv[e];
            }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float cs[NT], cd[NT];
            int cj[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                cs[nt] = -1.0f;
                cj[nt] = -1;
                cd[nt] = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float d = acc[mt][nt][i];
                    const float sc = fabsf(d) * w[nt][i];
                    const bool win = sc > cs[nt];  // false for NaN
                    cs[nt] = win ? sc : cs[nt];
                    cj[nt] = win ? gen_of(nt, i) : cj[nt];
                    cd[nt] = win ? d : cd[nt];
                }
            }
#pragma unroll
            for (int nt = 1; nt < NT; ++nt) {
                const bool win = cs[nt] > cs[0];
                cs[0] = win ? cs[nt] : cs[0];
                cj[0] = win ? cj[nt] : cj[0];
                cd[0] = win ? cd[nt] : cd[0];
            }
            publish(mt, cs[0], cj[0] < 0 ? 0x7fffffff : gen0 + jb + cj[0], cd[0]);
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float bs = -1.0f, bd = 0.f;
            int bg = 0x7fffffff;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j0 = jb + gen_of(nt, 4 * q);
                    const f32x4 cv = *reinterpret_cast<const f32x4*>(s_cn2 + j0);
                    const f32x4 rv = *reinterpret_cast<const f32x4*>(s_rinv + j0);
                    const f32x4 fv = *reinterpret_cast<const f32x4*>(s_floor + j0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // a padding generator (|c|^2 = -1) scores -1 and
                        // never wins; |c|^2 = 0 or NaN scores 0
                        const float d = acc[mt][nt][4 * q + e];
                        const float sc = cv[e] > 0.f ? fabsf(d) * rv[e] : fv[e];
                        const bool win = sc > bs;
                        bs = win ? sc : bs;
                        bg = win ? gen0 + j0 + e : bg;
                        bd = win ? d : bd;
                    }
                }
            publish(mt, bs, bg, bd);
        }
    }
    __syncthreads();
    // ---- one thread per row: merge the column winners, eps test, write
    for (int r = tid; r < BM; r += NTH) {
        const int64_t row = m0 + r;
        if (row >= a.n) continue;
        float bs = s_ms[0][r], bd = s_md[0][r];
        int bg = s_mg[0][r];
#pragma unroll
        for (int c = 1; c < NWC; ++c) {
            const float os = s_ms[c][r];
            const int og = s_mg[c][r];
            if (os > bs || (os == bs && og < bg)) { bs = os; bg = og; bd = s_md[c][r]; }
        }
        const bool found = bg != 0x7fffffff;
        float al = 0.f;
        if (found) {
            const float cn = s_cn2[bg - gen0];
            al = cn > 0.f ? bd / cn : 0.f;
        }
        const float xn2 = s_xn2[r];
        if (a.partial) {
            PartialBest pb;
            pb.score = found ? bs : -1.0f;
            pb.gen = found ? bg : -1;
            pb.alpha = al;
            a.partial[(int64_t)tile * a.n + row] = pb;
            if (tile == 0) a.xn2[row] = xn2;
        } else {
            const float cs = xn2 == 0.f ? 0.f : bs / sqrtf(xn2);
            const bool keep = found && cs >= a.eps;
            a.f[row] = keep ? bg : -1;
            a.alpha[row] = keep ? al : 0.f;
        }
    }
}

// Generator pass of the GEMM-shaped path: C = X[gen_idx] and |c_j|^2 (fp32
// dot2 sums of the stored bf16 values).  One 256-thread workgroup per
// generator row; each thread issues all its 16-byte chunk loads (up to 8)
// before using them, so a row costs about one memory round trip.
__global__ __launch_bounds__(256) void gen_prep_kernel(CompressArgs a) {
    constexpr int UNR = 8;
    __shared__ float s_part[4];
    const int tid = threadIdx.x;
    const char* __restrict__ X = reinterpret_cast<const char*>(a.X);
    const int64_t row_chunks = (a.d + 7) / 8;
    for (int64_t j = blockIdx.x; j < a.k; j += gridDim.x) {
        int64_t r = a.gen_idx[j];
        r = r < 0 ? 0 : (r >= a.n ? a.n - 1 : r);
        const char* src = X + r * a.ldx_bytes;
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.C) + j * a.d;
        float sum = 0.f;
        for (int64_t c0 = tid; c0 < row_chunks; c0 += 256 * UNR) {
            uint4 u[UNR];
#pragma unroll
            for (int t = 0; t < UNR; ++t) {
                const int64_t c = c0 + 256 * t;
                u[t] = c < row_chunks ? load16_tail<DT_BF16>(src, c * 8, a.d) : make_uint4(0, 0, 0, 0);  // zeros past d
            }
#pragma unroll
            for (int t = 0; t < UNR; ++t) {
                const int64_t c = c0 + 256 * t;
                const v4u32 v = {u[t].x, u[t].y, u[t].z, u[t].w};
                sum = sumsq_dot2(v, sum);
                if (c >= row_chunks) continue;
                if (a.c_vec_ok && c * 8 + 8 <= a.d) {
                    *reinterpret_cast<uint4*>(dst + c * 8) = u[t];
                } else {
                    for (int e = 0; e < 8 && c * 8 + e < a.d; ++e) dst[c * 8 + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += shfl_xor(sum, m);
        if ((tid & 63) == 0) s_part[tid >> 6] = sum;
        __syncthreads();
        if (tid == 0) a.cn2[j] = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
        __syncthreads();
    }
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

template <int MT, int NT, int NWR, int NWC>
static hipError_t launch_compress_gemm(const CompressArgs& a, int ntiles, hipStream_t st) {
    constexpr int BM = 32 * MT * NWR;
    const int64_t nrb = (a.n + BM - 1) / BM;
    const dim3 grid((unsigned)(ntiles > 1 ? (nrb + 7) / 8 * 8 * ntiles : nrb));
    const int64_t nst = (a.d + 63) / 64;
    if (a.d % 64 != 0 || nst % 2 != 0)
        hipLaunchKernelGGL((compress_gemm_kernel<MT, NT, NWR, NWC, true>), grid, dim3(64 * NWR * NWC), 0, st, a);
    else
        hipLaunchKernelGGL((compress_gemm_kernel<MT, NT, NWR, NWC, false>), grid, dim3(64 * NWR * NWC), 0, st, a);
    return hipGetLastError();
}

// Tile shapes per generator-tile width: rows per wave, waves, generators,
// register prefetch depth (stages), bytes of each row per stage.  The
// 8-wave tiles prefetch two stages: measured against four (same outputs),
// two took 0.5-1.5 us less at 7B and on the 1B sweep, and six or eight took
// more.  The 256-generator tile could not hold four anyway: its
// accumulators, fragments and ring would exceed the 256 registers a wave of
// a 512-thread workgroup may hold.  The 2-wave tiles for few rows keep four.
#ifndef PAMM_COMPRESS_FEW_PD
#define PAMM_COMPRESS_FEW_PD 4
#endif
#ifndef PAMM_COMPRESS_RS16
#define PAMM_COMPRESS_RS16 16, 8, 16, 2, 128
#endif
#ifndef PAMM_COMPRESS_RS32
#define PAMM_COMPRESS_RS32 16, 8, 32, 2, 128
#endif
#ifndef PAMM_COMPRESS_RS64
#define PAMM_COMPRESS_RS64 16, 8, 64, 2, 128
#endif
#ifndef PAMM_COMPRESS_RS128
#define PAMM_COMPRESS_RS128 16, 8, 128, 2, 128
#endif
#ifndef PAMM_COMPRESS_RS256
#define PAMM_COMPRESS_RS256 16, 8, 256, 2, 128
#endif
// bf16 tiles of 256 generators: rows and generators per wave (in 32s), waves
// along rows and along generators.
#ifndef PAMM_COMPRESS_GEMM
#define PAMM_COMPRESS_GEMM 4, 4, 2, 2
#endif
// with several generator tiles (k > 256): 2 x 4 waves of 128 rows x 64
// generators, two waves per SIMD, so that one wave's LDS and global traffic
// runs while the other's MFMAs do.  The X lines of a row block then come
// from L2 (its tiles run together on one XCD); with one tile, X streams from
// HBM and the 4-wave tile, with a third fewer LDS fragment reads, is faster.
#ifndef PAMM_COMPRESS_GEMM_MULTI
#define PAMM_COMPRESS_GEMM_MULTI 4, 2, 2, 4
#endif
// the same with 128-row blocks (2 x 2 waves of 64 rows x 128 generators), for
// inputs whose 256-row blocks leave compute units idle
#ifndef PAMM_COMPRESS_GEMM_HALF
#define PAMM_COMPRESS_GEMM_HALF 2, 4, 2, 2
#endif
#ifndef PAMM_COMPRESS_USE_GEMM
#define PAMM_COMPRESS_USE_GEMM 1
#endif

// The GEMM-shaped kernel addresses X with 32-bit offsets from a uniform
// base: every row offset, plus one stage, must stay below 4 GiB.  With one
// workgroup per compute unit it also needs at least as many (row block,
// generator tile) pairs as compute units: the 256-row blocks where they fill
// the device, else 128-row blocks where those do, else the 128-row kernel.
template <int MT, int NWR>
static bool gemm_pays(const CompressArgs& a, int ntiles) {
    constexpr int BM = 32 * MT * NWR;
    const int64_t nrb = (a.n + BM - 1) / BM;
    return (uint64_t)a.n * (uint64_t)a.ldx_bytes + 256u <= 0xffffffffull && nrb * ntiles >= a.num_cus;
}
template <int MT, int NT, int NWR, int NWC>
static bool gemm_pays_cfg(const CompressArgs& a, int ntiles) { return gemm_pays<MT, NWR>(a, ntiles); }

template <int DT>
static hipError_t compress_dispatch(const CompressArgs& a, int kn, int ntiles, hipStream_t st) {
    // Few rows (fewer 128-row blocks than compute units, e.g. GPT-2's 8192
    // tokens) and one small generator tile: 2-wave workgroups of 32 rows put
    // four times as many workgroups in flight, at the price of a generator
    // tile read per 32 rows instead of per 128 (2-8 KB per stage at k <= 64).
    // GPT-2 and the tiny fp32 case: compress ~20% faster.
    const bool few_rows = ntiles == 1 && (a.n + 127) / 128 < (int64_t)a.num_cus;
    constexpr int FP = PAMM_COMPRESS_FEW_PD;
    switch (kn) {
        case 16: return few_rows ? launch_compress_rs<DT, 16, 2, 16, FP, 128>(a, ntiles, st)
                                 : launch_compress_rs<DT, PAMM_COMPRESS_RS16>(a, ntiles, st);
        case 32: return few_rows ? launch_compress_rs<DT, 16, 2, 32, FP, 128>(a, ntiles, st)
                                 : launch_compress_rs<DT, PAMM_COMPRESS_RS32>(a, ntiles, st);
        case 64: return few_rows ? launch_compress_rs<DT, 16, 2, 64, FP, 128>(a, ntiles, st)
                                 : launch_compress_rs<DT, PAMM_COMPRESS_RS64>(a, ntiles, st);
        case 128: return launch_compress_rs<DT, PAMM_COMPRESS_RS128>(a, ntiles, st);
        default:
            if constexpr (DT == DT_BF16) {
                const bool full = gemm_pays_cfg<PAMM_COMPRESS_GEMM>(a, ntiles);
                if (PAMM_COMPRESS_USE_GEMM && a.cn2 && (full || gemm_pays_cfg<PAMM_COMPRESS_GEMM_HALF>(a, ntiles))) {
                    const unsigned pblocks = (unsigned)std::min<int64_t>(a.k, 4096);
                    hipLaunchKernelGGL(gen_prep_kernel, dim3(pblocks), dim3(256), 0, st, a);
                    const hipError_t e = hipGetLastError();
                    if (e != hipSuccess) return e;
                    if (!full) return launch_compress_gemm<PAMM_COMPRESS_GEMM_HALF>(a, ntiles, st);
                    return ntiles > 1 ? launch_compress_gemm<PAMM_COMPRESS_GEMM_MULTI>(a, ntiles, st)
                                      : launch_compress_gemm<PAMM_COMPRESS_GEMM>(a, ntiles, st);
                }
            }
            return launch_compress_rs<DT, PAMM_COMPRESS_RS256>(a, ntiles, st);
    }
}

// the fused pass re-reads each X panel from L2 for every column tile: the
// 8-wave tile, as for several generator tiles
#ifndef PAMM_FUSED_GEMM
#define PAMM_FUSED_GEMM 4, 2, 2, 4
#endif
template <int MT, int NT, int NWR, int NWC>
static hipError_t launch_forward(const CompressArgs& a0, hipStream_t st);

hipError_t run_forward_compress(const CompressArgs& a0, hipStream_t st) {
    return launch_forward<PAMM_FUSED_GEMM>(a0, st);
}

template <int MT, int NT, int NWR, int NWC>
static hipError_t launch_forward(const CompressArgs& a0, hipStream_t st) {
    constexpr int BM = 32 * MT * NWR, BN = 32 * NT * NWC;
    CompressArgs a = a0;
    a.ntiles = (int)((a.k + BN - 1) / BN);
    a.tiles_w = (int)((a.d_out + BN - 1) / BN);
    if (a.ntiles <= 1) { a.partial = nullptr; a.xn2 = nullptr; }
    if (a.k > 0) {
        const unsigned pblocks = (unsigned)std::min<int64_t>(a.k, 4096);
        hipLaunchKernelGGL(gen_prep_kernel, dim3(pblocks), dim3(256), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL(compress_empty_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, st, a.n, a.f,
                           a.alpha);
    }
    // groups of 4 row blocks x 8 column tiles, padded to a multiple of the 8 XCDs
    const int64_t nrb = (a.n + BM - 1) / BM;
    const int64_t ngroups = ((nrb + 3) / 4) * ((a.tiles_w + a.ntiles + 7) / 8);
    const dim3 grid((unsigned)((ngroups + 7) / 8 * 8 * 32));
    const int64_t nst = (a.d + 63) / 64;
    if (a.d % 64 != 0 || nst % 2 != 0)
        hipLaunchKernelGGL((compress_gemm_kernel<MT, NT, NWR, NWC, true, true>), grid, dim3(64 * NWR * NWC), 0, st, a);
    else
        hipLaunchKernelGGL((compress_gemm_kernel<MT, NT, NWR, NWC, false, true>), grid, dim3(64 * NWR * NWC), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ntiles <= 1) return e;
    hipLaunchKernelGGL(compress_merge_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, st, a.partial,
                       a.xn2, a.n, a.ntiles, a.eps, a.f, a.alpha);
    return hipGetLastError();
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
