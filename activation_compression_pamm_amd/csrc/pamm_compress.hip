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
//   * X and C (= rows gen_idx of X) stream through an NS-deep LDS ring with
//     direct global->LDS 16-byte loads (no VGPR round trip), 128 bytes of each
//     row per stage, XOR-swizzled so MFMA fragment reads avoid bank clashes.
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
// workspace and pamm_compress_merge picks the overall winner.
#include <type_traits>

#include "pamm_device.hpp"
#include "pamm_kernels.hpp"

namespace pamm {

namespace {

constexpr int kRowBytes = 128;  // bytes of every row staged per pipeline stage

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their maxima).
template <int N>
struct VmWait {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    static constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
};

template <int N>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(VmWait<N>::imm); }

// Workgroup barrier for the DMA ring.  Each wave has already waited for its
// own DMA of the stage (wait_vm) and, where it wrote LDS itself, for those
// stores (lgkmcnt 0), so the barrier needs no memory fence; a full
// __syncthreads() fence would also drain the DMA of later stages.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14)); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

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

// Byte offset in a staged tile of 16-byte chunk `q` (0..7) of tile row `r`.
__device__ __forceinline__ int swz(int r, int q) { return r * kRowBytes + ((q ^ (r & 7)) << 4); }

// Call f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace

template <int DT, int WM, int NW, int KN, int NS>
__global__ __launch_bounds__(64 * NW) void compress_kernel(CompressArgs a) {
    constexpr int BM = WM * NW;
    constexpr int MT = WM / 16;
    constexpr int NTL = KN / 16;
    constexpr int NDG = (NTL + NW - 1) / NW;
    constexpr int XLD = BM / (8 * NW);               // X dma per wave per stage
    constexpr int CLD = (KN + 8 * NW - 1) / (8 * NW);  // C dma per wave per stage (rounded up)
    constexpr int LPS = XLD + CLD;
    constexpr int E = kRowBytes / Elem<DT>::size;     // elements of a row per stage
    constexpr int P = Elem<DT>::per16;
    static_assert(BM % (8 * NW) == 0, "tile shape");
    static_assert((NS - 2) * LPS < 64, "vmcnt window");

    // One LDS object per ring slot: with the slot known at compile time the
    // compiler can tell a DMA into one slot from reads of another, and does
    // not drain the whole DMA queue before every LDS read.
    constexpr int CROWS = CLD * NW * 8;
    __shared__ __align__(16) char s_x0[BM * kRowBytes];
    __shared__ __align__(16) char s_x1[BM * kRowBytes];
    __shared__ __align__(16) char s_x2[BM * kRowBytes];
    __shared__ __align__(16) char s_x3[NS > 3 ? BM * kRowBytes : 16];
    __shared__ __align__(16) char s_c0[CROWS * kRowBytes];
    __shared__ __align__(16) char s_c1[CROWS * kRowBytes];
    __shared__ __align__(16) char s_c2[CROWS * kRowBytes];
    __shared__ __align__(16) char s_c3[NS > 3 ? CROWS * kRowBytes : 16];
    static_assert(NS == 3 || NS == 4, "ring depth");
    __shared__ float s_cn2[KN];
    __shared__ float s_rinv[KN];
    __shared__ float s_xn2[BM];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int gen0 = blockIdx.y * KN;
    const int ktile = min(KN, a.k - gen0);
    const int nst = (int)((a.d + E - 1) / E);
    const char* __restrict__ X = reinterpret_cast<const char*>(a.X);

    // ---- copy out the generator rows C = X[gen_idx] (spread over all workgroups)
    if (a.C) {
        const int64_t row_chunks = (a.d + P - 1) / P;
        const int64_t total = (int64_t)a.k * row_chunks;
        const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
        const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
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

    // ---- per-lane source rows for the DMA (fixed for the whole d loop)
    // DMA instruction `i` of this wave covers tile rows 8*(wave + NW*i) .. +8;
    // lane L of it lands in row 8*(...) + L/8, swizzled slot L%8, and fetches
    // chunk (L%8) ^ (row & 7) of that row.
    const char* xsrc[XLD];
    int xq[XLD];
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
        const int r = 8 * (wave + NW * i) + (lane >> 3);
        int64_t g = m0 + r;
        if (g >= a.n) g = a.n - 1;  // padding rows: any valid row, results unused
        xsrc[i] = X + g * a.ldx_bytes;
        xq[i] = (lane & 7) ^ (r & 7);
    }
    const char* csrc[CLD];
    int cq[CLD];
#pragma unroll
    for (int i = 0; i < CLD; ++i) {
        const int r = 8 * (wave + NW * i) + (lane >> 3);
        const int jj = min(r, max(ktile - 1, 0));  // padding generators: any valid one, masked later
        int64_t g = a.k > 0 ? a.gen_idx[gen0 + jj] : 0;
        g = g < 0 ? 0 : (g >= a.n ? a.n - 1 : g);
        csrc[i] = X + g * a.ldx_bytes;
        cq[i] = (lane & 7) ^ (r & 7);
    }

    auto xslot = [&](auto uc) -> char* {
        constexpr int U = decltype(uc)::value;
        if constexpr (U == 0) return s_x0;
        else if constexpr (U == 1) return s_x1;
        else if constexpr (U == 2) return s_x2;
        else return s_x3;
    };
    auto cslot = [&](auto uc) -> char* {
        constexpr int U = decltype(uc)::value;
        if constexpr (U == 0) return s_c0;
        else if constexpr (U == 1) return s_c1;
        else if constexpr (U == 2) return s_c2;
        else return s_c3;
    };
    auto issue = [&](int s, auto slotc) {
        char* sx = xslot(slotc);
        char* sc = cslot(slotc);
        const int64_t colb = (int64_t)s * kRowBytes;
#pragma unroll
        for (int i = 0; i < XLD; ++i) {
            int64_t off = colb + (xq[i] << 4);
            if (off >= a.row_bytes) off = 0;  // past the row end: fetch chunk 0, zeroed below
            dma16(xsrc[i] + off, sx + 8 * (wave + NW * i) * kRowBytes);
        }
#pragma unroll
        for (int i = 0; i < CLD; ++i) {
            int64_t off = colb + (cq[i] << 4);
            if (off >= a.row_bytes) off = 0;
            dma16(csrc[i] + off, sc + 8 * (wave + NW * i) * kRowBytes);
        }
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

    // the C copy-out above used vector memory; drain it so the DMA counts are exact
    wait_vm<0>();

    // ---- prologue: stages 0 .. NS-2
    static_for<0, NS - 1>([&](auto uc) {
        if (decltype(uc)::value < nst) issue(decltype(uc)::value, uc);
    });

    const int tail_elems = (int)(a.d - (int64_t)(nst - 1) * E);  // valid elements in the last stage

    for (int s0 = 0; s0 < nst; s0 += NS) {
        static_for<0, NS>([&](auto uc) {
            constexpr int U = decltype(uc)::value;
            const int s = s0 + U;
            if (s < nst) {
                char* sx = xslot(uc);
                char* sc = cslot(uc);
                // wait for this wave's DMA of stage s: stages s+1 .. min(s+NS-2, nst-1) may stay in flight
                const int ahead = min(NS - 2, nst - 1 - s);
                if constexpr (NS >= 4) {
                    if (ahead >= 2) wait_vm<2 * LPS>();
                    else if (ahead == 1) wait_vm<LPS>();
                    else wait_vm<0>();
                } else {
                    if (ahead >= 1) wait_vm<LPS>();
                    else wait_vm<0>();
                }
                ring_barrier();
                if (s == nst - 1 && tail_elems < E) {
                    // zero the elements past d in the last stage (both tiles)
                    for (int r = tid; r < BM + CROWS; r += 64 * NW) {
                        const int rr = r < BM ? r : r - BM;
                        char* row = r < BM ? sx + r * kRowBytes : sc + rr * kRowBytes;
                        for (int e = tail_elems; e < E; ++e) {
                            const int byte = e * Elem<DT>::size;
                            char* p = row + (((byte >> 4) ^ (rr & 7)) << 4) + (byte & 15);
                            if constexpr (DT == DT_BF16) *reinterpret_cast<uint16_t*>(p) = 0;
                            else *reinterpret_cast<uint32_t*>(p) = 0;
                        }
                    }
                    wait_lds();
                    ring_barrier();
                }
                if (s + NS - 1 < nst) issue(s + NS - 1, std::integral_constant<int, (U + NS - 1) % NS>{});

                // ---- compute stage s from ring slot U
#pragma unroll
                for (int sub = 0; sub < kRowBytes / 64; ++sub) {
                    const int q = sub * 4 + (lane >> 4);
                    uint4 xf[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int r = wave * WM + mt * 16 + (lane & 15);
                        xf[mt] = *reinterpret_cast<const uint4*>(sx + swz(r, q));
                        xsq[mt] += sumsq16<DT>(xf[mt]);
                    }
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) {
                        const int r = nt * 16 + (lane & 15);
                        const uint4 cf = *reinterpret_cast<const uint4*>(sc + swz(r, q));
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) mma16<DT>(xf[mt], cf, acc[mt][nt]);
                    }
                    // |c|^2: wave w squares generator tiles w, w+NW, ...  MFMA
                    // ignores the EXEC mask, so the tile is chosen through the
                    // LDS address, never through a lane-dependent branch.
#pragma unroll
                    for (int g = 0; g < NDG; ++g) {
                        const int nt = min(wave + g * NW, NTL - 1);
                        const uint4 cd = *reinterpret_cast<const uint4*>(sc + swz(nt * 16 + (lane & 15), q));
                        mma16<DT>(cd, cd, dacc[g]);
                    }
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
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float v = xsq[mt];
        v += shfl_xor(v, 16);
        v += shfl_xor(v, 32);
        if (lane < 16) s_xn2[wave * WM + mt * 16 + lane] = v;
    }
    __syncthreads();

    // ---- epilogue: per-row winner among this tile's generators
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rloc = wave * WM + mt * 16 + 4 * (lane >> 4) + i;
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
            const int64_t row = m0 + rloc;
            if ((lane & 15) == i && row < a.n) {
                const bool found = bg != 0x7fffffff;
                float al = 0.f;
                if (found) {
                    const float cn = s_cn2[bg - gen0];
                    al = cn > 0.f ? bd / cn : 0.f;
                }
                const float xn2 = s_xn2[rloc];
                if (a.partial) {
                    PartialBest pb;
                    pb.score = found ? bs : -1.0f;
                    pb.gen = found ? bg : -1;
                    pb.alpha = al;
                    a.partial[(int64_t)blockIdx.y * a.n + row] = pb;
                    if (blockIdx.y == 0) a.xn2[row] = xn2;
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

template <int DT, int WM, int NW, int KN, int NS>
static hipError_t launch_compress(const CompressArgs& a, int ntiles, hipStream_t st) {
    constexpr int BM = WM * NW;
    dim3 grid((unsigned)((a.n + BM - 1) / BM), (unsigned)ntiles);
    hipLaunchKernelGGL((compress_kernel<DT, WM, NW, KN, NS>), grid, dim3(64 * NW), 0, st, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t compress_dispatch(const CompressArgs& a, int kn, int ntiles, hipStream_t st) {
    switch (kn) {
        case 16: return launch_compress<DT, 32, 4, 16, 4>(a, ntiles, st);
        case 32: return launch_compress<DT, 32, 4, 32, 4>(a, ntiles, st);
        case 64: return launch_compress<DT, 32, 4, 64, 4>(a, ntiles, st);
        case 128: return launch_compress<DT, 32, 4, 128, 4>(a, ntiles, st);
        default: return launch_compress<DT, 16, 8, 256, 3>(a, ntiles, st);
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
    if (ntiles == 1) { b.partial = nullptr; b.xn2 = nullptr; }
    hipError_t e = dtype == DT_BF16 ? compress_dispatch<DT_BF16>(b, kn, ntiles, st)
                                    : compress_dispatch<DT_F32>(b, kn, ntiles, st);
    if (e != hipSuccess || ntiles == 1) return e;
    hipLaunchKernelGGL(compress_merge_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, st, a.partial,
                       a.xn2, a.n, ntiles, a.eps, a.f, a.alpha);
    return hipGetLastError();
}

}  // namespace pamm
