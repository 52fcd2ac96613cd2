// bf16 GEMM kernels for gfx950 (MI355X) matrix cores.
//
// These run the three local products of one GPU's FC-layer shard under the
// 3D parallel matrix multiply (sciencestack.ai/paper/2502.08145, Figure 1):
// Y = X.W, dX = dY.W^T and dW = X^T.dY, in bf16 with fp32 accumulation
// (mlsanity.com/paper/2502.08145, Abstract: bf16 training). The pages tuned
// vendor BLAS on A100, MI250X and H100; nothing of that design is reused here.
//
// Design (one workgroup = 256 threads = 4 wave64s, 2 x 2 waves):
//  * Block tile BM x BN, reduction step BK = 64. Each wave owns a
//    (BM/2) x (BN/2) sub-tile made of 32 x 32 blocks computed with
//    v_mfma_f32_32x32x16_bf16 (8 bf16 per lane per operand).
//  * Both operands are staged in LDS as [tile row][64 reduction values]
//    (128 B per row) so every MFMA operand is one 16-byte ds_read. The 16-byte
//    chunk index inside a row is XOR-swizzled with (row ^ row >> 3) & 7, so
//    that 32 lanes reading 32 consecutive rows, and the transposed writes
//    below, spread over the LDS banks.
//  * Two LDS stages: while the MFMAs consume stage s, the next reduction step
//    is already in flight from global memory into registers; it is written to
//    stage s^1 afterwards, and one barrier per step orders the two.
//  * Reduction-contiguous operands are fetched as 16-byte vectors along the
//    reduction. Output-contiguous operands (e.g. W stored K x N in the forward
//    product) are fetched as 8 x 8 sub-blocks, 16-byte vectors along the
//    output dimension, and transposed in registers before the LDS write.
//  * The MFMA is issued with the operands swapped (B fragment as source A), so
//    each lane's accumulators hold 4 consecutive output columns of one output
//    row: the epilogue writes 8-byte (bf16) or 16-byte (fp32) vectors.
//  * Block ids are remapped so that each of the 8 XCDs (which dispatch
//    workgroups round robin) works on one contiguous range of tiles, walked
//    in groups of 8 tile-rows, so that concurrent blocks on an XCD share A
//    and B panels in that XCD's L2.
//  * Split-K: blockIdx also enumerates reduction slices; each slice writes
//    fp32 partials that a separate kernel sums in a fixed order.
#include "fcshard_internal.h"

namespace fcs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;          // reduction elements per stage
constexpr int kRowBytes = 128;   // one LDS tile row: 64 bf16
constexpr int kThreads = 256;
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dispatched round robin
constexpr int kGroupM = 8;       // tile-rows per raster group

__device__ __forceinline__ int lds_offset(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// Reduction-contiguous operand: R tile rows x 64 reduction values.
// Thread t moves 16-byte chunks c = t + 256 j: row c / 8, chunk c % 8.
template <int R, bool ALIGNED>
struct LoaderRC {
    static constexpr int kPer = R * 8 / kThreads;
    u16x8 v[kPer];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                         int64_t rows, int64_t k0, int64_t kend, int tid) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int c = tid + j * kThreads;
            const int64_t gr = row0 + (c >> 3);
            const int64_t gk = k0 + ((c & 7) << 3);
            if (ALIGNED) {
                if (gr < rows && gk < kend) {
                    v[j] = *reinterpret_cast<const u16x8*>(p + gr * ld + gk);
                } else {
                    v[j] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[j][e] = (gr < rows && gk + e < kend) ? p[gr * ld + gk + e] : (uint16_t)0;
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int c = tid + j * kThreads;
            *reinterpret_cast<u16x8*>(lds + lds_offset(c >> 3, c & 7)) = v[j];
        }
    }
};

// Output-contiguous operand: R tile rows (output index) x 64 reduction values,
// stored in memory with the output index contiguous. Sub-block b covers tile
// rows 8 (b % (R/8)) .. +7 and reduction values 8 (b / (R/8)) .. +7; it is
// fetched as 8 vectors along the tile rows and transposed in registers.
template <int R, bool ALIGNED>
struct LoaderOC {
    static constexpr int kBlocks = R;  // (R / 8) * (64 / 8)
    static constexpr int kPer = (kBlocks + kThreads - 1) / kThreads;
    u16x8 v[kPer][8];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                         int64_t rows, int64_t k0, int64_t kend, int tid) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int b = tid + j * kThreads;
            if (kBlocks % kThreads != 0 && b >= kBlocks) break;
            const int64_t gi = row0 + ((b % (R / 8)) << 3);
            const int64_t gk = k0 + ((b / (R / 8)) << 3);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t r = gk + q;
                if (ALIGNED) {
                    if (r < kend && gi < rows) {
                        v[j][q] = *reinterpret_cast<const u16x8*>(p + r * ld + gi);
                    } else {
                        v[j][q] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[j][q][e] = (r < kend && gi + e < rows) ? p[r * ld + gi + e] : (uint16_t)0;
                }
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int b = tid + j * kThreads;
            if (kBlocks % kThreads != 0 && b >= kBlocks) break;
            const int i0 = (b % (R / 8)) << 3;
            const int kc = b / (R / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u16x8 w;
#pragma unroll
                for (int q = 0; q < 8; ++q) w[q] = v[j][q][e];
                *reinterpret_cast<u16x8*>(lds + lds_offset(i0 + e, kc)) = w;
            }
        }
    }
};

template <int R, bool OC, bool ALIGNED>
struct LoaderSel;
template <int R, bool ALIGNED>
struct LoaderSel<R, false, ALIGNED> {
    using type = LoaderRC<R, ALIGNED>;
};
template <int R, bool ALIGNED>
struct LoaderSel<R, true, ALIGNED> {
    using type = LoaderOC<R, ALIGNED>;
};

template <int BM, int BN, bool A_OC, bool B_OC, bool OUT_F32, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA blocks per wave
    constexpr int kStageBytes = (BM + BN) * kRowBytes;
    __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave >> 1) * WTM;
    const int wn0 = (wave & 1) * WTN;

    // ---- block id -> (slice, tile row, tile col)
    const int nbm = (int)((g.M + BM - 1) / BM);
    const int nbn = (int)((g.N + BN - 1) / BN);
    const int tiles = nbm * nbn;
    const int total = gridDim.x;
    const int lin = blockIdx.x;
    const int q = total / kXcds, rem = total % kXcds;
    const int xcd = lin % kXcds, loc = lin / kXcds;
    const int id = xcd * q + (xcd < rem ? xcd : rem) + loc;
    const int slice = id / tiles;
    const int pid = id - slice * tiles;
    const int per_group = kGroupM * nbn;
    const int first_m = (pid / per_group) * kGroupM;
    const int gsz = (nbm - first_m) < kGroupM ? (nbm - first_m) : kGroupM;
    const int tm = first_m + (pid % per_group) % gsz;
    const int tn = (pid % per_group) / gsz;
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    const int64_t kbeg = (int64_t)slice * g.k_split;
    const int64_t kend = (kbeg + g.k_split < g.K) ? kbeg + g.k_split : g.K;
    const int nkt = kend > kbeg ? (int)((kend - kbeg + kBK - 1) / kBK) : 0;

    typename LoaderSel<BM, A_OC, ALIGNED>::type la;
    typename LoaderSel<BN, B_OC, ALIGNED>::type lb;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nkt > 0) {
        la.load(g.A, g.lda, m0, g.M, kbeg, kend, tid);
        lb.load(g.B, g.ldb, n0, g.N, kbeg, kend, tid);
        la.store(smem, tid);
        lb.store(smem + BM * kRowBytes, tid);
        __syncthreads();
    }

    const int lr = lane & 31;  // row of the 32-row operand block this lane feeds
    const int lk = lane >> 5;  // which 8-value half of a 16-value reduction step

    for (int kt = 0; kt < nkt; ++kt) {
        const char* sA = smem + (kt & 1) * kStageBytes;
        const char* sB = sA + BM * kRowBytes;
        const bool more = kt + 1 < nkt;
        if (more) {
            const int64_t k0 = kbeg + (int64_t)(kt + 1) * kBK;
            la.load(g.A, g.lda, m0, g.M, k0, kend, tid);
            lb.load(g.B, g.ldb, n0, g.N, k0, kend, tid);
        }
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(sA + lds_offset(wm0 + i * 32 + lr, ks * 2 + lk));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(sB + lds_offset(wn0 + j * 32 + lr, ks * 2 + lk));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
        if (more) {
            char* nA = smem + ((kt + 1) & 1) * kStageBytes;
            la.store(nA, tid);
            lb.store(nA + BM * kRowBytes, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds C[m][n .. n+3] for each 32x32 block and group
    const int64_t ldc = g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm0 + i * 32 + lr;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int64_t n = n0 + wn0 + j * 32 + grp * 8 + lk * 4;
                const float v0 = acc[i][j][grp * 4 + 0], v1 = acc[i][j][grp * 4 + 1];
                const float v2 = acc[i][j][grp * 4 + 2], v3 = acc[i][j][grp * 4 + 3];
                if (OUT_F32) {
                    float* c = static_cast<float*>(g.C) + (int64_t)slice * g.c_split_stride + m * ldc + n;
                    if (ALIGNED) {
                        if (n < g.N) {
                            f32x4 v{v0, v1, v2, v3};
                            if (g.accumulate) v += *reinterpret_cast<const f32x4*>(c);
                            *reinterpret_cast<f32x4*>(c) = v;
                        }
                    } else {
                        const float vs[4] = {v0, v1, v2, v3};
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (n + q < g.N) c[q] = g.accumulate ? c[q] + vs[q] : vs[q];
                    }
                } else {
                    __bf16* c = static_cast<__bf16*>(g.C) + m * ldc + n;
                    const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
                    if (ALIGNED) {
                        if (n < g.N) {
                            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                            *reinterpret_cast<bf16x4*>(c) = bf16x4{b0, b1, b2, b3};
                        }
                    } else {
                        if (n + 0 < g.N) c[0] = b0;
                        if (n + 1 < g.N) c[1] = b1;
                        if (n + 2 < g.N) c[2] = b2;
                        if (n + 3 < g.N) c[3] = b3;
                    }
                }
            }
        }
    }
}

using KernelFn = void (*)(GemmArgs);

struct KernelEntry {
    KernelFn fn;
    const char* name;
};

#define FCS_STR2(x) #x
#define FCS_STR(x) FCS_STR2(x)
#define FCS_K(BM, BN, AOC, BOC, F32, AL)                                                        \
    KernelEntry {                                                                               \
        gemm_bf16_kernel<BM, BN, AOC, BOC, F32, AL>,                                            \
            "gemm_bf16_kernel<" #BM ", " #BN ", " #AOC ", " #BOC ", " #F32 ", " #AL ">"          \
    }
#define FCS_LAYOUTS(BM, BN, F32, AL)                                                            \
    FCS_K(BM, BN, false, false, F32, AL), FCS_K(BM, BN, false, true, F32, AL),                 \
        FCS_K(BM, BN, true, false, F32, AL), FCS_K(BM, BN, true, true, F32, AL)
#define FCS_TILE(BM, BN) FCS_LAYOUTS(BM, BN, false, true), FCS_LAYOUTS(BM, BN, true, true)

// [tile][out_f32][a_oc][b_oc] for the aligned kernels
const KernelEntry kAligned[kNumTiles * 8] = {
    FCS_TILE(256, 256),
    FCS_TILE(256, 128),
    FCS_TILE(128, 256),
    FCS_TILE(128, 128),
};
// [out_f32][a_oc][b_oc] for the unaligned kernels (tile kUnalignedTile)
const KernelEntry kUnaligned[8] = {
    FCS_LAYOUTS(128, 128, false, false),
    FCS_LAYOUTS(128, 128, true, false),
};

const KernelEntry& entry(int tile, bool a_oc, bool b_oc, bool out_f32, bool aligned) {
    const int lay = (a_oc ? 2 : 0) + (b_oc ? 1 : 0) + (out_f32 ? 4 : 0);
    return aligned ? kAligned[tile * 8 + lay] : kUnaligned[lay];
}

}  // namespace

const TileCfg kTiles[kNumTiles] = {
    {256, 256, "256x256"},
    {256, 128, "256x128"},
    {128, 256, "128x256"},
    {128, 128, "128x128"},
};

const char* gemm_kernel_name(int tile, bool a_oc, bool b_oc, bool out_f32, bool aligned) {
    return entry(tile, a_oc, b_oc, out_f32, aligned).name;
}

hipError_t launch_gemm(int tile, bool a_oc, bool b_oc, bool out_f32, bool aligned,
                       const GemmArgs& args, hipStream_t stream) {
    if (!aligned) tile = kUnalignedTile;
    const TileCfg& t = kTiles[tile];
    const int64_t nbm = (args.M + t.bm - 1) / t.bm;
    const int64_t nbn = (args.N + t.bn - 1) / t.bn;
    const int64_t blocks = nbm * nbn * (int64_t)args.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(entry(tile, a_oc, b_oc, out_f32, aligned).fn, dim3((unsigned)blocks), dim3(kThreads),
                       0, stream, args);
    return hipGetLastError();
}

}  // namespace fcs
