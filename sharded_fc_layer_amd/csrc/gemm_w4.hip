// 4-wave bf16 GEMM for gfx950 (MI355X), one wave per SIMD: the local
// products of one GPU's FC-layer shard under the 3D parallel matrix multiply
// (sciencestack.ai/paper/2502.08145, Figure 1), bf16 in with fp32
// accumulation (mlsanity.com/paper/2502.08145, Abstract: bf16 training).
//
// Requirements (checked by the caller): M, N multiples of 8, K and the
// split-K slice length multiples of 64, 16-byte aligned operands and output,
// every operand smaller than 2 GiB.
//
// Structure (256 threads = 4 wave64s in a 2 x 2 grid, 256 x 256 block tile):
//  * Each wave owns a 128 x 128 output tile: 8 x 8 blocks of
//    v_mfma_f32_16x16x32_bf16, 256 fp32 accumulators per lane. With one wave
//    per SIMD a wave has the SIMD's whole register file, so its tile is four
//    times that of an 8-wave kernel's wave, and each byte read from LDS feeds
//    twice the MFMA work (A and B fragments are each shared by 8 MFMAs).
//  * Reduction stages of 32 values in a ring of S = 4 LDS slots (128 KB),
//    filled by direct-to-LDS buffer loads issued S stages ahead; layouts and
//    swizzles are those of gemm_common.h.
//  * Stage t: the wave issues the LDS reads of stage t + 1 into the second
//    fragment register set while it runs the 64 MFMAs of stage t from the
//    first. Scheduling groups put one LDS read after each of the first MFMAs
//    and then spread the stage's loads evenly over the remaining MFMAs: a
//    burst of loads would fill the address unit's queue, and a wave stalled
//    on a load issue leaves its SIMD's MFMA pipe idle (one wave per SIMD).
//  * Barriers (template argument P): with P = 1 every stage opens with one.
//    Each wave first waits for its own loads of stage t + 1 and its LDS reads
//    of stage t (already in registers), then the barrier; after it the wave
//    issues the loads of stage t + S into stage t's slot, which every wave
//    has finished reading. With P = 2 only even stages open with a barrier:
//    it certifies stages t + 1 and t + 2 (the next two stages' LDS reads)
//    and frees the slots of stages t - 1 and t for the loads of t + 3 and
//    t + 4, which then have two stages of MFMA work to land. Half the
//    barriers, the same ring.
//  * The stage loop is unrolled twice (the two fragment register sets) with
//    no odd tail, so the reduction of every slice must be a multiple of 64.
//  * Every stage issues the same number of loads (the prefetches past the end
//    of the reduction reload its last stage into slots nobody reads), so "at
//    most two stages of loads in flight" is exactly "stage t + 1 has landed".
//    Output rows and columns past the matrix keep an out-of-range offset and
//    read zeros.
#include "gemm_common.h"

namespace fcs {

namespace {

constexpr int kW4Threads = 256;

template <bool A_OC, bool B_OC, bool OUT_F32, int P>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4_kernel(
    GemmArgs g) {
    static_assert(P == 1 || P == 2, "a barrier every stage or every second stage");
    constexpr int BM = 256, BN = 256, MF = 16;
    constexpr int TM = 8, TN = 8;  // 16 x 16 blocks per wave tile
    constexpr int BKP = 32, S = 4;
    constexpr int kABytes = BM * BKP * 2, kBBytes = BN * BKP * 2;
    constexpr int kStageBytes = kABytes + kBBytes;
    constexpr int kLoads = DmaPP<A_OC, BKP>::kInstr + DmaPP<B_OC, BKP>::kInstr;  // per wave per stage
    // P = 1: the barrier before stage t lets stage t + 1 be read and frees
    // stage t's slot for stage t + S (two stages of loads stay in flight).
    // P = 2: the barrier before an even stage t lets stages t + 1 and t + 2
    // be read and frees the slots of t - 1 and t for stages t + 3 and t + 4,
    // which have the two stages up to the next barrier to land.
    constexpr int kInFlight = P == 1 ? (S - 2) * kLoads : 0;
    constexpr int kReads = (A_OC ? 2 : 1) * TM + (B_OC ? 2 : 1) * TN;  // LDS read instructions per stage
    __shared__ __attribute__((aligned(1024))) char smem[S * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave >> 1) * 128;
    const int wn0 = (wave & 1) * 128;

    const BlockTile bt = map_block<BM, BN>(g);
    const int slice = bt.slice;
    const int64_t m0 = bt.m0, n0 = bt.n0;

    const int64_t kbeg = (int64_t)slice * g.k_split;
    const int64_t kend = (kbeg + g.k_split < g.K) ? kbeg + g.k_split : g.K;
    const int nkt = kend > kbeg ? (int)((kend - kbeg + BKP - 1) / BKP) : 0;

    const int64_t a_rows = A_OC ? g.K : g.M;  // storage rows of each operand
    const int64_t b_rows = B_OC ? g.K : g.N;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, (int)(a_rows * g.lda * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)g.B, 0, (int)(b_rows * g.ldb * 2), kRsrcWord3);
    DmaPP<A_OC, BKP> da;
    DmaPP<B_OC, BKP> db;
    da.init(wave, lane, g.lda, m0, g.M);
    db.init(wave, lane, g.ldb, n0, g.N);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    bf16x8 fa[2][TM], fb[2][TN];

    // Stage SIDX into its ring slot. Stages past the end (the last S - 1
    // prefetches, never read) reload the last stage instead, so every load
    // stays inside its operand and no reduction check is needed.
#define FCW4_ISSUE(SIDX)                                                                  \
    {                                                                                     \
        char* st_ = smem + ((SIDX) % S) * kStageBytes;                                    \
        const int64_t k0_ = kbeg + (int64_t)((SIDX) < nkt ? (SIDX) : nkt - 1) * BKP;      \
        da.issue_full(ra, st_, (uint32_t)(A_OC ? k0_ * g.lda * 2 : k0_ * 2), wave);       \
        db.issue_full(rb, st_ + kABytes, (uint32_t)(B_OC ? k0_ * g.ldb * 2 : k0_ * 2), wave); \
    }
#define FCW4_READ(T, BUF)                                                                                    \
    {                                                                                                        \
        const char* st_ = smem + ((T) % S) * kStageBytes;                                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[BUF][i] =                                          \
            fragment_mf<A_OC, BKP, MF>(st_, wm0 + i * MF, 0, lane);                                          \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[BUF][j] =                                          \
            fragment_mf<B_OC, BKP, MF>(st_ + kABytes, wn0 + j * MF, 0, lane);                                \
    }
    // one stage: T uses fragment set CUR and reads stage T + 1 into set NXT;
    // SYNC: the stage opens with the barrier (and the loads it allows)
#define FCW4_STAGE(T, CUR, NXT, SYNC)                                                                        \
    {                                                                                                        \
        constexpr int nl_ = (SYNC) ? P * kLoads : 0;                                                         \
        constexpr int gap_ = nl_ > 0 ? (TM * TN - kReads) / nl_ : 1;                                         \
        if constexpr (SYNC) {                                                                                \
            waitcnt<kInFlight, 0>();                                                                         \
            __builtin_amdgcn_s_barrier();                                                                    \
            __builtin_amdgcn_sched_barrier(0);                                                               \
        }                                                                                                    \
        FCW4_READ((T) + 1, NXT)                                                                              \
        if constexpr (SYNC) {                                                                                \
            if constexpr (P == 1) {                                                                          \
                FCW4_ISSUE((T) + S)                                                                          \
            } else {                                                                                         \
                FCW4_ISSUE((T) + 3)                                                                          \
                FCW4_ISSUE((T) + 4)                                                                          \
            }                                                                                                \
        }                                                                                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) _Pragma("unroll") for (int j = 0; j < TN; ++j)        \
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[CUR][j], fa[CUR][i], acc[i][j], 0, 0, 0); \
        _Pragma("unroll") for (int u = 0; u < TM * TN; ++u) {                                                \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                               \
            if (u < kReads)                                                                                  \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
            else if ((u - kReads) % gap_ == 0 && (u - kReads) / gap_ < nl_)                                  \
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                           \
        }                                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                                   \
    }

    if (nkt > 0) {
        constexpr int kPrologue = P == 1 ? S : S - 1;  // stages requested before the loop
#pragma unroll
        for (int s = 0; s < kPrologue; ++s) FCW4_ISSUE(s)
        waitcnt<(kPrologue - 1) * kLoads, 0>();
        __builtin_amdgcn_s_barrier();
        FCW4_READ(0, 0)
        for (int t = 0; t < nkt; t += 2) {  // nkt is even: the reduction is a multiple of 64
            FCW4_STAGE(t, 0, 1, true)
            FCW4_STAGE(t + 1, 1, 0, P == 1)
        }
        waitcnt<0, 0>();  // drain the trailing (out-of-range) loads
    }
#undef FCW4_ISSUE
#undef FCW4_READ
#undef FCW4_STAGE

    store_tile<MF, TM, TN, OUT_F32>(g, slice, m0, n0, wm0, wn0, lane, acc);
}

// Explicit instantiations: the host pass must emit a launch stub for every
// instance the table below names.
template __global__ void gemm_w4_kernel<false, false, false, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<false, false, false, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<false, true, false, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<false, true, false, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<true, false, false, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<true, false, false, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<true, true, false, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<true, true, false, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<false, false, true, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<false, false, true, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<false, true, true, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<false, true, true, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<true, false, true, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<true, false, true, 2>(GemmArgs);
template __global__ void gemm_w4_kernel<true, true, true, 1>(GemmArgs);
template __global__ void gemm_w4_kernel<true, true, true, 2>(GemmArgs);

using KernelFn = void (*)(GemmArgs);
struct W4Entry {
    KernelFn fn;
    const char* name;
};

#define FCW4_K(AOC, BOC, F32, P) \
    W4Entry { gemm_w4_kernel<AOC, BOC, F32, P>, "gemm_w4_kernel<" #AOC ", " #BOC ", " #F32 ", " #P ">" }
#define FCW4_ALL(P)                                                                                  \
    FCW4_K(false, false, false, P), FCW4_K(false, true, false, P), FCW4_K(true, false, false, P),     \
        FCW4_K(true, true, false, P), FCW4_K(false, false, true, P), FCW4_K(false, true, true, P),    \
        FCW4_K(true, false, true, P), FCW4_K(true, true, true, P)
// [barrier every P stages, P - 1][out_f32][a_oc][b_oc]
const W4Entry kW4[2][8] = {{FCW4_ALL(1)}, {FCW4_ALL(2)}};

const W4Entry& w4_entry(int variant, bool a_oc, bool b_oc, bool out_f32) {
    return kW4[variant & 1][(out_f32 ? 4 : 0) + (a_oc ? 2 : 0) + (b_oc ? 1 : 0)];
}

}  // namespace

const char* w4_kernel_name(int variant, bool a_oc, bool b_oc, bool out_f32) {
    return w4_entry(variant, a_oc, b_oc, out_f32).name;
}

hipError_t launch_gemm_w4(int variant, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                          hipStream_t stream) {
    const int64_t blocks = ((args.M + 255) / 256) * ((args.N + 255) / 256) * (int64_t)args.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(w4_entry(variant, a_oc, b_oc, out_f32).fn, dim3((unsigned)blocks), dim3(kW4Threads), 0, stream,
                       args);
    return hipGetLastError();
}

}  // namespace fcs
