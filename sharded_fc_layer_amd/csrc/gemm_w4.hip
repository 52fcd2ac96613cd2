// 4-wave bf16 GEMMs for gfx950 (MI355X), one wave per SIMD: the local
// products of one GPU's FC-layer shard under the 3D parallel matrix multiply
// (sciencestack.ai/paper/2502.08145, Figure 1), bf16 in with fp32
// accumulation (mlsanity.com/paper/2502.08145, Abstract: bf16 training).
//
// Requirements (checked by the caller): M, N, K multiples of 8, the split-K
// slice length a multiple of 64, K too for the 32-value-stage kernel (the
// others run a partial last stage: the two-slot kernel on operands padded
// with zeros, the rings by themselves), 16-byte aligned operands and output,
// every operand smaller than 2 GiB.
//
// Common structure (256 threads = 4 wave64s in a 2 x 2 grid, 256 x 256 tile):
//  * Each wave owns a 128 x 128 output tile: 8 x 8 blocks of
//    v_mfma_f32_16x16x32_bf16, 256 fp32 accumulators per lane. With one wave
//    per SIMD a wave has the SIMD's whole register file, so its tile is four
//    times that of an 8-wave kernel's wave, and each byte read from LDS feeds
//    twice the MFMA work (A and B fragments are each shared by 8 MFMAs).
//  * Operands reach LDS through direct-to-LDS buffer loads; layouts and
//    swizzles are those of gemm_common.h.
//  * Two fragment register sets: the wave issues the LDS reads of the next
//    32-value reduction step into one set while it runs the 64 MFMAs of the
//    current step from the other. Scheduling groups put one LDS read after
//    each of the first MFMAs and then spread the loads evenly over the
//    remaining MFMAs: a burst of loads would fill the address unit's queue,
//    and a wave stalled on a load issue leaves its SIMD's MFMA pipe idle.
//  * Stages past the end of the reduction (prefetches nobody reads) reload
//    the last stage, so every load stays inside its operand and each stage
//    issues the same number of loads; output rows and columns past the
//    matrix keep an out-of-range offset and read zeros.
//
// gemm_w4_kernel: stages of 32 values in a ring of 4 slots (128 KB). Each
// stage opens with a barrier: every wave first waits for its own loads of
// stage t + 1 and its LDS reads of stage t (already in registers); after the
// barrier it issues the loads of stage t + 4 into stage t's slot, which every
// wave has finished reading. Loads have three stages of MFMA work to land.
//
// gemm_w4k64_kernel: stages of 64 values (reduction-contiguous tile rows are
// then one whole 128-byte cache line; with 64-byte rows every line is fetched
// from L2 twice) in two slots of 64 KB; each operand tile of each slot is its
// own __shared__ array so that the compiler can tell the loads into one from
// the reads of another (and waits only where a read needs them). A stage
// is two 32-value steps; the barrier sits before the second: it certifies
// stage t + 1 (whose first step the wave reads next) and frees stage t's
// slot for the loads of stage t + 2, which have two steps to land.
// The ring variant (gemm_w4k64r_kernel, and its stamped form) lives in
// gemm_w4_ring_impl.h with its body in gemm_w4_ring_body.inc, built per
// block-tile width and tile split in gemm_w4_ring256.hip, gemm_w4_ring192.hip,
// gemm_w4_ring256b.hip and gemm_w4_ring192b.hip.
#include <algorithm>

#include "gemm_w4_common.h"

namespace fcs {

namespace {

#define FCW4_MFMA_STEP(SET)                                                                          \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) _Pragma("unroll") for (int j = 0; j < 8; ++j)      \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[SET][j], fa[SET][i], acc[i][j], 0, 0, 0);

template <bool A_OC, bool B_OC, bool OUT_F32>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4_kernel(
    GemmArgs g) {
    constexpr int MF = 16, BKP = 32, S = 4;
    constexpr int kABytes = 256 * BKP * 2;
    constexpr int kStageBytes = 2 * kABytes;
    constexpr int kLoads = DmaPP<A_OC, BKP>::kInstr + DmaPP<B_OC, BKP>::kInstr;  // per wave per stage
    constexpr int kInFlight = (S - 2) * kLoads;
    constexpr int kReads = (A_OC ? 16 : 8) + (B_OC ? 16 : 8);  // LDS read instructions per step
    __shared__ __attribute__((aligned(1024))) char smem[S * kStageBytes];

    const W4Setup w = w4_setup<A_OC, B_OC, BKP>(g);
    const int lane = w.lane, wave = w.wave, wm0 = w.wm0, wn0 = w.wn0, nkt = w.nkt;
    DmaPP<A_OC, BKP> da;
    DmaPP<B_OC, BKP> db;
    da.init(wave, lane, g.lda, w.m0, g.M);
    db.init(wave, lane, g.ldb, w.n0, g.N);

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 fa[2][8], fb[2][8];

#define FCW4_ISSUE(SIDX)                                                                          \
    {                                                                                             \
        char* st_ = smem + ((SIDX) % S) * kStageBytes;                                            \
        const int64_t k0_ = w.kbeg + (int64_t)((SIDX) < nkt ? (SIDX) : nkt - 1) * BKP;            \
        da.issue_full(w.ra, st_, (uint32_t)(A_OC ? k0_ * g.lda * 2 : k0_ * 2), wave);             \
        db.issue_full(w.rb, st_ + kABytes, (uint32_t)(B_OC ? k0_ * g.ldb * 2 : k0_ * 2), wave);   \
    }
#define FCW4_READ(T, SET)                                                                                 \
    {                                                                                                     \
        const char* st_ = smem + ((T) % S) * kStageBytes;                                                 \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) fa[SET][i] =                                        \
            fragment_mf<A_OC, BKP, MF>(st_, wm0 + i * MF, 0, lane);                                       \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) fb[SET][j] =                                        \
            fragment_mf<B_OC, BKP, MF>(st_ + kABytes, wn0 + j * MF, 0, lane);                             \
    }
    // stage T from fragment set CUR; reads stage T + 1 into set NXT
#define FCW4_STAGE(T, CUR, NXT)                  \
    {                                            \
        waitcnt<kInFlight, 0>();                 \
        __builtin_amdgcn_s_barrier();            \
        __builtin_amdgcn_sched_barrier(0);       \
        FCW4_READ((T) + 1, NXT)                  \
        FCW4_ISSUE((T) + S)                      \
        FCW4_MFMA_STEP(CUR)                      \
        w4_interleave<kReads, kLoads>();         \
        __builtin_amdgcn_sched_barrier(0);       \
    }

    if (nkt > 0) {
#pragma unroll
        for (int s = 0; s < S; ++s) FCW4_ISSUE(s)
        waitcnt<(S - 1) * kLoads, 0>();
        __builtin_amdgcn_s_barrier();
        FCW4_READ(0, 0)
        for (int t = 0; t < nkt; t += 2) {  // nkt is even: the reduction is a multiple of 64
            FCW4_STAGE(t, 0, 1)
            FCW4_STAGE(t + 1, 1, 0)
        }
        waitcnt<0, 0>();  // drain the trailing prefetches
    }
#undef FCW4_ISSUE
#undef FCW4_READ
#undef FCW4_STAGE

    // the tiles become staging space: every wave's loads must have landed
    // and its LDS reads finished before any wave writes there
    waitcnt<0, 0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (OUT_F32)
        store_tile_f32_staged(g, w.slice, w.m0, w.n0, wm0, wn0, lane, acc, smem + wave * (128 * 256));
    else
        store_tile_bf16_staged(g, w.m0, w.n0, wm0, wn0, lane, acc, smem + wave * (128 * 256));
}

template <bool A_OC, bool B_OC, bool OUT_F32, int BN>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4k64_kernel(
    GemmArgs g) {
    constexpr int MF = 16, BKP = 64;
    constexpr int TN = BN / 32;                                                  // 16-column blocks per wave
    constexpr int kABytes = 256 * BKP * 2;                                       // 32 KB per operand tile
    constexpr int kLA = DmaPP<A_OC, BKP>::kInstr;                                // 8
    constexpr int kLoads = kLA + DmaPP<B_OC, BKP, BN>::kInstr;                   // per wave per stage
    // one array per slot and operand: the compiler tracks each array's
    // direct-to-LDS writes separately, so an LDS read waits only for the
    // loads into the array it reads. B tiles narrower than 256 rows keep
    // 32 KB arrays: each array is one wave's epilogue staging space.
    __shared__ __attribute__((aligned(1024))) char a0[kABytes];
    __shared__ __attribute__((aligned(1024))) char b0[kABytes];
    __shared__ __attribute__((aligned(1024))) char a1[kABytes];
    __shared__ __attribute__((aligned(1024))) char b1[kABytes];

    const W4Setup w = w4_setup<A_OC, B_OC, BKP, BN>(g);
    const int lane = w.lane, wave = w.wave, wm0 = w.wm0, wn0 = w.wn0, nkt = w.nkt;
    DmaPP<A_OC, BKP> da;
    DmaPP<B_OC, BKP, BN> db;
    da.init(wave, lane, g.lda, w.m0, g.M);
    db.init(wave, lane, g.ldb, w.n0, g.N);

    // zeroed by MFMAs once the first stage's loads are on their way (w4_acc_zero)
    f32x4 acc[8][TN];
    bf16x8 fa[2][8], fb[2][TN];

    // byte offsets of stage SIDX along the reduction (past the end: the last stage)
#define FCW64_STEPS(SIDX)                                                                  \
    const int64_t k0_ = w.kbeg + (int64_t)((SIDX) < nkt ? (SIDX) : nkt - 1) * BKP;         \
    const uint32_t sa_ = (uint32_t)(A_OC ? k0_ * g.lda * 2 : k0_ * 2);                     \
    const uint32_t sb_ = (uint32_t)(B_OC ? k0_ * g.ldb * 2 : k0_ * 2);

#define FCW64_ISSUE(SA, SB, SIDX)                        \
    {                                                    \
        FCW64_STEPS(SIDX)                                \
        da.issue_full(w.ra, SA, sa_, wave);              \
        db.issue_full(w.rb, SB, sb_, wave);              \
    }
    // one 32-value step: 8 TN MFMAs from set CUR, interleaved (w64_read_after,
    // w64_load_after) with the LDS reads of the fragments of step KS of slot
    // (RA, RB) into set NXT and the loads LOADS selects (bit 0: operand A into
    // LA, bit 1: operand B into LB) of stage LSTAGE
#define FCW64_STEP(CUR, NXT, RA, RB, KS, LOADS, LA, LB, LSTAGE)                                        \
    {                                                                                                  \
        FCW64_STEPS(LSTAGE)                                                                            \
        constexpr int la_ = ((LOADS) & 1) ? kLA : 0;                                                   \
        constexpr int nl_ = la_ + (((LOADS) & 2) ? kLoads - kLA : 0);                                  \
        _Pragma("unroll") for (int u = 0; u < 8 * TN; ++u) {                                           \
            mfma_agpr(acc[u / TN][u % TN], fb[CUR][u % TN], fa[CUR][u / TN]);                          \
            const int r_ = w64_read_after<TN>(nl_, u);                                                 \
            if (r_ >= 0 && r_ < 8) {                                                                   \
                fa[NXT][r_] = fragment_mf<A_OC, BKP, MF>(RA, wm0 + r_ * MF, KS, lane);                 \
            } else if (r_ >= 8) {                                                                      \
                fb[NXT][r_ - 8] = fragment_mf<B_OC, BKP, MF, BN>(RB, wn0 + (r_ - 8) * MF, KS, lane);   \
            }                                                                                          \
            const int l_ = w64_load_after<TN>(nl_, u);                                                 \
            if (l_ >= 0 && l_ < la_)                                                                   \
                da.issue_one(w.ra, LA, sa_, wave, l_);                                                 \
            else if (l_ >= la_)                                                                        \
                db.issue_one(w.rb, LB, sb_, wave, l_ - la_);                                           \
        }                                                                                              \
    }
    // stage T in slot (XA, XB), stage T + 1 in slot (YA, YB). Step 1 opens with
    // the barrier that certifies stage T + 1 and frees slot X (its last reads,
    // of step 1, were issued during step 0), then loads stage T + 2 into slot X.
    // (Splitting a stage's loads over both steps halved the time they had to
    // land and was slower.)
#define FCW64_STAGE(T, XA, XB, YA, YB)                                                    \
    {                                                                                     \
        FCW64_STEP(0, 1, XA, XB, 1, 0, YA, YB, (T) + 1)                                   \
        waitcnt<0, 0>();                                                                  \
        __builtin_amdgcn_s_barrier();                                                     \
        FCW64_STEP(1, 0, YA, YB, 0, 3, XA, XB, (T) + 2)                                   \
    }

    if (nkt > 0) {
        FCW64_ISSUE(a0, b0, 0)
        w4_acc_zero(acc);
        FCW64_ISSUE(a1, b1, 1)
        waitcnt<kLoads, 0>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[0][i] = fragment_mf<A_OC, BKP, MF>(a0, wm0 + i * MF, 0, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[0][j] = fragment_mf<B_OC, BKP, MF, BN>(b0, wn0 + j * MF, 0, lane);
        w4_acc_fence(acc);  // zeroed accumulators before the first MFMA reads them
        for (int t = 0; t < nkt; t += 2) {     // nkt is even: the reduction is a multiple of 128
            FCW64_STAGE(t, a0, b0, a1, b1)
            FCW64_STAGE(t + 1, a1, b1, a0, b0)
        }
        waitcnt<0, 0>();  // drain the trailing prefetches
    } else {
        w4_acc_zero(acc);
    }
#undef FCW64_STEPS
#undef FCW64_ISSUE
#undef FCW64_STEP
#undef FCW64_STAGE
    w4_acc_drain(acc);  // the last MFMAs must have written their results before the epilogue reads them

    // the tiles become staging space: every wave's loads must have landed
    // and its LDS reads finished before any wave writes there
    waitcnt<0, 0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (OUT_F32)
        store_tile_f32_staged(g, w.slice, w.m0, w.n0, wm0, wn0, lane, acc, wave == 0 ? a0 : wave == 1 ? b0 : wave == 2 ? a1 : b1);
    else
        store_tile_bf16_staged(g, w.m0, w.n0, wm0, wn0, lane, acc, wave == 0 ? a0 : wave == 1 ? b0 : wave == 2 ? a1 : b1);
}
#undef FCW4_MFMA_STEP

// Explicit instantiations: the host pass must emit a launch stub for every
// instance the table below names.
#define FCW4_INST(AOC, BOC, F32)                                               \
    template __global__ void gemm_w4_kernel<AOC, BOC, F32>(GemmArgs);          \
    template __global__ void gemm_w4k64_kernel<AOC, BOC, F32, 256>(GemmArgs);  \
    template __global__ void gemm_w4k64_kernel<AOC, BOC, F32, 192>(GemmArgs);
FCW4_INST(false, false, false)
FCW4_INST(false, true, false)
FCW4_INST(true, false, false)
FCW4_INST(true, true, false)
FCW4_INST(false, false, true)
FCW4_INST(false, true, true)
FCW4_INST(true, false, true)
FCW4_INST(true, true, true)
#undef FCW4_INST

#define FCW4_K(KN, AOC, BOC, F32) \
    W4Kernel { KN<AOC, BOC, F32>, #KN "<" #AOC ", " #BOC ", " #F32 ">" }
#define FCW4_2S(BN, AOC, BOC, F32) \
    W4Kernel { gemm_w4k64_kernel<AOC, BOC, F32, BN>, "gemm_w4k64_kernel<" #AOC ", " #BOC ", " #F32 ", " #BN ">" }
#define FCW4_ALL(K, X)                                                                   \
    K(X, false, false, false), K(X, false, true, false), K(X, true, false, false),       \
        K(X, true, true, false), K(X, false, false, true), K(X, false, true, true),      \
        K(X, true, false, true), K(X, true, true, true)
// [kernel][out_f32][a_oc][b_oc]: the 32-value-stage kernel; the two-slot
// kernel with 256- and 192-column block tiles
const W4Kernel kW4[3][8] = {{FCW4_ALL(FCW4_K, gemm_w4_kernel)}, {FCW4_ALL(FCW4_2S, 256)}, {FCW4_ALL(FCW4_2S, 192)}};
#undef FCW4_K
#undef FCW4_2S
#undef FCW4_ALL

// The ring kernel's head for this launch: the reduction slices' stage count
// mod 6 when it is 2 or 4 for every slice and every slice has a whole period
// after its head, else -1 (pad at the front). The kernel tables map head
// forms that are not built (they would spill) to the padded form. A
// reduction that is not a multiple of 64 takes the padded form, which runs
// its partial last stage in the place of the first virtual stage.
int ring_head(int64_t K, int64_t k_split, int splits) {
    if (K % 64 != 0) return -1;
    const int64_t first = (std::min(k_split, K) + 63) / 64;
    const int64_t last = (K - (int64_t)(splits - 1) * k_split + 63) / 64;
    const int r = (int)(first % 6);
    return (r == 2 || r == 4) && last % 6 == r && std::min(first, last) > 6 ? r : -1;
}

W4Kernel w4_entry(int variant, int bn, int head, bool a_oc, bool b_oc, bool out_f32) {
    if (variant == 2)
        return bn == 192 ? w4_ring_kernel<192, 3>(head, a_oc, b_oc, out_f32)
                         : w4_ring_kernel<256, 3>(head, a_oc, b_oc, out_f32);
    if (variant == 3)
        return bn == 192 ? w4_ring_kernel<192, 2>(head, a_oc, b_oc, out_f32)
                         : w4_ring_kernel<256, 2>(head, a_oc, b_oc, out_f32);
    const int row = variant == 0 ? 0 : bn == 192 ? 2 : 1;
    return kW4[row][(out_f32 ? 4 : 0) + (a_oc ? 2 : 0) + (b_oc ? 1 : 0)];
}

}  // namespace

const char* w4_kernel_name(int variant, int bn, bool a_oc, bool b_oc, bool out_f32, int64_t K, int64_t k_split,
                           int splits) {
    return w4_entry(variant, bn, variant >= 2 ? ring_head(K, k_split, splits) : -1, a_oc, b_oc, out_f32).name;
}

hipError_t launch_gemm_w4(int variant, int bn, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                          hipStream_t stream) {
    if (variant < 0 || variant > 3) return hipErrorInvalidValue;
    if (bn != 256 && (variant == 0 || bn != 192)) return hipErrorInvalidValue;
    const int64_t blocks = ((args.M + 255) / 256) * ((args.N + bn - 1) / bn) * (int64_t)args.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    // a ring's partial last stage must follow a whole one
    if (variant >= 2 && args.K % 64 != 0 && args.K - (int64_t)(args.splits - 1) * args.k_split < 64)
        return hipErrorInvalidValue;
    const int head = variant >= 2 ? ring_head(args.K, args.k_split, args.splits) : -1;
    hipLaunchKernelGGL(w4_entry(variant, bn, head, a_oc, b_oc, out_f32).fn, dim3((unsigned)blocks),
                       dim3(kW4Threads), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_gemm_w4_stamped(int variant, bool a_oc, bool b_oc, const GemmArgs& args, hipStream_t stream) {
    if (args.splits != 1 || args.stamps == nullptr || (variant != 2 && variant != 3)) return hipErrorInvalidValue;
    const int64_t blocks = ((args.M + 255) / 256) * ((args.N + 255) / 256);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (args.K % 64 != 0 && args.K < 64) return hipErrorInvalidValue;
    const int head = ring_head(args.K, args.k_split, 1);
    const W4Kernel k = variant == 2 ? w4_ring_stamp_kernel<3>(head, a_oc, b_oc)
                                    : w4_ring_stamp_kernel<2>(head, a_oc, b_oc);
    hipLaunchKernelGGL(k.fn, dim3((unsigned)blocks), dim3(kW4Threads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace fcs
