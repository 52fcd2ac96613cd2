// 4-wave bf16 GEMMs for gfx950 (MI355X), one wave per SIMD: the local
// products of one GPU's FC-layer shard under the 3D parallel matrix multiply
// (sciencestack.ai/paper/2502.08145, Figure 1), bf16 in with fp32
// accumulation (mlsanity.com/paper/2502.08145, Abstract: bf16 training).
//
// Requirements (checked by the caller): M, N multiples of 8, K and the
// split-K slice length multiples of 64 (128 for the 64-value-stage kernel),
// 16-byte aligned operands and output, every operand smaller than 2 GiB.
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
#include <algorithm>

#include "gemm_common.h"

namespace fcs {

namespace {

constexpr int kW4Threads = 256;

// block set-up shared by both kernels
struct W4Setup {
    int lane, wave, wm0, wn0, slice, nkt;
    int64_t m0, n0, kbeg, kend;
    __amdgpu_buffer_rsrc_t ra, rb;
};

template <bool A_OC, bool B_OC, int BKP, int BN = 256>
__device__ __forceinline__ W4Setup w4_setup(const GemmArgs& g) {
    W4Setup w;
    const int tid = threadIdx.x;
    w.lane = tid & 63;
    w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    w.wm0 = (w.wave >> 1) * 128;
    w.wn0 = (w.wave & 1) * (BN / 2);
    const BlockTile bt = map_block<256, BN>(g);
    w.slice = bt.slice;
    w.m0 = bt.m0;
    w.n0 = bt.n0;
    w.kbeg = (int64_t)w.slice * g.k_split;
    w.kend = (w.kbeg + g.k_split < g.K) ? w.kbeg + g.k_split : g.K;
    w.nkt = w.kend > w.kbeg ? (int)((w.kend - w.kbeg + BKP - 1) / BKP) : 0;
    const int64_t a_rows = A_OC ? g.K : g.M;  // storage rows of each operand
    const int64_t b_rows = B_OC ? g.K : g.N;
    w.ra = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, (int)(a_rows * g.lda * 2), kRsrcWord3);
    w.rb = __builtin_amdgcn_make_buffer_rsrc((void*)g.B, 0, (int)(b_rows * g.ldb * 2), kRsrcWord3);
    return w;
}

// scheduling groups of one 64-MFMA step: one LDS read after each of the
// first READS MFMAs, then LOADS loads spread evenly over the rest
template <int READS, int LOADS>
__device__ __forceinline__ void w4_interleave() {
    constexpr int kGap = LOADS > 0 ? (64 - READS) / LOADS : 1;
    static_assert(LOADS == 0 || kGap >= 1, "too many loads for one step");
#pragma unroll
    for (int u = 0; u < 64; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (u < READS)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        else if ((u - READS) % kGap == 0 && (u - READS) / kGap < LOADS)
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one load
    }
}

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

// Placement of the 8 + TN fragment reads and NL loads (NL <= 8 + TN) of one
// 8 TN-MFMA step: the index of the read or load issued right after MFMA u, or
// -1. The step's MFMAs form 16 groups of TN / 2. With loads, one load after
// the first MFMA of a group and the reads after the next one or two MFMAs of
// the first groups; without loads, the reads after MFMAs 0 .. 7 + TN. (For
// TN = 8, measured and slower or equal: the reads first and the loads spread
// over the rest; the loads first, one after every second MFMA; a load after
// every third MFMA; a loadless step's reads after every second MFMA.)
template <int TN>
__device__ constexpr int w64_read_after(int nl, int u) {
    constexpr int gs = TN / 2, rpg = gs > 2 ? 2 : gs - 1, nr = 8 + TN;
    if (nl == 0) return u < nr ? u : -1;
    const int r = rpg * (u / gs) + (u % gs) - 1;
    return (u % gs != 0 && u % gs <= rpg && r < nr) ? r : -1;
}
template <int TN>
__device__ constexpr int w64_load_after(int nl, int u) {
    constexpr int gs = TN / 2;
    return (nl > 0 && u % gs == 0 && u / gs < nl) ? u / gs : -1;
}

// Orders every compiler write of the accumulators (their zero
// initialisation, copies where control paths merge) before the asm MFMAs
// that read them: every accumulator passes through an empty asm (so such
// writes must come before it), then a few wait states pass before the next
// MFMA.
template <int TN>
__device__ __forceinline__ void w4_acc_fence(f32x4 (&acc)[8][TN]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]));
    asm volatile("s_nop 4" ::: "memory");
}

// The last MFMAs must have written their results before anything else
// reads the accumulators: wait states, then every accumulator through an
// empty asm (reads of them come after it).
template <int TN>
__device__ __forceinline__ void w4_acc_drain(f32x4 (&acc)[8][TN]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// One v_mfma_f32_16x16x32_bf16 (B fragment as source A) whose accumulator is
// pinned to AGPRs, and whose position relative to the loads, LDS reads and
// barriers is its place in the source. The compiler's register allocator
// otherwise moves 256 accumulators between AGPRs and VGPRs when a step issues
// many loads. Hazards the compiler no longer sees are covered by the kernel:
// an accumulator is read again only by the same MFMA 32 or more MFMAs later, sources
// come from LDS reads the compiler waits for, and s_nops follow the zero
// initialisation and precede the epilogue.
__device__ __forceinline__ void mfma_agpr(f32x4& acc, const bf16x8& b, const bf16x8& a) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
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

    f32x4 acc[8][TN];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
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
// gemm_w4k64r_kernel: the 64-value stages of gemm_w4k64_kernel in the whole
// 160 KB LDS, as a ring of three A tiles and two B tiles (32 KB each, one
// array each). Step 1 of stage t opens with the barrier that certifies stage
// t + 1 and frees stage t's tiles; it then loads the B tile of stage t + 2
// (into stage t's B tile) and the A tile of stage t + 3 (into stage t's A
// tile), so A loads have three steps to land and B loads at least one and a
// half. The loop body holds one period of six stages with every tile fixed
// (stage t in A tile t mod 3 and B tile t mod 2), and the control flow stays
// that one loop. A stage count that is not a multiple of 6 either
// (HEAD < 0) is padded at the front with virtual stages of zeros (up to five
// stages of extra MFMA work; the tuner weighs it against gemm_w4k64_kernel)
// or (HEAD = 1 .. 5, the stage count mod 6, the same for every block) starts
// with HEAD straight-line stages that take the last HEAD positions of a
// period: the padded schedule without its virtual stages, no extra work, and
// still one control path.
template <bool A_OC, bool B_OC, bool OUT_F32, int BN, int HEAD>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4k64r_kernel(
    GemmArgs g) {
    constexpr int MF = 16, BKP = 64;
    constexpr int TN = BN / 32;        // 16-column blocks per wave
    constexpr int kT = 256 * BKP * 2;  // 32 KB per tile array (also one wave's epilogue staging)
    constexpr int kLA = DmaPP<A_OC, BKP>::kInstr;
    constexpr int kLB = DmaPP<B_OC, BKP, BN>::kInstr;
    __shared__ __attribute__((aligned(1024))) char ta0[kT];
    __shared__ __attribute__((aligned(1024))) char ta1[kT];
    __shared__ __attribute__((aligned(1024))) char ta2[kT];
    __shared__ __attribute__((aligned(1024))) char tb0[kT];
    __shared__ __attribute__((aligned(1024))) char tb1[kT];

    const W4Setup w = w4_setup<A_OC, B_OC, BKP, BN>(g);
    const int lane = w.lane, wave = w.wave, wm0 = w.wm0, wn0 = w.wn0, nkt = w.nkt;
    DmaPP<A_OC, BKP> da;
    DmaPP<B_OC, BKP, BN> db;
    da.init(wave, lane, g.lda, w.m0, g.M);
    db.init(wave, lane, g.ldb, w.n0, g.N);

    f32x4 acc[8][TN];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 fa[2][8], fb[2][TN];

#define FCR_TA(I) ((I) == 0 ? ta0 : (I) == 1 ? ta1 : ta2)
#define FCR_TB(I) ((I) == 0 ? tb0 : tb1)
#define FCR_OFF(SIDX) (w.kbeg + (int64_t)((SIDX) < 0 ? 0 : (SIDX) < nkt ? (SIDX) : nkt - 1) * BKP)
#define FCR_STEP_A(SIDX) (uint32_t)(A_OC ? FCR_OFF(SIDX) * g.lda * 2 : FCR_OFF(SIDX) * 2)
#define FCR_STEP_B(SIDX) (uint32_t)(B_OC ? FCR_OFF(SIDX) * g.ldb * 2 : FCR_OFF(SIDX) * 2)
#define FCR_RA(SIDX) ((SIDX) < 0 ? rza : w.ra)
#define FCR_RB(SIDX) ((SIDX) < 0 ? rzb : w.rb)
    // 8 TN MFMAs from set CUR; fragment reads of step KS of tiles (RA, RB) into
    // set NXT; with LOADS, the B tile of stage T + 2 into LB, then the A tile
    // of stage T + 3 into LA, placed as w64_read_after / w64_load_after say
#define FCR_STEP(CUR, NXT, RA, RB, KS, LOADS, LA, LB, T)                                              \
    {                                                                                                  \
        const uint32_t sb_ = FCR_STEP_B((T) + 2), sa_ = FCR_STEP_A((T) + 3);                           \
        const __amdgpu_buffer_rsrc_t rb_ = FCR_RB((T) + 2), ra_ = FCR_RA((T) + 3);                     \
        constexpr int nl_ = (LOADS) ? kLA + kLB : 0;                                                   \
        _Pragma("unroll") for (int u = 0; u < 8 * TN; ++u) {                                           \
            mfma_agpr(acc[u / TN][u % TN], fb[CUR][u % TN], fa[CUR][u / TN]);                          \
            const int r_ = w64_read_after<TN>(nl_, u);                                                 \
            if (r_ >= 0 && r_ < 8) {                                                                   \
                fa[NXT][r_] = fragment_mf<A_OC, BKP, MF>(RA, wm0 + r_ * MF, KS, lane);                 \
            } else if (r_ >= 8) {                                                                      \
                fb[NXT][r_ - 8] = fragment_mf<B_OC, BKP, MF, BN>(RB, wn0 + (r_ - 8) * MF, KS, lane);   \
            }                                                                                          \
            const int l_ = w64_load_after<TN>(nl_, u);                                                 \
            if (l_ >= 0 && l_ < kLB)                                                                   \
                db.issue_one(rb_, LB, sb_, wave, l_);                                                  \
            else if (l_ >= kLB)                                                                        \
                da.issue_one(ra_, LA, sa_, wave, l_ - kLB);                                            \
        }                                                                                              \
    }
    // stage T with A tile P mod 3 and B tile P mod 2 (P = T mod 6): step 0,
    // the barrier (only the A loads of the last step may still be in
    // flight), step 1 (reads step 0 of stage T + 1)
#define FCR_STAGE(P, T)                                                                                \
    {                                                                                                  \
        FCR_STEP(0, 1, FCR_TA((P) % 3), FCR_TB((P) % 2), 1, false, ta0, tb0, T)                        \
        waitcnt<kLA, 0>();                                                                             \
        __builtin_amdgcn_s_barrier();                                                                  \
        FCR_STEP(1, 0, FCR_TA(((P) + 1) % 3), FCR_TB(((P) + 1) % 2), 0, true, FCR_TA((P) % 3),         \
                 FCR_TB((P) % 2), T)                                                                   \
    }

    if (nkt > 0) {
        const __amdgpu_buffer_rsrc_t rza = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, 0, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rzb = __builtin_amdgcn_make_buffer_rsrc((void*)g.B, 0, 0, kRsrcWord3);
        if constexpr (HEAD < 0) {
            // The loop runs whole periods of six stages: pad virtual stages
            // -pad .. -1 go first and load through zero-size descriptors, so
            // their tiles hold zeros and their MFMAs add nothing.
            const int pad = (6 - nkt % 6) % 6;
            // stages -pad, -pad + 1 and the A tile of -pad + 2; wait for the first; read its step 0
            da.issue_full(FCR_RA(-pad), ta0, FCR_STEP_A(-pad), wave);
            db.issue_full(FCR_RB(-pad), tb0, FCR_STEP_B(-pad), wave);
            da.issue_full(FCR_RA(1 - pad), ta1, FCR_STEP_A(1 - pad), wave);
            db.issue_full(FCR_RB(1 - pad), tb1, FCR_STEP_B(1 - pad), wave);
            da.issue_full(FCR_RA(2 - pad), ta2, FCR_STEP_A(2 - pad), wave);
            waitcnt<2 * kLA + kLB, 0>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[0][i] = fragment_mf<A_OC, BKP, MF>(ta0, wm0 + i * MF, 0, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[0][j] = fragment_mf<B_OC, BKP, MF, BN>(tb0, wn0 + j * MF, 0, lane);
            w4_acc_fence(acc);
            for (int t = -pad; t < nkt; t += 6) {  // nkt + pad is a multiple of 6
                FCR_STAGE(0, t)
                FCR_STAGE(1, t + 1)
                FCR_STAGE(2, t + 2)
                FCR_STAGE(3, t + 3)
                FCR_STAGE(4, t + 4)
                FCR_STAGE(5, t + 5)
            }
        } else {
            // stages 0 .. HEAD - 1 take period positions P0 .. 5; stages 0, 1
            // and the A tile of stage 2 go to those positions' tiles
            constexpr int P0 = 6 - HEAD;
            da.issue_full(w.ra, FCR_TA(P0 % 3), FCR_STEP_A(0), wave);
            db.issue_full(w.rb, FCR_TB(P0 % 2), FCR_STEP_B(0), wave);
            da.issue_full(w.ra, FCR_TA((P0 + 1) % 3), FCR_STEP_A(1), wave);
            db.issue_full(w.rb, FCR_TB((P0 + 1) % 2), FCR_STEP_B(1), wave);
            da.issue_full(w.ra, FCR_TA((P0 + 2) % 3), FCR_STEP_A(2), wave);
            waitcnt<2 * kLA + kLB, 0>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int i = 0; i < 8; ++i)
                fa[0][i] = fragment_mf<A_OC, BKP, MF>(FCR_TA(P0 % 3), wm0 + i * MF, 0, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[0][j] = fragment_mf<B_OC, BKP, MF, BN>(FCR_TB(P0 % 2), wn0 + j * MF, 0, lane);
            w4_acc_fence(acc);
            if constexpr (HEAD >= 5) FCR_STAGE(1, HEAD - 5)
            if constexpr (HEAD >= 4) FCR_STAGE(2, HEAD - 4)
            if constexpr (HEAD >= 3) FCR_STAGE(3, HEAD - 3)
            if constexpr (HEAD >= 2) FCR_STAGE(4, HEAD - 2)
            if constexpr (HEAD >= 1) FCR_STAGE(5, HEAD - 1)
            // nkt - HEAD is a positive multiple of 6 (the launcher picks this
            // form only then). A do-while: with a path around the loop the
            // compiler merges two sets of accumulators at its exit and may copy
            // the last MFMA's result before that MFMA has written it.
            int t = HEAD;
            do {
                FCR_STAGE(0, t)
                FCR_STAGE(1, t + 1)
                FCR_STAGE(2, t + 2)
                FCR_STAGE(3, t + 3)
                FCR_STAGE(4, t + 4)
                FCR_STAGE(5, t + 5)
                t += 6;
            } while (t < nkt);
        }
        waitcnt<0, 0>();  // drain the trailing prefetches
    }
#undef FCR_TA
#undef FCR_TB
#undef FCR_OFF
#undef FCR_STEP_A
#undef FCR_STEP_B
#undef FCR_RA
#undef FCR_RB
#undef FCR_STEP
#undef FCR_STAGE
    w4_acc_drain(acc);  // the last MFMAs must have written their results before the epilogue reads them

    // the tiles become staging space: every wave's loads must have landed
    // and its LDS reads finished before any wave writes there
    waitcnt<0, 0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (OUT_F32)
        store_tile_f32_staged(g, w.slice, w.m0, w.n0, wm0, wn0, lane, acc, wave == 0 ? ta0 : wave == 1 ? ta1 : wave == 2 ? ta2 : tb0);
    else
        store_tile_bf16_staged(g, w.m0, w.n0, wm0, wn0, lane, acc, wave == 0 ? ta0 : wave == 1 ? ta1 : wave == 2 ? ta2 : tb0);
}
#undef FCW4_MFMA_STEP

// Explicit instantiations: the host pass must emit a launch stub for every
// instance the table below names. (The ring kernel's head forms with both
// operands output-contiguous at 256 columns are not built: they spill.)
#define FCW4_HINST(AOC, BOC, F32, BN)                                          \
    template __global__ void gemm_w4k64r_kernel<AOC, BOC, F32, BN, 2>(GemmArgs); \
    template __global__ void gemm_w4k64r_kernel<AOC, BOC, F32, BN, 4>(GemmArgs);
#define FCW4_HINST_256_false_false(F32) FCW4_HINST(false, false, F32, 256)
#define FCW4_HINST_256_false_true(F32) FCW4_HINST(false, true, F32, 256)
#define FCW4_HINST_256_true_false(F32) FCW4_HINST(true, false, F32, 256)
#define FCW4_HINST_256_true_true(F32)
#define FCW4_INST(AOC, BOC, F32)                                               \
    template __global__ void gemm_w4_kernel<AOC, BOC, F32>(GemmArgs);          \
    template __global__ void gemm_w4k64_kernel<AOC, BOC, F32, 256>(GemmArgs);  \
    template __global__ void gemm_w4k64_kernel<AOC, BOC, F32, 192>(GemmArgs);  \
    template __global__ void gemm_w4k64r_kernel<AOC, BOC, F32, 256, -1>(GemmArgs);  \
    template __global__ void gemm_w4k64r_kernel<AOC, BOC, F32, 192, -1>(GemmArgs);  \
    FCW4_HINST(AOC, BOC, F32, 192)                                                   \
    FCW4_HINST_256_##AOC##_##BOC(F32)
FCW4_INST(false, false, false)
FCW4_INST(false, true, false)
FCW4_INST(true, false, false)
FCW4_INST(true, true, false)
FCW4_INST(false, false, true)
FCW4_INST(false, true, true)
FCW4_INST(true, false, true)
FCW4_INST(true, true, true)
#undef FCW4_INST
#undef FCW4_HINST
#undef FCW4_HINST_256_false_false
#undef FCW4_HINST_256_false_true
#undef FCW4_HINST_256_true_false
#undef FCW4_HINST_256_true_true

using KernelFn = void (*)(GemmArgs);
struct W4Entry {
    KernelFn fn;
    const char* name;
};

#define FCW4_K(KN, AOC, BOC, F32) \
    W4Entry { KN<AOC, BOC, F32>, #KN "<" #AOC ", " #BOC ", " #F32 ">" }
#define FCW4_2S(BN, AOC, BOC, F32) \
    W4Entry { gemm_w4k64_kernel<AOC, BOC, F32, BN>, "gemm_w4k64_kernel<" #AOC ", " #BOC ", " #F32 ", " #BN ">" }
// the ring kernel with head HEAD, or the padded one where no head form is built
template <bool AOC, bool BOC, bool F32, int BN, int HEAD>
constexpr KernelFn ring_fn() {
    if constexpr (HEAD > 0 && AOC && BOC && BN == 256)
        return gemm_w4k64r_kernel<AOC, BOC, F32, BN, -1>;
    else
        return gemm_w4k64r_kernel<AOC, BOC, F32, BN, HEAD>;
}
#define FCW4_R(BN, TL, AOC, BOC, F32)                                                                  \
    W4Entry {                                                                                          \
        ring_fn<AOC, BOC, F32, BN, TL>(),                                                              \
            (TL > 0 && AOC && BOC && BN == 256)                                                        \
                ? "gemm_w4k64r_kernel<" #AOC ", " #BOC ", " #F32 ", " #BN ", -1>"                      \
                : "gemm_w4k64r_kernel<" #AOC ", " #BOC ", " #F32 ", " #BN ", " #TL ">"                 \
    }
#define FCW4_RING_P(BN, AOC, BOC, F32) FCW4_R(BN, -1, AOC, BOC, F32)
#define FCW4_RING_H2(BN, AOC, BOC, F32) FCW4_R(BN, 2, AOC, BOC, F32)
#define FCW4_RING_H4(BN, AOC, BOC, F32) FCW4_R(BN, 4, AOC, BOC, F32)
#define FCW4_ALL(K, X)                                                                   \
    K(X, false, false, false), K(X, false, true, false), K(X, true, false, false),       \
        K(X, true, true, false), K(X, false, false, true), K(X, false, true, true),      \
        K(X, true, false, true), K(X, true, true, true)
// [kernel][out_f32][a_oc][b_oc]: the 32-value-stage kernel; the two-slot
// kernel with 256- and 192-column block tiles; the ring kernel with 256- and
// 192-column tiles, each padded at the front or starting with a head of 2 or
// 4 stages
const W4Entry kW4[9][8] = {{FCW4_ALL(FCW4_K, gemm_w4_kernel)},
                           {FCW4_ALL(FCW4_2S, 256)},
                           {FCW4_ALL(FCW4_2S, 192)},
                           {FCW4_ALL(FCW4_RING_P, 256)},
                           {FCW4_ALL(FCW4_RING_P, 192)},
                           {FCW4_ALL(FCW4_RING_H2, 256)},
                           {FCW4_ALL(FCW4_RING_H2, 192)},
                           {FCW4_ALL(FCW4_RING_H4, 256)},
                           {FCW4_ALL(FCW4_RING_H4, 192)}};

int w4_row(int variant, int bn, int head) {
    if (variant == 0) return 0;
    if (variant == 1) return bn == 192 ? 2 : 1;
    return (head == 2 ? 5 : head == 4 ? 7 : 3) + (bn == 192 ? 1 : 0);
}

// The ring kernel's head for this launch: the reduction slices' stage count
// mod 6 when it is 2 or 4 for every slice and every slice has a whole period
// after its head, else -1 (pad at the front).
// (Both operands output-contiguous at 256 columns keep the padded form: with
// a head, that kernel runs out of registers and spills in its main loop.)
int ring_head(int64_t K, int64_t k_split, int splits, int bn, bool a_oc, bool b_oc) {
    if (bn == 256 && a_oc && b_oc) return -1;
    const int64_t first = (std::min(k_split, K) + 63) / 64;
    const int64_t last = (K - (int64_t)(splits - 1) * k_split + 63) / 64;
    const int r = (int)(first % 6);
    return (r == 2 || r == 4) && last % 6 == r && std::min(first, last) > 6 ? r : -1;
}

const W4Entry& w4_entry(int variant, int bn, int head, bool a_oc, bool b_oc, bool out_f32) {
    return kW4[w4_row(variant, bn, head)][(out_f32 ? 4 : 0) + (a_oc ? 2 : 0) + (b_oc ? 1 : 0)];
}

}  // namespace

const char* w4_kernel_name(int variant, int bn, bool a_oc, bool b_oc, bool out_f32, int64_t K, int64_t k_split,
                           int splits) {
    return w4_entry(variant, bn, variant == 2 ? ring_head(K, k_split, splits, bn, a_oc, b_oc) : -1, a_oc, b_oc,
                    out_f32)
        .name;
}

hipError_t launch_gemm_w4(int variant, int bn, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                          hipStream_t stream) {
    if (bn != 256 && (variant == 0 || bn != 192)) return hipErrorInvalidValue;
    const int64_t blocks = ((args.M + 255) / 256) * ((args.N + bn - 1) / bn) * (int64_t)args.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int head = variant == 2 ? ring_head(args.K, args.k_split, args.splits, bn, a_oc, b_oc) : -1;
    hipLaunchKernelGGL(w4_entry(variant, bn, head, a_oc, b_oc, out_f32).fn, dim3((unsigned)blocks),
                       dim3(kW4Threads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace fcs
