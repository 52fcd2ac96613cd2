// Pipelined bf16 GEMM for gfx950 (MI355X): the main kernels of the three
// local products of one GPU's FC-layer shard under the 3D parallel matrix
// multiply (sciencestack.ai/paper/2502.08145, Figure 1), bf16 in with fp32
// accumulation (mlsanity.com/paper/2502.08145, Abstract: bf16 training).
//
// Requirements (checked by the caller): M, N, K multiples of 8, 16-byte
// aligned operands and output, every operand smaller than 2 GiB.
//
// Structure (256 threads = 4 wave64s in a 2 x 2 grid, block tile BM x BN):
//  * Reduction stages of 32 values; a ring of 4 LDS stages. Global data goes
//    straight into LDS with buffer_load ... lds (16 bytes per lane), no
//    register staging. Stage t + 4 is requested as soon as every wave has
//    finished reading stage t, i.e. three stages of MFMA work ahead.
//  * Out-of-range chunks (tile tails in M, N and the reduction) are given an
//    offset past the buffer's size, so the hardware fills them with zeros.
//  * Reduction-contiguous operands: LDS row = one tile row, 32 values (64 B),
//    16-byte chunk index XOR-swizzled with (row >> 2) & 3; MFMA operands are
//    single ds_read_b128.
//  * Output-contiguous operands are stored untransposed (LDS row = one
//    reduction index, chunk index XOR-swizzled by oc_swizzle(k)) and read
//    with ds_read_b64_tr_b16: within each 16-lane group, lane j addresses
//    reduction row k0 + j / 4 at columns base + 4 (j % 4), and lane i
//    receives the four reduction values k0 .. k0+3 of column base + i. Two
//    such reads give one 8-value MFMA operand.
//  * Per stage, each wave runs two 16-deep steps of v_mfma_f32_32x32x16_bf16
//    over its (BM/2) x (BN/2) sub-tile. The operands of the first step of the
//    next stage are read right after the stage barrier, which itself sits
//    between the two MFMA steps of the current stage, so MFMA issue
//    continues across the barrier.
//  * MFMAs take the B fragment as source A, so each lane's accumulators hold
//    4 consecutive output columns of one output row (vector stores).
//  * Blocks are remapped so that each XCD works through one contiguous range
//    of tiles, in groups of 8 tile-rows (L2 sharing within an XCD).
//  * Reduction slices (split-K) write fp32 partials to separate planes.
#include "gemm_common.h"

namespace fcs {

namespace {

template <int BM, int BN, bool A_OC, bool B_OC, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void gemm_pipe_kernel(GemmArgs g) {
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int kABytes = BM * kBK * 2, kBBytes = BN * kBK * 2;
    constexpr int kStageBytes = kABytes + kBBytes;
    constexpr int L = (BM + BN) / 64;  // load instructions per wave per stage
    __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave >> 1) * WTM;
    const int wn0 = (wave & 1) * WTN;

    const BlockTile bt = map_block<BM, BN>(g);
    const int slice = bt.slice;
    const int64_t m0 = bt.m0, n0 = bt.n0;

    const int64_t kbeg = (int64_t)slice * g.k_split;
    const int64_t kend = (kbeg + g.k_split < g.K) ? kbeg + g.k_split : g.K;
    const int nkt = kend > kbeg ? (int)((kend - kbeg + kBK - 1) / kBK) : 0;

    const int64_t a_rows = A_OC ? g.K : g.M;  // storage rows of each operand
    const int64_t b_rows = B_OC ? g.K : g.N;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, (int)(a_rows * g.lda * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)g.B, 0, (int)(b_rows * g.ldb * 2), kRsrcWord3);

    Dma<BM, A_OC> da;
    Dma<BN, B_OC> db;
    da.init(wave, lane, g.lda, m0, g.M);
    db.init(wave, lane, g.ldb, n0, g.N);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nkt > 0) {
        // Prologue: fill the whole ring. Stages past the end of the reduction
        // get out-of-range offsets everywhere (zeros into a free slot), so every
        // iteration below issues and waits for the same number of loads.
#pragma unroll
        for (int s = 0; s < kStages; ++s) {
            char* st = smem + s * kStageBytes;
            da.template issue<0, Dma<BM, A_OC>::kInstr>(ra, st, kbeg + s * kBK, kend, g.lda, wave);
            db.template issue<0, Dma<BN, B_OC>::kInstr>(rb, st + kABytes, kbeg + s * kBK, kend, g.ldb, wave);
        }
        waitcnt<(kStages - 1) * L, 0>();
        __builtin_amdgcn_s_barrier();

        bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa0[i] = fragment<BM, A_OC>(smem, wm0 + i * 32, 0, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb0[j] = fragment<BN, B_OC>(smem + kABytes, wn0 + j * 32, 0, lane);

        constexpr int LA = Dma<BM, A_OC>::kInstr;
        for (int t = 0; t < nkt; ++t) {
            const char* st = smem + (t % kStages) * kStageBytes;
#pragma unroll
            for (int i = 0; i < TM; ++i) fa1[i] = fragment<BM, A_OC>(st, wm0 + i * 32, 1, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb1[j] = fragment<BN, B_OC>(st + kABytes, wn0 + j * 32, 1, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // stage t is fully read by this wave; stage t + 1 must have landed
            waitcnt<(kStages - 2) * L, 0>();
            __builtin_amdgcn_s_barrier();
            const char* nx = smem + ((t + 1) % kStages) * kStageBytes;
#pragma unroll
            for (int i = 0; i < TM; ++i) fa0[i] = fragment<BM, A_OC>(nx, wm0 + i * 32, 0, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb0[j] = fragment<BN, B_OC>(nx + kABytes, wn0 + j * 32, 0, lane);
            __builtin_amdgcn_sched_barrier(0);
            // second MFMA step of stage t; the loads of stage t + 4 (into the slot
            // of stage t, free since the barrier) are spread between its rows
            char* slot = smem + (t % kStages) * kStageBytes;
            const int64_t k0 = kbeg + (int64_t)(t + kStages) * kBK;
#define FCP_STEP1_ROW(I)                                                                   \
    if constexpr ((I) < TM) {                                                              \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) acc[I][j] =                         \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1[I], acc[I][j], 0, 0, 0);   \
        __builtin_amdgcn_sched_barrier(0);                                                 \
        constexpr int lo = ((I) * L + TM - 1) / TM, hi = (((I) + 1) * L + TM - 1) / TM;   \
        da.template issue<lo, hi>(ra, slot, k0, kend, g.lda, wave);                        \
        db.template issue<lo - LA, hi - LA>(rb, slot + kABytes, k0, kend, g.ldb, wave);    \
        __builtin_amdgcn_sched_barrier(0);                                                 \
    }
            FCP_STEP1_ROW(0)
            FCP_STEP1_ROW(1)
            FCP_STEP1_ROW(2)
            FCP_STEP1_ROW(3)
#undef FCP_STEP1_ROW
        }
        waitcnt<0, 0>();  // drain the trailing (out-of-range) loads
    }

    // ---- epilogue: lane holds C[m][n .. n+3] per 32x32 block and group
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm0 + i * 32 + lr;
        if (m >= g.M) continue;
        float* crow = static_cast<float*>(g.C) + (int64_t)slice * g.c_split_stride + m * g.N;
        // an accumulating output: this row block's old values are loaded
        // first, so their latencies overlap
        [[maybe_unused]] f32x4 old[TN][4];
        if (OUT_F32 && g.accumulate) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    const int64_t n = n0 + wn0 + j * 32 + grp * 8 + lk * 4;
                    old[j][grp] = n < g.N ? *reinterpret_cast<const f32x4*>(crow + n) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int64_t n = n0 + wn0 + j * 32 + grp * 8 + lk * 4;
                if (n >= g.N) continue;
                const float v0 = acc[i][j][grp * 4 + 0], v1 = acc[i][j][grp * 4 + 1];
                const float v2 = acc[i][j][grp * 4 + 2], v3 = acc[i][j][grp * 4 + 3];
                if (OUT_F32) {
                    f32x4 v{v0, v1, v2, v3};
                    if (g.accumulate) v += old[j][grp];
                    *reinterpret_cast<f32x4*>(crow + n) = v;
                } else {
                    __bf16* c = static_cast<__bf16*>(g.C) + m * g.N + n;
                    *reinterpret_cast<bf16x4*>(c) = bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 8-wave ping-pong variant, 256 x 256 block tile (512 threads, 2 waves/SIMD).
//
// Waves 0-3 (group 0) compute output rows 0-127 of the tile, waves 4-7
// (group 1) rows 128-255; inside a group the 4 waves form a 2 x 2 grid of
// 64 x 128 wave tiles. Time is cut into phases separated by workgroup
// barriers. In each phase one group reads its operand fragments of a stage
// from LDS (and issues its half of the loads of a later stage) while the
// other group runs the MFMAs of the stage it read in the previous phase:
//
//   phase     0     1     2     3    ...   2t     2t+1
//   group 0   M(0)  C(0)  M(1)  C(1) ...   M(t)   C(t)
//   group 1   -     M(0)  C(0)  M(1) ...   C(t-1) M(t)
//
// so each SIMD always holds one wave with MFMA work. A stage holds 32
// reduction values; the ring has S = 4 slots (128 KB). Group 0 loads the A
// operand of every stage and group 1 the B operand; M(t) requests stage
// t + S - 1 into the slot of stage t - 1, which both groups finished reading
// before the barrier that opens the phase.
// Every wave issues the same number of loads in every M phase (out-of-range
// offsets past the end of the reduction), so "at most S - 2 stages of loads
// in flight" before every barrier is exactly "the stage the next M phase
// reads has landed".


template <bool A_OC, bool B_OC, bool OUT_F32, int MF>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256;
    constexpr int TM = 64 / MF, TN = 128 / MF;  // 64 x 128 wave tile
    constexpr int BKP = 32;                     // reduction values per stage
    constexpr int KSM = MF == 32 ? 2 : 1;       // MFMA reduction steps per stage
    constexpr int S = 4;
    constexpr int kABytes = BM * BKP * 2, kBBytes = BN * BKP * 2;
    constexpr int kStageBytes = kABytes + kBBytes;
    constexpr int kLoads = DmaPP<A_OC, BKP>::kInstr;  // per wave per M phase (same for B)
    static_assert(DmaPP<A_OC, BKP>::kInstr == DmaPP<B_OC, BKP>::kInstr, "balanced loaders");
    constexpr int kInFlight = (S - 2) * kLoads;
    __shared__ __attribute__((aligned(1024))) char smem[S * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int q = wave & 3;
    const int wm0 = grp * 128 + (q >> 1) * 64;
    const int wn0 = (q & 1) * 128;

    const BlockTile bt = map_block<BM, BN>(g);
    const int slice = bt.slice;
    const int64_t m0 = bt.m0, n0 = bt.n0;

    const int64_t kbeg = (int64_t)slice * g.k_split;
    const int64_t kend = (kbeg + g.k_split < g.K) ? kbeg + g.k_split : g.K;
    const int nkt = kend > kbeg ? (int)((kend - kbeg + BKP - 1) / BKP) : 0;

    const bool loadA = grp == 0;
    const int64_t rows_st = loadA ? (A_OC ? g.K : g.M) : (B_OC ? g.K : g.N);
    const int64_t ld = loadA ? g.lda : g.ldb;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(loadA ? g.A : g.B), 0, (int)(rows_st * ld * 2), kRsrcWord3);
    DmaPP<A_OC, BKP> da;
    DmaPP<B_OC, BKP> db;
    if (loadA)
        da.init(q, lane, g.lda, m0, g.M);
    else
        db.init(q, lane, g.ldb, n0, g.N);

    typename AccT<MF>::type acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<MF>::n; ++e) acc[i][j][e] = 0.0f;

    // stage s into its ring slot; A half from group 0, B half from group 1
    auto issue_stage = [&](int s) {
        char* st = smem + (s % S) * kStageBytes;
        const int64_t k0 = kbeg + (int64_t)s * BKP;
        if (loadA)
            da.issue(rs, st, k0, kend, g.lda, q);
        else
            db.issue(rs, st + kABytes, k0, kend, g.ldb, q);
    };

    if (nkt > 0) {
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue_stage(s);
        waitcnt<kInFlight, 0>();
        __builtin_amdgcn_s_barrier();
        if (grp == 1) {  // group 1 starts one phase later
            waitcnt<kInFlight, 0>();
            __builtin_amdgcn_s_barrier();
        }
        bf16x8 fa[KSM][TM], fb[KSM][TN];
        for (int t = 0; t < nkt; ++t) {
            // ---- M(t): fragments of stage t, loads of stage t + S - 1
            const char* st = smem + (t % S) * kStageBytes;
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[ks][i] = fragment_mf<A_OC, BKP, MF>(st, wm0 + i * MF, ks, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    fb[ks][j] = fragment_mf<B_OC, BKP, MF>(st + kABytes, wn0 + j * MF, ks, lane);
            }
            issue_stage(t + S - 1);
            waitcnt<kInFlight, 0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // ---- C(t)
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16<MF>(fb[ks][j], fa[ks][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
            waitcnt<kInFlight, 0>();
            __builtin_amdgcn_s_barrier();
        }
        if (grp == 0) {  // matching trailing phase
            waitcnt<kInFlight, 0>();
            __builtin_amdgcn_s_barrier();
        }
        waitcnt<0, 0>();  // drain the trailing (out-of-range) loads
    }

    store_tile<MF, TM, TN, OUT_F32>(g, slice, m0, n0, wm0, wn0, lane, acc);
}

// ---------------------------------------------------------------------------
// 8-wave ping-pong with one barrier per stage (ping-pong-1b), 256 x 256.
//
// Same tiles, ring (4 slots of 32-value stages) and load split as
// gemm_pp_kernel, but the interval between two barriers holds one stage of
// both groups with their phases in opposite order:
//
//   interval t:   group 0: M(t) then C(t)      group 1: C(t - 1) then M(t)
//
// On each SIMD the group-1 wave computes while the group-0 wave reads, then
// the group-0 wave computes (as soon as its own fragments are in registers:
// no barrier needed) while the group-1 wave reads. A barrier is only needed
// where data crosses waves: stage t + 1 must have landed (every wave waits
// for its own loads first) and stage t - 1 must be free before M(t) refills
// its slot. That halves the barriers per MFMA compared with gemm_pp_kernel.
template <bool A_OC, bool B_OC, bool OUT_F32, int MF>
__global__ __launch_bounds__(512) void gemm_pp1b_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256;
    constexpr int TM = 64 / MF, TN = 128 / MF;
    constexpr int BKP = 32, S = 4;
    constexpr int KS = MF == 32 ? 2 : 1;  // MFMA reduction steps per stage
    constexpr int kABytes = BM * BKP * 2, kBBytes = BN * BKP * 2;
    constexpr int kStageBytes = kABytes + kBBytes;
    constexpr int kLoads = DmaPP<A_OC, BKP>::kInstr;
    constexpr int kInFlight = (S - 2) * kLoads;
    __shared__ __attribute__((aligned(1024))) char smem[S * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int q = wave & 3;
    const int wm0 = grp * 128 + (q >> 1) * 64;
    const int wn0 = (q & 1) * 128;

    const BlockTile bt = map_block<BM, BN>(g);
    const int slice = bt.slice;
    const int64_t m0 = bt.m0, n0 = bt.n0;

    const int64_t kbeg = (int64_t)slice * g.k_split;
    const int64_t kend = (kbeg + g.k_split < g.K) ? kbeg + g.k_split : g.K;
    const int nkt = kend > kbeg ? (int)((kend - kbeg + BKP - 1) / BKP) : 0;

    const bool loadA = grp == 0;
    const int64_t rows_st = loadA ? (A_OC ? g.K : g.M) : (B_OC ? g.K : g.N);
    const int64_t ld = loadA ? g.lda : g.ldb;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(loadA ? g.A : g.B), 0, (int)(rows_st * ld * 2), kRsrcWord3);
    DmaPP<A_OC, BKP> da;
    DmaPP<B_OC, BKP> db;
    if (loadA)
        da.init(q, lane, g.lda, m0, g.M);
    else
        db.init(q, lane, g.ldb, n0, g.N);

    typename AccT<MF>::type acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < AccT<MF>::n; ++e) acc[i][j][e] = 0.0f;

#define FCP1B_ISSUE(SIDX)                                                                      \
    {                                                                                          \
        char* st_ = smem + ((SIDX) % S) * kStageBytes;                                         \
        const int64_t k0_ = kbeg + (int64_t)(SIDX) * BKP;                                      \
        if (loadA)                                                                             \
            da.issue(rs, st_, k0_, kend, g.lda, q);                                            \
        else                                                                                   \
            db.issue(rs, st_ + kABytes, k0_, kend, g.ldb, q);                                  \
    }
#define FCP1B_M(T)                                                                                       \
    {                                                                                                    \
        const char* st_ = smem + ((T) % S) * kStageBytes;                                                \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                              \
            _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[ks][i] =                                   \
                fragment_mf<A_OC, BKP, MF>(st_, wm0 + i * MF, ks, lane);                                 \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[ks][j] =                                   \
                fragment_mf<B_OC, BKP, MF>(st_ + kABytes, wn0 + j * MF, ks, lane);                       \
        }                                                                                                \
        FCP1B_ISSUE((T) + S - 1)                                                                         \
        __builtin_amdgcn_sched_barrier(0);                                                               \
    }
#define FCP1B_C()                                                                                        \
    {                                                                                                    \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) _Pragma("unroll") for (int i = 0; i < TM; ++i) \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) acc[i][j] =                                   \
                mfma_bf16<MF>(fb[ks][j], fa[ks][i], acc[i][j]);                                          \
        __builtin_amdgcn_sched_barrier(0);                                                               \
    }
#define FCP1B_SYNC()                 \
    {                                \
        waitcnt<kInFlight, 0>();     \
        __builtin_amdgcn_s_barrier(); \
        __builtin_amdgcn_sched_barrier(0); \
    }

    if (nkt > 0) {
        FCP1B_ISSUE(0)
        FCP1B_ISSUE(1)
        FCP1B_ISSUE(2)
        FCP1B_SYNC()
        bf16x8 fa[KS][TM], fb[KS][TN];
        if (loadA) {
            for (int t = 0; t < nkt; ++t) {
                FCP1B_M(t)
                FCP1B_C()
                FCP1B_SYNC()
            }
            FCP1B_SYNC()  // the interval in which group 1 finishes its last stage
        } else {
            FCP1B_M(0)
            FCP1B_SYNC()
            for (int t = 1; t < nkt; ++t) {
                FCP1B_C()
                FCP1B_M(t)
                FCP1B_SYNC()
            }
            FCP1B_C()
            FCP1B_SYNC()
        }
        waitcnt<0, 0>();
    }
#undef FCP1B_ISSUE
#undef FCP1B_M
#undef FCP1B_C
#undef FCP1B_SYNC

    store_tile<MF, TM, TN, OUT_F32>(g, slice, m0, n0, wm0, wn0, lane, acc);
}

using KernelFn = void (*)(GemmArgs);
struct Entry {
    KernelFn fn;
    const char* name;
};

#define FCP_K(BM, BN, AOC, BOC, F32) \
    Entry { gemm_pipe_kernel<BM, BN, AOC, BOC, F32>, "gemm_pipe_kernel<" #BM ", " #BN ", " #AOC ", " #BOC ", " #F32 ">" }
#define FCP_LAYOUTS(BM, BN, F32)                                                                 \
    FCP_K(BM, BN, false, false, F32), FCP_K(BM, BN, false, true, F32), FCP_K(BM, BN, true, false, F32), \
        FCP_K(BM, BN, true, true, F32)
#define FCP_TILE(BM, BN) FCP_LAYOUTS(BM, BN, false), FCP_LAYOUTS(BM, BN, true)

// [tile][out_f32][a_oc][b_oc], tiles in the order of kTiles
const Entry kPipe[kNumTiles * 8] = {
    FCP_TILE(256, 256),
    FCP_TILE(256, 128),
    FCP_TILE(128, 256),
    FCP_TILE(128, 128),
};

#define FCPP_K(AOC, BOC, F32, MF) \
    Entry { gemm_pp_kernel<AOC, BOC, F32, MF>, "gemm_pp_kernel<" #AOC ", " #BOC ", " #F32 ", " #MF ">" }
#define FCPP_ALL(MF)                                                                                    \
    FCPP_K(false, false, false, MF), FCPP_K(false, true, false, MF), FCPP_K(true, false, false, MF),    \
        FCPP_K(true, true, false, MF), FCPP_K(false, false, true, MF), FCPP_K(false, true, true, MF),   \
        FCPP_K(true, false, true, MF), FCPP_K(true, true, true, MF)
// [MFMA: 32x32x16, 16x16x32][out_f32][a_oc][b_oc]
const Entry kPingPong[2][8] = {{FCPP_ALL(32)}, {FCPP_ALL(16)}};

#define FCPP1B_K(AOC, BOC, F32, MF) \
    Entry { gemm_pp1b_kernel<AOC, BOC, F32, MF>, "gemm_pp1b_kernel<" #AOC ", " #BOC ", " #F32 ", " #MF ">" }
#define FCPP1B_ALL(MF)                                                                                  \
    FCPP1B_K(false, false, false, MF), FCPP1B_K(false, true, false, MF), FCPP1B_K(true, false, false, MF), \
        FCPP1B_K(true, true, false, MF), FCPP1B_K(false, false, true, MF), FCPP1B_K(false, true, true, MF), \
        FCPP1B_K(true, false, true, MF), FCPP1B_K(true, true, true, MF)
const Entry kPingPong1b[2][8] = {{FCPP1B_ALL(32)}, {FCPP1B_ALL(16)}};

const Entry& pipe_entry(int tile, bool a_oc, bool b_oc, bool out_f32) {
    return kPipe[tile * 8 + (out_f32 ? 4 : 0) + (a_oc ? 2 : 0) + (b_oc ? 1 : 0)];
}

}  // namespace

const char* pipe_kernel_name(int tile, bool a_oc, bool b_oc, bool out_f32) {
    return pipe_entry(tile, a_oc, b_oc, out_f32).name;
}

const Entry& pingpong_entry(int variant, bool a_oc, bool b_oc, bool out_f32) {
    const int i = (out_f32 ? 4 : 0) + (a_oc ? 2 : 0) + (b_oc ? 1 : 0);
    // variant bit 0: one barrier per stage; bit 1: 16x16x32 MFMAs
    const int mf = (variant >> 1) & 1;
    return (variant & 1) ? kPingPong1b[mf][i] : kPingPong[mf][i];
}

const char* pingpong_kernel_name(int variant, bool a_oc, bool b_oc, bool out_f32) {
    return pingpong_entry(variant, a_oc, b_oc, out_f32).name;
}

hipError_t launch_gemm_pingpong(int variant, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                                hipStream_t stream) {
    const int64_t blocks = ((args.M + 255) / 256) * ((args.N + 255) / 256) * (int64_t)args.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pingpong_entry(variant, a_oc, b_oc, out_f32).fn, dim3((unsigned)blocks),
                       dim3(512), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_gemm_pipe(int tile, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                            hipStream_t stream) {
    const TileCfg& t = kTiles[tile];
    const int64_t blocks = ((args.M + t.bm - 1) / t.bm) * ((args.N + t.bn - 1) / t.bn) * (int64_t)args.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pipe_entry(tile, a_oc, b_oc, out_f32).fn, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       args);
    return hipGetLastError();
}

}  // namespace fcs
