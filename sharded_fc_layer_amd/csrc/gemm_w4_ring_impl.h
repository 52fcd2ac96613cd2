// The ring kernel (gemm_w4k64r_kernel) and its instances for one block-tile
// width, FCW4_RING_BN (256 or 192), and one split of the five LDS tiles,
// FCW4_RING_NA A tiles (3 unless set), set by the including source file; each
// such pair is its own translation unit so that the build compiles them in
// parallel. Requirements as in gemm_w4.hip (K and split slices multiples of
// 64).
#include "gemm_w4_common.h"

#ifndef FCW4_RING_BN
#error "FCW4_RING_BN must be defined (256 or 192)"
#endif
#ifndef FCW4_RING_NA
#define FCW4_RING_NA 3
#endif

namespace fcs {
namespace {

// gemm_w4k64r_kernel: the 64-value stages of gemm_w4k64_kernel in the whole
// 160 KB LDS, as a ring of three A tiles and two B tiles (32 KB each, one
// array each). Step 1 of stage t opens with the barrier that certifies stage
// t + 1 and frees stage t's tiles; it then loads the B tile of stage t + 2
// into stage t's B tile. The A tile of stage t + 2 goes into the A tile that
// stage t - 1 freed, loaded in step 0 of stage t: each step then issues half
// a stage's loads, spread over the step (w64_load_spread), B loads have about
// one and a half steps to land and A loads two and a half. The loop body
// holds one period of six stages with every tile fixed
// (stage t in A tile t mod 3 and B tile t mod 2), and the control flow stays
// that one loop. A stage count that is not a multiple of 6 either
// (HEAD < 0) is padded at the front with virtual stages of zeros (up to five
// stages of extra MFMA work; the tuner weighs it against gemm_w4k64_kernel)
// or (HEAD = the stage count mod 6, the same for every block, with at least
// one whole period after it; 2 and 4 are built) starts with HEAD
// straight-line stages that take the last HEAD positions of a period, then
// runs the periods as a do-while: the padded schedule without its virtual
// stages, no extra work, and still one control path.
//
// NA = 2 mirrors the ring: two A tiles and three B tiles (ta2 is the third B
// tile); the B tile of stage t + 2 is loaded in step 0 and the A tile in
// step 1, so the B operand gets the longer lead.
template <bool A_OC, bool B_OC, bool OUT_F32, int BN, int HEAD, int NA>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4k64r_kernel(
    GemmArgs g) {
    static_assert(NA == 3 || NA == 2, "three A and two B tiles, or two A and three B");
    constexpr int NB = 5 - NA;
    constexpr int MF = 16, BKP = 64;
    constexpr int TN = BN / 32;        // 16-column blocks per wave
    constexpr int kT = 256 * BKP * 2;  // 32 KB per tile array (also one wave's epilogue staging)
    constexpr int kLA = DmaPP<A_OC, BKP>::kInstr;
    constexpr int kLB = DmaPP<B_OC, BKP, BN>::kInstr;
    constexpr int kFar = NA == 3 ? kLA : kLB;  // loads of the operand with three tiles
    // loads spread over both steps of a stage (the schedule without it, all 16
    // loads of a stage in step 1 as w64_load_after places them, is kept for
    // comparison)
    constexpr bool kSpread = true;
    // Where registers are short (both operands output-contiguous at 256
    // columns), the A fragments of rows 0 .. kSingleA - 1 are single-buffered:
    // row i's fragment for the next step is read right after the last MFMA
    // of this step that uses it (MFMA TN i + TN - 1), into the same registers.
    // The last of those reads still has 8 - kSingleA rows of MFMAs to finish
    // before the stage's barrier, which waits for every LDS read.
    constexpr int kSingleA = (A_OC && B_OC && BN == 256) ? 6 : 0;
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

#define FCR_TA(I) (NA == 3 ? ((I) == 0 ? ta0 : (I) == 1 ? ta1 : ta2) : ((I) == 0 ? ta0 : ta1))
#define FCR_TB(I) (NA == 3 ? ((I) == 0 ? tb0 : tb1) : ((I) == 0 ? tb0 : (I) == 1 ? tb1 : ta2))
#define FCR_OFF(SIDX) (w.kbeg + (int64_t)((SIDX) < 0 ? 0 : (SIDX) < nkt ? (SIDX) : nkt - 1) * BKP)
#define FCR_STEP_A(SIDX) (uint32_t)(A_OC ? FCR_OFF(SIDX) * g.lda * 2 : FCR_OFF(SIDX) * 2)
#define FCR_STEP_B(SIDX) (uint32_t)(B_OC ? FCR_OFF(SIDX) * g.ldb * 2 : FCR_OFF(SIDX) * 2)
#define FCR_RA(SIDX) ((SIDX) < 0 ? rza : w.ra)
#define FCR_RB(SIDX) ((SIDX) < 0 ? rzb : w.rb)
    // 8 TN MFMAs from set CUR; fragment reads of step KS of tiles (RA, RB) into
    // set NXT (single-buffered A rows: after their last MFMA; the other A rows
    // and the B fragments as w64_read_after_n places them); with LOADS, the
    // loads of stage T + 2 of the operand with three tiles (FAR) or of the
    // other one (near) into tile L, placed as w64_load_spread says
#define FCR_FA(SET, I) fa[(I) < kSingleA ? 0 : (SET)][I]
#define FCR_STEP(CUR, NXT, RA, RB, KS, LOADS, FAR, L, T)                                              \
    {                                                                                                  \
        constexpr bool load_a_ = (FAR) == (NA == 3);                                                   \
        const uint32_t so_ = load_a_ ? FCR_STEP_A((T) + 2) : FCR_STEP_B((T) + 2);                      \
        const __amdgpu_buffer_rsrc_t ro_ = load_a_ ? FCR_RA((T) + 2) : FCR_RB((T) + 2);                \
        constexpr int nl_ = (LOADS) ? (load_a_ ? kLA : kLB) : 0;                                       \
        _Pragma("unroll") for (int u = 0; u < 8 * TN; ++u) {                                           \
            mfma_agpr(acc[u / TN][u % TN], fb[CUR][u % TN], FCR_FA(CUR, u / TN));                      \
            if (u % TN == TN - 1 && u / TN < kSingleA)                                                 \
                FCR_FA(NXT, u / TN) = fragment_mf<A_OC, BKP, MF>(RA, wm0 + (u / TN) * MF, KS, lane);  \
            const int r_ = w64_read_after_n<TN>(8 - kSingleA + TN, u);                                 \
            if (r_ >= 0 && r_ < 8 - kSingleA) {                                                        \
                const int i_ = r_ + kSingleA;                                                          \
                FCR_FA(NXT, i_) = fragment_mf<A_OC, BKP, MF>(RA, wm0 + i_ * MF, KS, lane);             \
            } else if (r_ >= 8 - kSingleA) {                                                           \
                const int j_ = r_ - (8 - kSingleA);                                                    \
                fb[NXT][j_] = fragment_mf<B_OC, BKP, MF, BN>(RB, wn0 + j_ * MF, KS, lane);             \
            }                                                                                          \
            const int l_ = w64_load_spread<TN>(nl_, u);                                                \
            if (l_ >= 0) {                                                                             \
                if constexpr (load_a_)                                                                 \
                    da.issue_one(ro_, L, so_, wave, l_);                                               \
                else                                                                                   \
                    db.issue_one(ro_, L, so_, wave, l_);                                               \
            }                                                                                          \
        }                                                                                              \
    }
    // The same step with all of a stage's loads: the B tile of stage T + NB
    // into LB, then the A tile of stage T + NA into LA (NA = 2: A first),
    // placed as w64_load_after says.
#define FCR_STEP2(CUR, NXT, RA, RB, KS, LOADS, LA, LB, T)                                             \
    {                                                                                                  \
        const uint32_t sb_ = FCR_STEP_B((T) + NB), sa_ = FCR_STEP_A((T) + NA);                         \
        const __amdgpu_buffer_rsrc_t rb_ = FCR_RB((T) + NB), ra_ = FCR_RA((T) + NA);                   \
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
            if constexpr (NA == 3) {                                                                   \
                if (l_ >= 0 && l_ < kLB)                                                               \
                    db.issue_one(rb_, LB, sb_, wave, l_);                                              \
                else if (l_ >= kLB)                                                                    \
                    da.issue_one(ra_, LA, sa_, wave, l_ - kLB);                                        \
            } else {                                                                                   \
                if (l_ >= 0 && l_ < kLA)                                                               \
                    da.issue_one(ra_, LA, sa_, wave, l_);                                              \
                else if (l_ >= kLA)                                                                    \
                    db.issue_one(rb_, LB, sb_, wave, l_ - kLA);                                        \
            }                                                                                          \
        }                                                                                              \
    }
    // stage T with A tile P mod NA and B tile P mod NB (P = T mod 6): step 0
    // (loads the far operand's tile of stage T + 2, into the tile stage T - 1
    // freed), the barrier (those loads may still be in flight), step 1 (reads
    // step 0 of stage T + 1; loads the near operand's tile of stage T + 2 into
    // the tile stage T frees). Without kSpread: step 0 without loads, the
    // barrier (the far operand's loads, issued last, may still be in flight),
    // step 1 with the B tile of stage T + NB and the A tile of stage T + NA,
    // both into the tiles stage T frees.
#define FCR_FAR_TILE(I) (NA == 3 ? FCR_TA(I) : FCR_TB(I))
#define FCR_NEAR_TILE(I) (NA == 3 ? FCR_TB(I) : FCR_TA(I))
#define FCR_STAGE(P, T)                                                                                \
    if constexpr (kSpread) {                                                                           \
        FCR_STEP(0, 1, FCR_TA((P) % NA), FCR_TB((P) % NB), 1, true, true, FCR_FAR_TILE(((P) + 2) % 3), T) \
        waitcnt<kFar, 0>();                                                                            \
        __builtin_amdgcn_s_barrier();                                                                  \
        FCR_STEP(1, 0, FCR_TA(((P) + 1) % NA), FCR_TB(((P) + 1) % NB), 0, true, false,                 \
                 FCR_NEAR_TILE((P) % 2), T)                                                            \
    } else {                                                                                           \
        FCR_STEP2(0, 1, FCR_TA((P) % NA), FCR_TB((P) % NB), 1, false, ta0, tb0, T)                     \
        waitcnt<kFar, 0>();                                                                            \
        __builtin_amdgcn_s_barrier();                                                                  \
        FCR_STEP2(1, 0, FCR_TA(((P) + 1) % NA), FCR_TB(((P) + 1) % NB), 0, true, FCR_TA((P) % NA),     \
                  FCR_TB((P) % NB), T)                                                                 \
    }

    if (nkt > 0) {
        const __amdgpu_buffer_rsrc_t rza = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, 0, 0, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rzb = __builtin_amdgcn_make_buffer_rsrc((void*)g.B, 0, 0, kRsrcWord3);
        if constexpr (HEAD < 0) {
            // The loop runs whole periods of six stages: pad virtual stages
            // -pad .. -1 go first and load through zero-size descriptors, so
            // their tiles hold zeros and their MFMAs add nothing.
            const int pad = (6 - nkt % 6) % 6;
            // stages -pad and -pad + 1, and without kSpread the far operand's
            // tile of -pad + 2 (else stage -pad's step 0 loads it); wait for
            // the first; read its step 0
            da.issue_full(FCR_RA(-pad), ta0, FCR_STEP_A(-pad), wave);
            db.issue_full(FCR_RB(-pad), tb0, FCR_STEP_B(-pad), wave);
            da.issue_full(FCR_RA(1 - pad), ta1, FCR_STEP_A(1 - pad), wave);
            db.issue_full(FCR_RB(1 - pad), tb1, FCR_STEP_B(1 - pad), wave);
            if constexpr (!kSpread) {
                if constexpr (NA == 3)
                    da.issue_full(FCR_RA(2 - pad), ta2, FCR_STEP_A(2 - pad), wave);
                else
                    db.issue_full(FCR_RB(2 - pad), ta2, FCR_STEP_B(2 - pad), wave);
            }
            waitcnt<kLA + kLB + (kSpread ? 0 : kFar), 0>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int i = 0; i < 8; ++i) FCR_FA(0, i) = fragment_mf<A_OC, BKP, MF>(ta0, wm0 + i * MF, 0, lane);
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
            // stages 0 .. HEAD - 1 take period positions P0 .. 5; stages 0 and
            // 1 (without kSpread also stage 2's tile of the operand with three
            // tiles) go to those positions' tiles
            constexpr int P0 = 6 - HEAD;
            da.issue_full(w.ra, FCR_TA(P0 % NA), FCR_STEP_A(0), wave);
            db.issue_full(w.rb, FCR_TB(P0 % NB), FCR_STEP_B(0), wave);
            da.issue_full(w.ra, FCR_TA((P0 + 1) % NA), FCR_STEP_A(1), wave);
            db.issue_full(w.rb, FCR_TB((P0 + 1) % NB), FCR_STEP_B(1), wave);
            if constexpr (!kSpread) {
                if constexpr (NA == 3)
                    da.issue_full(w.ra, FCR_TA((P0 + 2) % 3), FCR_STEP_A(2), wave);
                else
                    db.issue_full(w.rb, FCR_TB((P0 + 2) % 3), FCR_STEP_B(2), wave);
            }
            waitcnt<kLA + kLB + (kSpread ? 0 : kFar), 0>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int i = 0; i < 8; ++i)
                FCR_FA(0, i) = fragment_mf<A_OC, BKP, MF>(FCR_TA(P0 % NA), wm0 + i * MF, 0, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[0][j] = fragment_mf<B_OC, BKP, MF, BN>(FCR_TB(P0 % NB), wn0 + j * MF, 0, lane);
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
#undef FCR_FA
#undef FCR_STEP2
#undef FCR_FAR_TILE
#undef FCR_NEAR_TILE
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

// Head forms that run out of registers and spill in their main loop are not
// built; those cases run the padded form: at 256 columns, both operands
// output-contiguous with a head of 4 stages.
constexpr bool head_spills(bool a_oc, bool b_oc, int head) { return FCW4_RING_BN == 256 && a_oc && b_oc && head == 4; }
#define FCW4_HEAD4_SPILLS_OC_OC (FCW4_RING_BN == 256)

// Explicit instantiations (the host pass emits a launch stub for each): the
// padded form and the head forms that are built.
#define FCW4_RI(AOC, BOC, F32, HEAD) \
    template __global__ void gemm_w4k64r_kernel<AOC, BOC, F32, FCW4_RING_BN, HEAD, FCW4_RING_NA>(GemmArgs);
#define FCW4_RI3(AOC, BOC, F32) FCW4_RI(AOC, BOC, F32, -1) FCW4_RI(AOC, BOC, F32, 2) FCW4_RI(AOC, BOC, F32, 4)
#define FCW4_RIH(AOC, BOC, F32) FCW4_RI(AOC, BOC, F32, 2) FCW4_RI(AOC, BOC, F32, 4)
FCW4_RI3(false, false, false)
FCW4_RI3(false, false, true)
FCW4_RI3(true, false, false)
FCW4_RI3(true, false, true)
FCW4_RI(false, true, false, -1)
FCW4_RI(false, true, true, -1)
FCW4_RI(true, true, false, -1)
FCW4_RI(true, true, true, -1)
FCW4_RIH(false, true, false)
FCW4_RIH(false, true, true)
FCW4_RI(true, true, false, 2)
FCW4_RI(true, true, true, 2)
#if !FCW4_HEAD4_SPILLS_OC_OC
FCW4_RI(true, true, false, 4)
FCW4_RI(true, true, true, 4)
#endif
#undef FCW4_RIH
#undef FCW4_RI3
#undef FCW4_RI
#undef FCW4_HEAD4_SPILLS_OC_OC

// the instance for a head form, or the padded one where no head form is
// built (the padded form is correct for any stage count); its name as
// profilers show it
template <bool AOC, bool BOC, bool F32, int HEAD>
constexpr W4Kernel ring_entry(const char* name, const char* padded_name) {
    constexpr bool padded = HEAD < 0 || head_spills(AOC, BOC, HEAD);
    return W4Kernel{gemm_w4k64r_kernel<AOC, BOC, F32, FCW4_RING_BN, padded ? -1 : HEAD, FCW4_RING_NA>,
                    padded ? padded_name : name};
}

}  // namespace

#define FCW4_STR2(X) #X
#define FCW4_STR(X) FCW4_STR2(X)
#define FCW4_RN(AOC, BOC, F32, H)                                                                                 \
    "gemm_w4k64r_kernel<" #AOC ", " #BOC ", " #F32 ", " FCW4_STR(FCW4_RING_BN) ", " #H ", " FCW4_STR(FCW4_RING_NA) \
    ">"
#define FCW4_RE1(AOC, BOC, F32, H) ring_entry<AOC, BOC, F32, H>(FCW4_RN(AOC, BOC, F32, H), FCW4_RN(AOC, BOC, F32, -1))

template <>
W4Kernel w4_ring_kernel<FCW4_RING_BN, FCW4_RING_NA>(int head, bool a_oc, bool b_oc, bool out_f32) {
#define FCW4_RE(AOC, BOC, F32) \
    {FCW4_RE1(AOC, BOC, F32, -1), FCW4_RE1(AOC, BOC, F32, 2), FCW4_RE1(AOC, BOC, F32, 4)}
    // [out_f32][a_oc][b_oc][padded, head 2, head 4]
    static const W4Kernel table[8][3] = {FCW4_RE(false, false, false), FCW4_RE(false, true, false),
                                         FCW4_RE(true, false, false),  FCW4_RE(true, true, false),
                                         FCW4_RE(false, false, true),  FCW4_RE(false, true, true),
                                         FCW4_RE(true, false, true),   FCW4_RE(true, true, true)};
#undef FCW4_RE
#undef FCW4_RE1
#undef FCW4_RN
#undef FCW4_STR
#undef FCW4_STR2
    return table[(out_f32 ? 4 : 0) + (a_oc ? 2 : 0) + (b_oc ? 1 : 0)][head == 2 ? 1 : head == 4 ? 2 : 0];
}

}  // namespace fcs
