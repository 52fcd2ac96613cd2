// Pieces shared by the 4-wave, one-wave-per-SIMD bf16 GEMM kernels for
// gfx950 (gemm_w4.hip, gemm_w4_ring*.hip): block set-up, the placement of
// fragment reads and loads within a step, the accumulator fences and the
// AGPR-pinned MFMA. Internal; every function is inline.
#pragma once

#include "gemm_common.h"

namespace fcs {
namespace {

constexpr int kW4Threads = 256;

// block set-up shared by the kernels
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

// The ring kernels' placement of NR fragment reads (NR <= 8 + TN) in a step:
// with SPREAD, one after the second MFMA of each group of TN / 2 (over the
// step's 16 groups), else one or two after the first MFMAs of the first
// groups. The rings spread them at 256 columns when an operand is
// output-contiguous (two transposing reads per fragment): against two per
// group, 2-3 % fewer main-loop cycles and 1-2.5 % less time; with both
// operands reduction-contiguous spreading cost about 1 %.
template <int TN, bool SPREAD = false>
__device__ constexpr int w64_read_after_n(int nr, int u) {
    constexpr int gs = TN / 2, rpg = SPREAD ? 1 : gs > 2 ? 2 : gs - 1;
    const int r = rpg * (u / gs) + (u % gs) - 1;
    return (u % gs != 0 && u % gs <= rpg && r < nr) ? r : -1;
}

// The ring kernels' placement of NL loads in a step (NL <= 16): spread over
// the whole step, load l after the first MFMA of group 16 l / NL (the reads
// go after later MFMAs of a group, w64_read_after_n). Half a stage's loads per step and at most
// one load per group keep the direct-to-LDS load rate of the 4 waves at half
// of what the texture path moves per clock; all 16 in one step hit that rate
// and the full address FIFO then blocks the wave's next MFMAs.
template <int TN>
__device__ constexpr int w64_load_spread(int nl, int u) {
    constexpr int gs = TN / 2;
    if (nl <= 0 || u % gs != 0) return -1;
    const int g = u / gs, l = (g * nl + 15) / 16;
    return (l < nl && (16 * l) / nl == g) ? l : -1;
}

// Zeroes the accumulators with MFMAs of zero operands (the MFMA pipe is
// idle while the first stages load): written in place by asm outputs, the
// zeros need no AGPR moves into the registers the asm MFMAs use (zeroed in
// C++, they were materialised elsewhere, then copied, about 1000 cycles
// after the first stage had landed). The zero operand is written by VALU
// moves the compiler places just before: an MFMA reading a VGPR that a VALU
// instruction wrote needs wait states first, which the compiler does not
// insert ahead of asm, so each MFMA brings its own. w4_acc_fence (or, with
// no stage to run, w4_acc_drain) must follow.
template <int TN>
__device__ __forceinline__ void w4_acc_zero(f32x4 (&acc)[8][TN]) {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            asm volatile("s_nop 2\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(acc[i][j]) : "v"(z));
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

}  // namespace
}  // namespace fcs
