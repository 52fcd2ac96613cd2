// The ring kernel (gemm_w4k64r_kernel) and its instances for one block-tile
// width, FCW4_RING_BN (256 or 192), and one split of the five LDS tiles,
// FCW4_RING_NA A tiles (3 unless set), set by the including source file; each
// such pair is its own translation unit so that the build compiles them in
// parallel. Requirements as in gemm_w4.hip (K a multiple of 8, split slices
// multiples of 64).
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
// stages, no extra work, and still one control path. A reduction range that
// ends with a partial stage (fewer than 64 values) takes the padded form:
// that stage goes first, in the place of the first virtual stage (one to six
// of them), and its loads alone check each 16-byte chunk against the end of
// the range, so the main loop is the same.
//
// NA = 2 mirrors the ring: two A tiles and three B tiles (ta2 is the third B
// tile); the B tile of stage t + 2 is loaded in step 0 and the A tile in
// step 1, so the B operand gets the longer lead.
template <bool A_OC, bool B_OC, bool OUT_F32, int BN, int HEAD, int NA>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4k64r_kernel(
    GemmArgs g) {
    constexpr bool STAMP = false;
#include "gemm_w4_ring_body.inc"
}

// The same kernel writing measurement stamps to g.stamps (a measurement aid:
// the same body, so the same main-loop instructions, plus the readings).
template <bool A_OC, bool B_OC, bool OUT_F32, int BN, int HEAD, int NA>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4k64r_stamped_kernel(
    GemmArgs g) {
    constexpr bool STAMP = true;
#include "gemm_w4_ring_body.inc"
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

#if FCW4_RING_BN == 256
// The stamped instances (STAMP = true) of the bf16-output forms, a
// measurement aid (launch_gemm_w4_stamped): the same code with counter
// readings written per block. The padded form stands in for head forms that
// are not built, as in the table below.
namespace {
#define FCW4_RS(AOC, BOC, HEAD) \
    template __global__ void gemm_w4k64r_stamped_kernel<AOC, BOC, false, 256, HEAD, FCW4_RING_NA>(GemmArgs);
FCW4_RS(false, false, -1) FCW4_RS(false, false, 2) FCW4_RS(false, false, 4)
FCW4_RS(false, true, -1) FCW4_RS(false, true, 2) FCW4_RS(false, true, 4)
FCW4_RS(true, false, -1) FCW4_RS(true, false, 2) FCW4_RS(true, false, 4)
FCW4_RS(true, true, -1) FCW4_RS(true, true, 2)
#undef FCW4_RS
template <bool AOC, bool BOC, int HEAD>
constexpr W4Kernel ring_stamp_entry() {
    constexpr bool padded = HEAD < 0 || head_spills(AOC, BOC, HEAD);
    return W4Kernel{gemm_w4k64r_stamped_kernel<AOC, BOC, false, 256, padded ? -1 : HEAD, FCW4_RING_NA>,
                    "gemm_w4k64r_stamped_kernel"};
}
}  // namespace

template <>
W4Kernel w4_ring_stamp_kernel<FCW4_RING_NA>(int head, bool a_oc, bool b_oc) {
#define FCW4_RSE(AOC, BOC) {ring_stamp_entry<AOC, BOC, -1>(), ring_stamp_entry<AOC, BOC, 2>(), ring_stamp_entry<AOC, BOC, 4>()}
    static const W4Kernel table[4][3] = {FCW4_RSE(false, false), FCW4_RSE(false, true), FCW4_RSE(true, false),
                                         FCW4_RSE(true, true)};
#undef FCW4_RSE
    return table[(a_oc ? 2 : 0) + (b_oc ? 1 : 0)][head == 2 ? 1 : head == 4 ? 2 : 0];
}
#endif

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
