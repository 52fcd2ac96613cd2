// Internal interface between the C ABI (fcshard_api.hip) and the gfx950
// kernels (gemm_bf16.hip, aux_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fcs {

// One GEMM C[M x N] = A[M x K] . B[K x N] in the kernels' own terms:
// M = output rows, N = output cols, K = reduction length. Each operand is
// either reduction-contiguous (RC) or output-contiguous (OC):
//   A RC: A(i, r) = A[i * lda + r]      A OC: A(i, r) = A[r * lda + i]
//   B RC: B(r, j) = B[j * ldb + r]      B OC: B(r, j) = B[r * ldb + j]
// C is row-major (bf16 or fp32) with leading dimension ldc: N, or more when
// C is a sub-rectangle of a wider output (the one-wave-per-SIMD kernels'
// epilogues honour ldc; every other kernel is only launched with ldc = N).
struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t M, N, K;
    int64_t lda, ldb;
    int64_t ldc;
    int64_t k_split;         // reduction elements per split slice (multiple of 64)
    int splits;              // number of reduction slices; 1 = no split
    int64_t c_split_stride;  // elements between the slices' fp32 partial outputs
    int accumulate;          // 1: fp32 C += product (one slice only); 0: C = product
    // measurement stamps: the stamped ring kernel (gemm_w4k64r_stamped_kernel)
    // writes kStampSlots counter readings per block there (slots described in
    // gemm_w4_ring_body.inc); every other kernel ignores it
    unsigned long long* stamps = nullptr;
};
constexpr int kStampSlots = 8;

struct TileCfg {
    int bm, bn;        // block tile (output rows x output cols)
    const char* name;  // e.g. "256x256"
};

constexpr int kNumTiles = 4;
extern const TileCfg kTiles[kNumTiles];
constexpr int kUnalignedTile = 3;  // the one tile the unaligned kernels use

// Enqueue one GEMM kernel. `aligned` selects the 16-byte vector kernels,
// valid only when M, N, K are multiples of 8 and A, B, C are 16-byte aligned.
hipError_t launch_gemm(int tile, bool a_oc, bool b_oc, bool out_f32, bool aligned,
                       const GemmArgs& args, hipStream_t stream);

// Name of that kernel instance, as profilers show it (for plan descriptions).
const char* gemm_kernel_name(int tile, bool a_oc, bool b_oc, bool out_f32, bool aligned);

// Enqueue one pipelined GEMM kernel (gemm_pipe.hip). Valid only when M, N,
// K are multiples of 8, A, B, C are 16-byte aligned and A and B each span
// less than 2 GiB.
hipError_t launch_gemm_pipe(int tile, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                            hipStream_t stream);
const char* pipe_kernel_name(int tile, bool a_oc, bool b_oc, bool out_f32);

// Enqueue an 8-wave ping-pong GEMM (256 x 256 tile; same requirements as
// launch_gemm_pipe). variant bit 0: one barrier per reduction stage
// (gemm_pp1b_kernel) instead of two (gemm_pp_kernel); bit 1: 16x16x32 MFMAs
// instead of 32x32x16.
hipError_t launch_gemm_pingpong(int variant, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                                hipStream_t stream);
const char* pingpong_kernel_name(int variant, bool a_oc, bool b_oc, bool out_f32);

// Enqueue the 4-wave (one wave per SIMD) GEMM, 256 x bn block tile, 128 x
// bn / 2 per wave with 16x16x32 MFMAs (gemm_w4.hip; same requirements as
// launch_gemm_pipe; variant 0: K and slices multiples of 64; variant 1: an
// even number of 64-value stages per slice). A reduction that is not a
// multiple of 64 ends with a partial stage. Variant 1: reduction-contiguous
// operands must then have rows padded with zeros up to the next multiple of
// 64 (lda / ldb the padded length); output-contiguous ones read zeros past
// row K. Variants 2 and 3 load the partial stage themselves, 16-byte chunks
// past K reading zeros (K a multiple of 8), and need no padding.
// variant 0: 32-value reduction stages in 4 LDS slots; 1: 64-value stages in
// 2 slots (whole-cache-line rows for reduction-contiguous operands); 2: the
// same 64-value stages in a ring of 3 A and 2 B tiles, so each load has about
// two stages to land; 3: the ring mirrored, with 2 A and 3 B tiles, so the B
// operand's loads have the longer lead. bn is 256, or 192 for variants 1
// to 3. The rings run
// its reduction in periods of 6 stages; when every slice's stage count mod
// 6 is 2 or 4 it starts with that many straight-line stages (the last
// positions of a period), else it pads the front with zero stages.
hipError_t launch_gemm_w4(int variant, int bn, bool a_oc, bool b_oc, bool out_f32, const GemmArgs& args,
                          hipStream_t stream);
// (K, k_split, splits: the reduction slicing, which picks the ring kernel's
// head form)
const char* w4_kernel_name(int variant, int bn, bool a_oc, bool b_oc, bool out_f32, int64_t K, int64_t k_split,
                           int splits);

// One kernel instance and its name as profilers show it.
struct W4Kernel {
    void (*fn)(GemmArgs);
    const char* name;
};

// The ring kernel (variant 2 above) for block-tile width BN (256 or 192)
// with NA A tiles and 5 - NA B tiles (3 + 2, or 2 + 3): head = 2 or 4 picks
// the head form, anything else the padded one. Defined in
// gemm_w4_ring256.hip, gemm_w4_ring192.hip, gemm_w4_ring256b.hip and
// gemm_w4_ring192b.hip.
template <int BN, int NA>
W4Kernel w4_ring_kernel(int head, bool a_oc, bool b_oc, bool out_f32);
template <>
W4Kernel w4_ring_kernel<256, 3>(int head, bool a_oc, bool b_oc, bool out_f32);
template <>
W4Kernel w4_ring_kernel<192, 3>(int head, bool a_oc, bool b_oc, bool out_f32);
template <>
W4Kernel w4_ring_kernel<256, 2>(int head, bool a_oc, bool b_oc, bool out_f32);
template <>
W4Kernel w4_ring_kernel<192, 2>(int head, bool a_oc, bool b_oc, bool out_f32);

// The ring kernel with measurement stamps (GemmArgs::stamps): 256-column
// block tiles, NA A tiles (3 or 2), bf16 output; head as for
// w4_ring_kernel. Defined in gemm_w4_ring256.hip and gemm_w4_ring256b.hip.
template <int NA>
W4Kernel w4_ring_stamp_kernel(int head, bool a_oc, bool b_oc);
template <>
W4Kernel w4_ring_stamp_kernel<3>(int head, bool a_oc, bool b_oc);
template <>
W4Kernel w4_ring_stamp_kernel<2>(int head, bool a_oc, bool b_oc);

// Enqueue that kernel (variant 2 or 3 of launch_gemm_w4, 256 columns): one
// reduction slice, bf16 output, args.stamps set (kStampSlots values per
// block, blocks = ceil(M / 256) * ceil(N / 256)).
hipError_t launch_gemm_w4_stamped(int variant, bool a_oc, bool b_oc, const GemmArgs& args, hipStream_t stream);

// dst (cols x rows, row-major) = transpose of src (rows x cols, row-major), bf16.
hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                 hipStream_t stream);

// dst (rows x ld, row-major) = src (rows x cols, row-major) with zeros in
// columns cols .. ld - 1; cols and ld multiples of 8, 16-byte aligned.
hipError_t launch_pad_rows_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols, int64_t ld,
                                hipStream_t stream);

// out[i] = sum_{s < splits} ws[s * stride + i] (fixed order), stored bf16 or
// fp32; with `accumulate` (fp32 only) out[i] = out[i] + that sum.
hipError_t launch_splitk_reduce(const float* ws, void* out, bool out_f32, bool accumulate, int64_t n, int splits,
                                int64_t stride, hipStream_t stream);

// The same sum into a sub-rectangle: out[r * ldc + c] (+)= sum_s ws[s * stride
// + r * cols + c], r < rows, c < cols (cols a multiple of 4; 16-byte aligned
// planes; the output 8- or 16-byte aligned).
hipError_t launch_splitk_reduce_rect(const float* ws, void* out, bool out_f32, bool accumulate, int64_t rows,
                                     int64_t cols, int64_t ldc, int splits, int64_t stride, hipStream_t stream);

// Deterministic pseudo-random bf16 fill in [-1, 1) (tuning buffers only).
hipError_t launch_fill_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t stream);

}  // namespace fcs
