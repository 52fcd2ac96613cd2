// Bandwidth-bound helper kernels of the shard GEMM path (gfx950):
//  * transpose_bf16 - the "copy" arm of the layout tuner: rewrites an
//    output-contiguous operand as reduction-contiguous, so the GEMM can run
//    with both operands read along the reduction;
//  * pad_rows_bf16  - copies a reduction-contiguous operand to rows padded
//    with zeros to a whole number of 64-value stages;
//  * splitk_reduce  - sums fp32 split-K partials in a fixed slice order and
//    rounds once (bf16 nearest-even) or stores fp32;
//  * fill_bf16      - deterministic values for the tuner's scratch operands.
#include <algorithm>

#include "fcshard_internal.h"

namespace fcs {

namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 64;  // transpose tile edge

// 64 x 64 tiles through LDS; 256 threads, each moves 16 elements in and out.
// The LDS row pitch of 65 elements keeps column reads free of bank conflicts.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int64_t rows,
                                                             int64_t cols, int64_t tiles_c) {
    __shared__ uint16_t t[kT][kT + 1];
    const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
    const int64_t r0 = tr * kT, c0 = tc * kT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 16 x 16 threads
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = ty + 16 * k;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = tx * 4 + e;
            const int64_t gr = r0 + r, gc = c0 + c;
            t[r][c] = (gr < rows && gc < cols) ? src[gr * cols + gc] : (uint16_t)0;
        }
    }
    __syncthreads();
    // dst[c][r] = t[r][c]; each thread writes 4 consecutive r of one c
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = ty + 16 * k;
        const int64_t gc = c0 + c;
        if (gc >= cols) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = tx * 4 + e;
            const int64_t gr = r0 + r;
            if (gr < rows) dst[gc * rows + gr] = t[r][c];
        }
    }
}

// Vectorized variant for rows, cols multiples of 8 and 16-byte aligned bases.
__global__ __launch_bounds__(256) void transpose_bf16_v8_kernel(const uint16_t* __restrict__ src,
                                                                uint16_t* __restrict__ dst, int64_t rows,
                                                                int64_t cols, int64_t tiles_c) {
    __shared__ uint16_t t[kT][kT + 2];
    const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
    const int64_t r0 = tr * kT, c0 = tc * kT;
    // load: 64 rows x 8 vectors of 8; thread -> (row = tid / 8 + 32 k, vec = tid % 8)
    const int vr = threadIdx.x >> 3, vc = threadIdx.x & 7;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = vr + 32 * k;
        const int64_t gr = r0 + r, gc = c0 + vc * 8;
        u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (gr < rows && gc < cols) v = *reinterpret_cast<const u16x8*>(src + gr * cols + gc);
#pragma unroll
        for (int e = 0; e < 8; ++e) t[r][vc * 8 + e] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = vr + 32 * k;
        const int64_t gc = c0 + c, gr = r0 + vc * 8;
        if (gc < cols && gr < rows) {
            u16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = t[vc * 8 + e][c];
            *reinterpret_cast<u16x8*>(dst + gc * rows + gr) = v;
        }
    }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, void* __restrict__ out,
                                                            bool out_f32, bool accumulate, int64_t n, int splits,
                                                            int64_t stride, bool vec) {
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= n) return;
    if (vec && i4 + 4 <= n) {
        f32x4 s = *reinterpret_cast<const f32x4*>(ws + i4);
        for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(ws + k * stride + i4);
        if (out_f32) {
            float* o = static_cast<float*>(out) + i4;
            if (accumulate) s = *reinterpret_cast<const f32x4*>(o) + s;
            *reinterpret_cast<f32x4*>(o) = s;
        } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + i4) =
                bf16x4{(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
        }
        return;
    }
    for (int64_t i = i4; i < n && i < i4 + 4; ++i) {
        float s = ws[i];
        for (int k = 1; k < splits; ++k) s += ws[k * stride + i];
        if (out_f32)
            static_cast<float*>(out)[i] = accumulate ? static_cast<float*>(out)[i] + s : s;
        else
            static_cast<__bf16*>(out)[i] = (__bf16)s;
    }
}

// splitk_reduce into a sub-rectangle of a wider output: 4 values per thread,
// cols a multiple of 4
__global__ __launch_bounds__(256) void splitk_reduce_rect_kernel(const float* __restrict__ ws, void* __restrict__ out,
                                                                 bool out_f32, bool accumulate, int64_t rows,
                                                                 int64_t cols, int64_t ldc, int splits,
                                                                 int64_t stride) {
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= rows * cols) return;
    const int64_t r = i4 / cols, c = i4 - r * cols;
    f32x4 s = *reinterpret_cast<const f32x4*>(ws + i4);
    for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(ws + k * stride + i4);
    if (out_f32) {
        float* o = static_cast<float*>(out) + r * ldc + c;
        if (accumulate) s = *reinterpret_cast<const f32x4*>(o) + s;
        *reinterpret_cast<f32x4*>(o) = s;
    } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + r * ldc + c) =
            bf16x4{(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
    }
}

// dst row r = src row r (cols values) then zeros up to ld; 8 values (16 B)
// per thread and step, grid-stride over rows x ld / 8
__global__ __launch_bounds__(256) void pad_rows_bf16_kernel(const uint16_t* __restrict__ src,
                                                            uint16_t* __restrict__ dst, int64_t rows, int64_t cols,
                                                            int64_t ld) {
    const int64_t per_row = ld / 8, total = rows * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / per_row, c = (i - r * per_row) * 8;
        uint4 v = {0u, 0u, 0u, 0u};
        if (c < cols) v = *reinterpret_cast<const uint4*>(src + r * cols + c);
        *reinterpret_cast<uint4*>(dst + r * ld + c) = v;
    }
}

__global__ __launch_bounds__(256) void fill_bf16_kernel(uint16_t* p, int64_t n, uint32_t seed) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    // integer hash -> 8 significant bits in [-1, 1)
    uint32_t h = (uint32_t)i * 0x9E3779B1u ^ seed;
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    const float v = (float)((int)(h & 0xFF) - 128) * (1.0f / 128.0f);
    const __bf16 b = (__bf16)v;
    p[i] = *reinterpret_cast<const uint16_t*>(&b);
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                 hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t tiles_r = (rows + kT - 1) / kT, tiles_c = (cols + kT - 1) / kT;
    const int64_t blocks = tiles_r * tiles_c;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const bool vec = (rows % 8 == 0) && (cols % 8 == 0) && ((uintptr_t)src % 16 == 0) &&
                     ((uintptr_t)dst % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(transpose_bf16_v8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, rows,
                           cols, tiles_c);
    else
        hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, rows,
                           cols, tiles_c);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* ws, void* out, bool out_f32, bool accumulate, int64_t n, int splits,
                                int64_t stride, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t threads = (n + 3) / 4;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    // vector path: 16-byte partial loads and 8/16-byte output stores
    const bool vec = (stride % 4 == 0) && ((uintptr_t)ws % 16 == 0) &&
                     ((uintptr_t)out % (out_f32 ? 16 : 8) == 0);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, out, out_f32,
                       out_f32 && accumulate, n, splits, stride, vec);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce_rect(const float* ws, void* out, bool out_f32, bool accumulate, int64_t rows,
                                     int64_t cols, int64_t ldc, int splits, int64_t stride, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    if (cols % 4 != 0 || ldc < cols || ldc % 4 != 0 || stride % 4 != 0 || (uintptr_t)ws % 16 != 0 ||
        (uintptr_t)out % (out_f32 ? 16 : 8) != 0)
        return hipErrorInvalidValue;
    const int64_t blocks = (rows * cols / 4 + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_reduce_rect_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, out, out_f32,
                       out_f32 && accumulate, rows, cols, ldc, splits, stride);
    return hipGetLastError();
}

hipError_t launch_pad_rows_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols, int64_t ld,
                                hipStream_t stream) {
    if (rows <= 0 || ld <= 0) return hipSuccess;
    if (cols % 8 != 0 || ld % 8 != 0 || cols > ld || (uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0)
        return hipErrorInvalidValue;
    const int64_t work = rows * (ld / 8);
    const int64_t blocks = std::min<int64_t>((work + 255) / 256, 8192);
    hipLaunchKernelGGL(pad_rows_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, rows, cols, ld);
    return hipGetLastError();
}

hipError_t launch_fill_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, seed);
    return hipGetLastError();
}

}  // namespace fcs
