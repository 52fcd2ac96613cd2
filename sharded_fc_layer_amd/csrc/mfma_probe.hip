// Measurement aid: the MFMA stream of the one-wave-per-SIMD GEMM kernels
// with everything else taken away. One block of 4 waves per compute unit
// (one wave per SIMD), each wave issuing v_mfma_f32_16x16x32_bf16 back to
// back into the 256 AGPR accumulators of a 128 x 128 wave tile, through the
// same AGPR-pinned MFMA as the GEMMs (mfma_agpr), with no loads, no LDS
// accesses and no barriers in the loop. Its rate is what the chip sustains
// for this instruction stream at the clock it holds under that load: the
// empirical peak that the GEMMs' utilisation is measured against (the pages
// quote their efficiency as a percentage of an empirical peak:
// pith.science/paper/2502.08145, "Assumptions & free parameters").
//
// Each block also reads the shader-clock counter (s_memtime) and the
// constant-rate counter (s_memrealtime) before and after its loop, so the
// host can derive the engine clock over the run. A short launch of it after
// each GEMM of a step (fc_mfma_probe_launch) samples the clock that the GEMM
// left the chip at.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <vector>

#include "fcshard.h"
#include "gemm_w4_common.h"

namespace fcs {
namespace {

constexpr int kProbeMfmaPerIter = 64;

__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void mfma_probe_kernel(
    int64_t iters, unsigned long long* clocks) {
    const int lane = threadIdx.x & 63;
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // operands that depend on the lane; small values keep the sums finite
    // (the MFMAs are volatile asm: they run whatever becomes of their results)
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)((float)((lane + e) & 7) * 0.0078125f);
        b[e] = (__bf16)((float)((lane * 3 + e) & 7) * 0.0078125f);
    }
    w4_acc_fence(acc);
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
        // each accumulator is read again 64 MFMAs later, as in the GEMMs' steps
#pragma unroll
        for (int u = 0; u < kProbeMfmaPerIter; ++u) mfma_agpr(acc[u / 8][u % 8], b, a);
    }
    w4_acc_drain(acc);
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clocks[4 * blockIdx.x + 0] = t0;
        clocks[4 * blockIdx.x + 1] = t1;
        clocks[4 * blockIdx.x + 2] = r0;
        clocks[4 * blockIdx.x + 3] = r1;
    }
}

fc_status probe_device(int* dev, int* cus, int* wall_khz) {
    hipDeviceProp_t prop;
    if (hipGetDevice(dev) != hipSuccess || hipGetDeviceProperties(&prop, *dev) != hipSuccess) return FC_E_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return FC_E_UNSUPPORTED;
    if (hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, *dev) != hipSuccess || *wall_khz <= 0)
        return FC_E_HIP;
    *cus = prop.multiProcessorCount;
    return FC_OK;
}

struct ProbeBuffers {
    unsigned long long* clocks = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    ~ProbeBuffers() {
        if (clocks) (void)hipFree(clocks);
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
    }
};

}  // namespace
}  // namespace fcs

using namespace fcs;

extern "C" fc_status fc_mfma_probe_launch(int64_t iters, int blocks, void* clocks, void* stream) {
    if (!clocks || iters < 1 || iters > ((int64_t)1 << 40) || blocks < 0 || blocks > (1 << 20)) return FC_E_INVALID;
    if ((uintptr_t)clocks % 8) return FC_E_INVALID;
    int dev, cus, wall_khz;
    fc_status st = probe_device(&dev, &cus, &wall_khz);
    if (st != FC_OK) return st;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks ? blocks : cus), dim3(kW4Threads), 0,
                       static_cast<hipStream_t>(stream), iters, static_cast<unsigned long long*>(clocks));
    return hipGetLastError() == hipSuccess ? FC_OK : FC_E_HIP;
}

extern "C" fc_status fc_mfma_probe(int64_t iters, fc_mfma_probe_result* out, void* stream) {
    if (!out || iters < 1 || iters > ((int64_t)1 << 40)) return FC_E_INVALID;
    int dev, blocks, wall_khz;
    fc_status st = probe_device(&dev, &blocks, &wall_khz);
    if (st != FC_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    ProbeBuffers b;
    if (hipMalloc(&b.clocks, (size_t)blocks * 4 * sizeof(unsigned long long)) != hipSuccess) {
        (void)hipGetLastError();
        return FC_E_NOMEM;
    }
    if (hipEventCreate(&b.ev[0]) != hipSuccess || hipEventCreate(&b.ev[1]) != hipSuccess) return FC_E_HIP;
    // a short warm-up launch, then the timed one
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kW4Threads), 0, s, (int64_t)1 + iters / 16, b.clocks);
    if (hipEventRecord(b.ev[0], s) != hipSuccess) return FC_E_HIP;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kW4Threads), 0, s, iters, b.clocks);
    if (hipGetLastError() != hipSuccess || hipEventRecord(b.ev[1], s) != hipSuccess) return FC_E_HIP;
    if (hipEventSynchronize(b.ev[1]) != hipSuccess) return FC_E_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, b.ev[0], b.ev[1]) != hipSuccess) return FC_E_HIP;
    std::vector<unsigned long long> c((size_t)blocks * 4);
    if (hipMemcpy(c.data(), b.clocks, c.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
        return FC_E_HIP;
    double ratio = 0.0;
    int n = 0;
    for (int i = 0; i < blocks; ++i) {
        const double dt = (double)(c[4 * i + 1] - c[4 * i + 0]), dr = (double)(c[4 * i + 3] - c[4 * i + 2]);
        if (dr > 0) ratio += dt / dr, ++n;
    }
    out->ms = ms;
    out->flops = (double)blocks * 4.0 * (double)iters * kProbeMfmaPerIter * (16.0 * 16.0 * 32.0 * 2.0);
    out->compute_units = blocks;
    out->counter_ratio = n ? ratio / n : 0.0;
    out->wall_clock_mhz = wall_khz / 1000.0;
    return FC_OK;
}
