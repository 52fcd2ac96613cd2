// Device-side building blocks shared by the gfx950 GEMM kernels
// (gemm_pipe.hip, gemm_w4.hip): LDS tile layouts and swizzles, direct-to-LDS
// loads, MFMA operand reads, the MFMA wrappers, the epilogue and the
// XCD-aware block-to-tile map. Internal; every function is inline.
#pragma once

#include "fcshard_internal.h"

namespace fcs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kBK = 32;        // reduction values per stage
constexpr int kStages = 4;     // LDS ring depth
constexpr int kThreads = 256;  // 4 waves
constexpr uint32_t kOOB = 0x80000000u;       // offset past any operand (< 2 GiB)
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data format

__device__ __forceinline__ uint32_t rc_slot(int i, int c) { return i * 64 + ((c ^ ((i >> 2) & 3)) << 4); }

// Reduction-contiguous tile row of BKP values: 16-byte chunk c of row i.
// 32 values (64 B rows): chunk ^ ((i >> 2) & 3). 64 values (128 B rows, one
// cache line): chunk ^ ((i >> 1) & 7), so the 16 rows one 16-lane group of a
// 16x16x32 operand read touches fall on 16 different 16-byte bank groups.
template <int BKP>
__device__ __forceinline__ int rc_swizzle(int i) {
    static_assert(BKP == 32 || BKP == 64, "32- or 64-value rows");
    return BKP == 32 ? ((i >> 2) & 3) : ((i >> 1) & 7);
}
template <int BKP>
__device__ __forceinline__ uint32_t rc_slot_k(int i, int c) {
    return i * (BKP * 2) + ((c ^ rc_swizzle<BKP>(i)) << 4);
}

// Output-contiguous tile row k (R values): 16-byte chunk c XOR (k & 3) << 2,
// and bit 1 of the XOR from bit 3 of k. A half-wave ds_read_b64_tr_b16 of a
// 16x16x32 operand reads rows k0 .. k0+3 and k0+8 .. k0+11 (32 B each); with
// bit 3 folded in, those 8 rows fall on 8 different 32-byte bank groups
// (conflict-free; with (k & 3) << 2 alone, rows k and k + 8 shared banks).
// The 32x32x16 operand reads 4 rows x 64 B per half-wave, conflict-free either way.
__device__ __forceinline__ int oc_swizzle(int k) { return ((k & 3) << 2) | ((k & 8) >> 2); }
// Rows of 192 values (384 B, 24 chunks): row k starts on 32-byte bank group
// 4 (k & 1) (mod 8), and the XOR may only permute chunks within groups of 8.
// XOR-ing the chunk with 2 t, t = bit 1 of k | (bit 3 of k) << 1, gives the
// even rows of a half-wave read (k0, k0+2, k0+8, k0+10) four different t, and
// the odd rows likewise: again 8 different bank groups.
template <int R>
__device__ __forceinline__ int oc_swizzle_r(int k) {
    if constexpr (R == 192)
        return (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1;
    else
        return oc_swizzle(k);
}
template <int R>
__device__ __forceinline__ uint32_t oc_slot(int k, int c) {
    return k * (R * 2) + ((c ^ oc_swizzle_r<R>(k)) << 4);
}

// s_waitcnt with vmcnt = vm, lgkmcnt = lgkm (expcnt not waited)
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
    static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14));
}

// One operand tile of R rows (output index) x 32 reduction values per stage.
template <int R, bool OC>
struct Dma {
    static constexpr int kInstr = R / 64;  // 1 KB instructions per wave per stage
    uint32_t base[kInstr];                 // byte offset at reduction 0, or kOOB
    int kk[kInstr];                        // reduction offset of the chunk within a stage

    __device__ __forceinline__ void init(int wave, int lane, int64_t ld, int64_t row0, int64_t rows) {
#pragma unroll
        for (int j = 0; j < kInstr; ++j) {
            if (!OC) {
                const int i = (wave * kInstr + j) * 16 + (lane >> 2);
                const int c = (lane & 3) ^ ((lane >> 4) & 3);
                kk[j] = 8 * c;
                base[j] = (row0 + i < rows) ? (uint32_t)(((row0 + i) * ld + 8 * c) * 2) : kOOB;
            } else {
                constexpr int CPR = R / 8;     // 16-byte chunks per reduction row
                constexpr int RPI = 64 / CPR;  // reduction rows per instruction
                const int k = (wave * kInstr + j) * RPI + lane / CPR;
                const int c = (lane % CPR) ^ oc_swizzle(k);
                kk[j] = k;
                base[j] = (row0 + 8 * c < rows) ? (uint32_t)(((int64_t)k * ld + row0 + 8 * c) * 2) : kOOB;
            }
        }
    }

    // issue instructions j in [lo, hi) of this wave's share of one stage
    template <int LO, int HI>
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, char* region, int64_t k0, int64_t kend,
                                          int64_t ld, int wave) const {
        const uint32_t step = OC ? (uint32_t)(k0 * ld * 2) : (uint32_t)(k0 * 2);
#pragma unroll
        for (int j = (LO > 0 ? LO : 0); j < (HI < kInstr ? HI : kInstr); ++j) {
            const uint32_t off = (base[j] == kOOB || k0 + kk[j] >= kend) ? kOOB : base[j] + step;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(region + (wave * kInstr + j) * 1024), 16,
                                                     off, 0, 0, 0);
        }
    }
};

// MFMA operand of one 32-row block (rows r0 .. r0+31), reduction step ks (16 values)
template <int R, bool OC>
__device__ __forceinline__ bf16x8 fragment(const char* region, int r0, int ks, int lane) {
    if (!OC) {
        const int i = r0 + (lane & 31);
        const int c = ks * 2 + (lane >> 5);
        return *reinterpret_cast<const bf16x8*>(region + rc_slot(i, c));
    } else {
        const int g = lane >> 4, j = lane & 15;
        const int col = r0 + 16 * (g & 1) + 4 * (j & 3);
        const int k = ks * 16 + 8 * (g >> 1) + (j >> 2);
        const int c = col >> 3, half = (col & 7) << 1;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(region + oc_slot<R>(k, c) + half));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(region + oc_slot<R>(k + 4, c) + half));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
}

// loads of one operand tile (R rows x BKP reduction values) shared by 4 waves
template <bool OC, int BKP, int R = 256>
struct DmaPP {
    static_assert(BKP == 32 || BKP == 64, "32- or 64-value stages");
    static_assert(R == 256 || (BKP == 64 && R == 192), "tile rows");
    static constexpr int kInstr = R * BKP * 2 / 1024 / 4;  // per wave
    uint32_t base[kInstr];
    int kk[kInstr];

    // 32-bit unsigned arithmetic: the operand is smaller than 2 GiB, so every
    // in-range offset fits, and rows and row0 are below 2^32 (an offset of a
    // row past the operand may wrap: it is replaced by kOOB)
    __device__ __forceinline__ void init(int wq, int lane, int64_t ld, int64_t row0, int64_t rows) {
        const uint32_t ld32 = (uint32_t)ld, r0 = (uint32_t)row0, nrows = (uint32_t)rows;
#pragma unroll
        for (int j = 0; j < kInstr; ++j) {
            const uint32_t p = (uint32_t)((wq * kInstr + j) * 64 + lane);  // 16-byte slot in the tile
            if (!OC) {
                constexpr uint32_t CPR = BKP / 8;
                const uint32_t i = p / CPR, pc = p % CPR;
                const uint32_t c = pc ^ (uint32_t)rc_swizzle<BKP>((int)i);
                kk[j] = (int)(8 * c);
                base[j] = r0 + i < nrows ? ((r0 + i) * ld32 + 8 * c) * 2 : kOOB;
            } else {
                constexpr uint32_t CPR = R / 8;
                const uint32_t k = p / CPR;
                const uint32_t c = (p % CPR) ^ (uint32_t)oc_swizzle_r<R>((int)k);
                kk[j] = (int)k;
                base[j] = r0 + 8 * c < nrows ? (k * ld32 + r0 + 8 * c) * 2 : kOOB;
            }
        }
    }

    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, char* region, int64_t k0, int64_t kend,
                                          int64_t ld, int wq) const {
        const uint32_t step = OC ? (uint32_t)(k0 * ld * 2) : (uint32_t)(k0 * 2);
#pragma unroll
        for (int j = 0; j < kInstr; ++j) {
            const uint32_t off = (base[j] == kOOB || k0 + kk[j] >= kend) ? kOOB : base[j] + step;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(region + (wq * kInstr + j) * 1024), 16,
                                                     off, 0, 0, 0);
        }
    }

    // Load instruction j alone of issue_full (for hand-interleaved schedules).
    // The stage offset goes in the scalar offset (no per-load vector add):
    // callers clamp stages to the reduction range, so in-range lanes stay
    // inside the operand, and rows past the matrix keep their out-of-range
    // vector offset (kOOB + step < 2^32 stays past the buffer either way).
    __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rsrc, char* region, uint32_t step, int wq,
                                              int j) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(region + (wq * kInstr + j) * 1024), 16,
                                                 base[j], step, 0, 0);
    }

    // Same loads for a stage that lies wholly inside the reduction range (no
    // per-chunk reduction check): `step` is the stage's byte offset along the
    // reduction. Rows past the operand keep their out-of-range base, and
    // kOOB + step stays below 2^32 and past the buffer, so they still read zeros.
    __device__ __forceinline__ void issue_full(__amdgpu_buffer_rsrc_t rsrc, char* region, uint32_t step,
                                               int wq) const {
#pragma unroll
        for (int j = 0; j < kInstr; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(region + (wq * kInstr + j) * 1024), 16,
                                                     base[j] + step, 0, 0, 0);
    }
};

template <bool OC, int BKP>
__device__ __forceinline__ bf16x8 fragment_pp(const char* region, int r0, int ks, int lane) {
    if constexpr (!OC) {
        const int i = r0 + (lane & 31);
        const int c = ks * 2 + (lane >> 5);
        return *reinterpret_cast<const bf16x8*>(region + rc_slot(i, c));
    } else {
        return fragment<256, true>(region, r0, ks, lane);
    }
}

// accumulator type and MFMA of one output block: 32 x 32 x 16 or 16 x 16 x 32
template <int MF>
struct AccT;
template <>
struct AccT<32> {
    typedef f32x16 type;
    static constexpr int n = 16;
};
template <>
struct AccT<16> {
    typedef f32x4 type;
    static constexpr int n = 4;
};

template <int MF>
__device__ __forceinline__ typename AccT<MF>::type mfma_bf16(bf16x8 a, bf16x8 b, typename AccT<MF>::type c) {
    if constexpr (MF == 32)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MFMA operand of an MF-row block at r0, reduction step ks of a BKP-value stage.
// 16 x 16 x 32: lane l holds block row l % 16 and reduction values
// 32 ks + 8 (l / 16) .. +7; for output-contiguous tiles the 16-lane group g
// reads rows 32 ks + 8 g (+4) with two ds_read_b64_tr_b16.
template <bool OC, int BKP, int MF, int R = 256>
__device__ __forceinline__ bf16x8 fragment_mf(const char* region, int r0, int ks, int lane) {
    if constexpr (MF == 32) {
        return fragment_pp<OC, BKP>(region, r0, ks, lane);
    } else if constexpr (!OC) {
        const int i = r0 + (lane & 15);
        const int c = ks * 4 + (lane >> 4);
        return *reinterpret_cast<const bf16x8*>(region + rc_slot_k<BKP>(i, c));
    } else {
        const int g = lane >> 4, j = lane & 15;
        const int col = r0 + 4 * (j & 3);
        const int k = ks * 32 + 8 * g + (j >> 2);
        const int c = col >> 3, half = (col & 7) << 1;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(region + oc_slot<R>(k, c) + half));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(region + oc_slot<R>(k + 4, c) + half));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
}

// epilogue of one wave tile: rows m0 + wm0 .., columns n0 + wn0 ..; each lane
// holds 4 consecutive output columns of one row per block
template <int MF, int TM, int TN, bool OUT_F32>
__device__ __forceinline__ void store_tile(const GemmArgs& g, int slice, int64_t m0, int64_t n0, int wm0, int wn0,
                                           int lane, const typename AccT<MF>::type (&acc)[TM][TN]) {
    constexpr int GR = MF == 32 ? 4 : 1;  // 4-column groups per lane per block
    const int lr = lane & (MF - 1), lk = MF == 32 ? (lane >> 5) : (lane >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm0 + i * MF + lr;
        if (m >= g.M) continue;
        float* crow = static_cast<float*>(g.C) + (int64_t)slice * g.c_split_stride + m * g.N;
        // an accumulating output: this row block's old values are loaded
        // first, so their latencies overlap (as in store_tile_f32_staged)
        [[maybe_unused]] f32x4 old[TN][GR];
        if (OUT_F32 && g.accumulate) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int gq = 0; gq < GR; ++gq) {
                    const int64_t n = n0 + wn0 + j * MF + gq * 8 + lk * 4;
                    old[j][gq] = n < g.N ? *reinterpret_cast<const f32x4*>(crow + n) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int gq = 0; gq < GR; ++gq) {
                const int64_t n = n0 + wn0 + j * MF + gq * 8 + lk * 4;
                if (n >= g.N) continue;
                const float v0 = acc[i][j][gq * 4 + 0], v1 = acc[i][j][gq * 4 + 1];
                const float v2 = acc[i][j][gq * 4 + 2], v3 = acc[i][j][gq * 4 + 3];
                if (OUT_F32) {
                    f32x4 v{v0, v1, v2, v3};
                    if (g.accumulate) v += old[j][gq];
                    *reinterpret_cast<f32x4*>(crow + n) = v;
                } else {
                    __bf16* c = static_cast<__bf16*>(g.C) + m * g.N + n;
                    *reinterpret_cast<bf16x4*>(c) = bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                }
            }
        }
    }
}

// bf16 epilogue of a 128 x 16 TN wave tile of 16 x 16 blocks (acc[i][j]: lane
// holds row 16 i + lane % 16, columns 16 j + 4 (lane / 16) .. +3), staged
// through `stage`, 32 KB of LDS that this wave alone uses (rows of 256 B
// whatever TN; chunks past the tile's columns stay unused). Written straight
// from the registers, each store instruction would cover 16 rows x 32 B
// (quarter cache lines); staged, the wave writes its 8-byte pieces into LDS
// rows of 256 B and reads back 16-byte chunks, so each store writes 4 rows x
// 256 B of whole 128-byte lines, with half as many store instructions. The
// 16-byte chunk index in an LDS row is XOR-swizzled by the row (mod 16):
// a half-wave's writes (16 rows x 16 B) and a row's reads (16 chunks) then
// fall on distinct banks. Needs N % 8 == 0, ldc % 8 == 0 and a 16-byte-aligned C.
template <int TN>
__device__ __forceinline__ void store_tile_bf16_staged(const GemmArgs& g, int64_t m0, int64_t n0, int wm0, int wn0,
                                                       int lane, const f32x4 (&acc)[8][TN], char* stage) {
    const int lr = lane & 15, lk = lane >> 4;
    // Reading back: lane = 16-byte chunk ch of rows 4 u + rq of a 16-row
    // group. Rows are stored in order, so the store address is one running
    // pointer (an add per store); a wave tile wholly inside the output
    // stores without per-row checks.
    const int rq = lane >> 4, ch = lane & 15;
    const int64_t row0 = m0 + wm0 + rq, col = n0 + wn0 + ch * 8;
    __bf16* cp = static_cast<__bf16*>(g.C) + row0 * g.ldc + col;
    const int64_t step = 4 * g.ldc;
    const bool full = m0 + wm0 + 128 <= g.M && n0 + wn0 + 16 * TN <= g.N;
    const bool col_in = col < g.N && (TN == 8 || ch < 2 * TN);
    // Software-pipelined over the 8 groups of 16 rows (acc[i]): group i is
    // converted and written while group i - 1's 4 stores drain, then read
    // back, so the AGPR reads and conversions (VALU) overlap the stores
    // (texture path) instead of preceding them all.
    bf16x8 v[2][4];
#pragma unroll
    for (int i = 0; i <= 8; ++i) {
        if (i < 8) {  // convert and write group i
            const int row = i * 16 + lr;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int cc = j * 16 + lk * 4;
                const uint32_t off = row * 256 + (((cc >> 3) ^ (row & 15)) << 4) + ((cc & 7) << 1);
                const f32x4 a = acc[i][j];
                *reinterpret_cast<bf16x4*>(stage + off) = bf16x4{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
            }
        }
        if (i > 0) {  // store group i - 1 (rows 16 (i - 1) + 4 u + rq)
            const bf16x8* w = v[(i - 1) & 1];
            if (full) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (TN == 8 || ch < 2 * TN) *reinterpret_cast<bf16x8*>(cp + u * step) = w[u];
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (col_in && row0 + 16 * (i - 1) + 4 * u < g.M) *reinterpret_cast<bf16x8*>(cp + u * step) = w[u];
            }
            cp += 4 * step;
        }
        if (i < 8) {  // read group i back
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int row = i * 16 + 4 * u + rq;
                v[i & 1][u] = *reinterpret_cast<const bf16x8*>(stage + row * 256 + ((ch ^ (row & 15)) << 4));
            }
        }
        asm volatile("" ::: "memory");  // keeps the groups in this order
    }
}

// fp32 epilogue of the same wave tile (fp32 and accumulating outputs,
// split-K partial planes), staged the same way and software-pipelined over
// the eight 16-row groups like the bf16 one: group i is written into one of
// two 8 KB LDS buffers (rows of 512 B, the 16-byte chunk XOR-swizzled by
// (row & 7) << 1, which spreads both a half-wave's writes and a row's reads
// evenly over the banks) while group i - 1's stores drain, then read back.
// Each store writes 2 rows x 512 B of whole lines. An accumulating output's
// old values are loaded one group ahead, so their latency overlaps a group's
// work, and added before the store. Within one wave, LDS accesses complete
// in order, so group i + 2 may overwrite the buffer group i was read from.
template <int TN>
__device__ __forceinline__ void store_tile_f32_staged(const GemmArgs& g, int slice, int64_t m0, int64_t n0, int wm0,
                                                      int wn0, int lane, const f32x4 (&acc)[8][TN], char* stage) {
    const int lr = lane & 15, lk = lane >> 4;
    float* C = static_cast<float*>(g.C) + (int64_t)slice * g.c_split_stride;
    // reading back: lane = 16-byte chunk ch of rows 2 u + rq of a group
    const int rq = lane >> 5, ch = lane & 31;
    const int64_t row0 = m0 + wm0 + rq, col = n0 + wn0 + 4 * ch;
    // running pointers (an add per access): stores, and an accumulating
    // output's old values one group ahead
    float* cp = C + row0 * g.ldc + col;
    const float* op = cp;
    const int64_t step = 2 * g.ldc;
    const bool full = m0 + wm0 + 128 <= g.M && n0 + wn0 + 16 * TN <= g.N;
    const bool col_in = col < g.N && (TN == 8 || ch < 4 * TN);
    f32x4 v[2][8], old[2][8];
    // the old values of group gi (accumulating output), zeros outside the output
#define FC_F32_LOAD_OLD(GI)                                                                                \
    _Pragma("unroll") for (int u = 0; u < 8; ++u) {                                                        \
        const int r_ = 16 * (GI) + 2 * u;                                                                  \
        old[(GI) & 1][u] = (col_in && row0 + r_ < g.M) ? *reinterpret_cast<const f32x4*>(op + u * step)    \
                                                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};                     \
    }                                                                                                      \
    op += 8 * step;
    if (g.accumulate) FC_F32_LOAD_OLD(0)
#pragma unroll
    for (int i = 0; i <= 8; ++i) {
        if (i < 8) {  // write group i
            char* buf = stage + (i & 1) * 8192;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c4 = 4 * j + lk;
                *reinterpret_cast<f32x4*>(buf + lr * 512 + ((c4 ^ ((lr & 7) << 1)) << 4)) = acc[i][j];
            }
        }
        if (i > 0) {  // store group i - 1 (rows 16 (i - 1) + 2 u + rq)
            const int gi = i - 1;
            f32x4 w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = g.accumulate ? v[gi & 1][u] + old[gi & 1][u] : v[gi & 1][u];
            if (full) {
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (TN == 8 || ch < 4 * TN) *reinterpret_cast<f32x4*>(cp + u * step) = w[u];
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (col_in && row0 + 16 * gi + 2 * u < g.M) *reinterpret_cast<f32x4*>(cp + u * step) = w[u];
            }
            cp += 8 * step;
        }
        if (i < 8) {
            if (i + 1 < 8 && g.accumulate) FC_F32_LOAD_OLD(i + 1)
            const char* buf = stage + (i & 1) * 8192;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 2 * u + rq;
                v[i & 1][u] = *reinterpret_cast<const f32x4*>(buf + r * 512 + ((ch ^ ((r & 7) << 1)) << 4));
            }
        }
        asm volatile("" ::: "memory");  // keeps the groups in this order
    }
#undef FC_F32_LOAD_OLD
}

// Output tile and reduction slice of this block. Blocks are dealt round robin
// to the 8 XCDs (block b to XCD b mod 8) and start roughly in block order, so
// the blocks running at one time are a window of consecutive ids. The map
// makes that window compact in two ways at once:
//  * across the chip: tiles are walked in super-tiles of 16 x 16 tiles (a
//    wave of 256 blocks), super-tiles left to right along a band of 16 tile
//    rows, bands top to bottom. A wave then reads 16 A and 16 B panels, which
//    the XCDs share through the MALL (each XCD owning its own band instead,
//    a wave would stream 8 x 12 different panels);
//  * within an XCD: id mod 8 is the XCD, and in a full super-tile XCD x
//    takes an 8 x 4 sub-block (rows 8 (x / 4) .., columns 4 (x mod 4) ..), so
//    its 32 running tiles share 8 A and 4 B panels in its L2.
// Partial super-tiles at the right and bottom edges split between the XCDs
// by columns (h rows x w / 8 columns each) or rows when the sizes allow it,
// else go column by column.
struct BlockTile {
    int slice;
    int64_t m0, n0;
};

template <int BM, int BN>
__device__ __forceinline__ BlockTile map_block(const GemmArgs& g) {
    constexpr int S = 16;  // super-tile side, in tiles
    const int nbm = (int)((g.M + BM - 1) / BM);
    const int nbn = (int)((g.N + BN - 1) / BN);
    const int tiles = nbm * nbn;
    const int lin = blockIdx.x;
    const int slice = lin / tiles;
    int t = lin - slice * tiles;
    const int sr = t / (S * nbn);  // band of S tile rows (the last one may be shorter)
    const int h = (nbm - S * sr) < S ? (nbm - S * sr) : S;
    t -= sr * S * nbn;
    const int sc = t / (S * h);  // super-tile in the band (the last one may be narrower)
    const int w = (nbn - S * sc) < S ? (nbn - S * sc) : S;
    const int q = t - sc * S * h;  // 0 .. h w - 1
    const int x = q & 7, k = q >> 3;
    int r, c;
    if (h == S && w % 4 == 0) {  // XCD x: rows 8 (x / 4) .. + 8, w / 4 columns
        r = 8 * (x >> 2) + (k & 7);
        c = (w >> 2) * (x & 3) + (k >> 3);
    } else if (w % 8 == 0) {  // XCD x: all h rows, w / 8 columns
        r = k % h;
        c = (w >> 3) * x + k / h;
    } else if (h % 8 == 0) {  // XCD x: h / 8 rows, all w columns
        const int hx = h >> 3;
        r = hx * x + k % hx;
        c = k / hx;
    } else {
        r = q % h;
        c = q / h;
    }
    return BlockTile{slice, (int64_t)(S * sr + r) * BM, (int64_t)(S * sc + c) * BN};
}

}  // namespace
}  // namespace fcs
