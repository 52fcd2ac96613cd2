// C ABI of the shard GEMM library: validation, storage-order resolution,
// plan space, plan cache, workspace and the per-shape tuner.
//
// The three products of one GPU's FC-layer shard (sciencestack.ai/paper/
// 2502.08145, Figure 1) map onto one GEMM family C = A.B whose operands are
// either reduction-contiguous (RC) or output-contiguous (OC) in memory:
//
//   product          A        B        row/row   row/col   col/row   col/col
//   forward Y=X.W    X        W        RC,OC     RC,RC     OC,OC     OC,RC
//   bwd-data dX      dY       W^T      RC,RC     RC,OC     RC,RC     RC,OC
//   bwd-weight dW    X^T      dY       OC,OC     OC,OC     RC,OC     RC,OC
//
// (orders are x_order/w_order). A plan chooses the block tile, a split of the
// reduction (fp32 partials summed in a fixed order) and whether OC operands
// are first copied to RC form in the workspace (the tuner's transpose-vs-copy
// choice, after the pages' automated kernel tuning: sciencestack.ai/paper/
// 2502.08145, TL;DR).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "fcshard.h"
#include "fcshard_internal.h"

namespace fcs {
namespace {

// split slot 3: split 2 of the tail only (tail_geometry below)
constexpr int kSplits[] = {1, 2, 4, 2};
constexpr int kNumSplits = 4;
constexpr int kTailSplit = 3;
constexpr int kNumCopy = 4;      // bit 0: copy A to RC, bit 1: copy B to RC
// 0: 4-wave pipelined, 1: simple, 2-5: 8-wave ping-pong (256 x 256), variant
// = family - 2: bit 0 one barrier per stage, bit 1 16x16x32 MFMAs;
// 6-8: 4-wave, one wave per SIMD, 128 x 128 wave tiles (256 x 256), with
// 32-value stages (6), 64-value stages in two LDS slots (7) or in a ring of
// three A and two B tiles (8), or in the mirrored ring of two A and three B
// tiles (9). Families 7-9 also run 256 x 192 block tiles (tile 2; 128 x 96
// per wave): where 256 x 256 tiles leave CUs idle (192 tiles on 256 CUs),
// 256 x 192 ones may fill them (256 tiles).
constexpr int kNumFamilies = 10;
constexpr int kFamilyW4 = 6;
constexpr int kNumPlans = kNumTiles * kNumSplits * kNumCopy * kNumFamilies;
constexpr int64_t kPipeMaxBytes = (int64_t)1 << 31;
constexpr int64_t kMaxDim = (int64_t)1 << 31;    // largest M, K or N
constexpr int64_t kMaxElems = (int64_t)1 << 46;  // largest element count of X, W, dY or an output
constexpr int kMaxDevices = 64;

struct Plan {
    int tile;
    int split;   // number of reduction slices requested (for tail plans: of the tail)
    bool tail;   // only the tiles past the last whole wave are split (families 8, 9)
    int copy;    // bit mask
    int family;  // 0 pipelined, 1 simple, 2-5 ping-pong variants (family - 2), 6-9 one wave per SIMD
};

Plan decode_plan(int id) {
    Plan p;
    p.tile = id % kNumTiles;
    const int si = (id / kNumTiles) % kNumSplits;
    p.split = kSplits[si];
    p.tail = si == kTailSplit;
    p.copy = (id / (kNumTiles * kNumSplits)) % kNumCopy;
    p.family = id / (kNumTiles * kNumSplits * kNumCopy);
    return p;
}

int encode_plan(int tile, int split_idx, int copy, int family) {
    return tile + kNumTiles * (split_idx + kNumSplits * (copy + kNumCopy * family));
}

// block-tile width (output columns) of a one-wave-per-SIMD plan
int w4_bn(const Plan& pl) { return pl.family > kFamilyW4 && pl.tile == 2 ? 192 : 256; }

// One GEMM in kernel terms, resolved from an ABI call.
struct Problem {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    bool a_oc, b_oc, out_f32;
    bool accumulate;  // fp32 output: C += product
    int64_t M, N, K;  // output rows, output cols, reduction
};

bool problem_aligned(const Problem& p) {
    return p.M % 8 == 0 && p.N % 8 == 0 && p.K % 8 == 0 && (uintptr_t)p.A % 16 == 0 &&
           (uintptr_t)p.B % 16 == 0 && (uintptr_t)p.C % 16 == 0;
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// A tail plan (families 8 and 9; 256-row block tiles): when the output's
// tiles are more than one wave (256 CUs) but not whole waves, the tiles of
// the last partial wave, at most 128 of them, either the last tile columns
// or the last tile rows, run as their own launch with the reduction split in
// two (fp32 partials, then the fixed-order sum into that part of the
// output): that wave then takes about half a round instead of a whole one.
// The rest (whole waves) runs unsplit. main = the output columns (along_n)
// or rows of the unsplit part.
struct TailGeo {
    bool ok, along_n;
    int64_t main;
};

int64_t gcd64(int64_t a, int64_t b) { return b ? gcd64(b, a % b) : a; }

TailGeo tail_geometry(const Problem& p, int bn) {
    TailGeo t{false, false, 0};
    const int64_t nbm = (p.M + 255) / 256, nbn = (p.N + bn - 1) / bn, tiles = nbm * nbn;
    if (tiles <= 256 || tiles % 256 == 0) return t;
    // tile columns (rows) whose count times the rows (columns) is a whole
    // number of waves, the rest at most 128 tiles
    const int64_t step_n = 256 / gcd64(nbm, 256), main_n = (nbn - 1) / step_n * step_n;
    if (main_n > 0 && nbm * (nbn - main_n) <= 128) return TailGeo{true, true, main_n * bn};
    const int64_t step_m = 256 / gcd64(nbn, 256), main_m = (nbm - 1) / step_m * step_m;
    if (main_m > 0 && nbn * (nbm - main_m) <= 128) return TailGeo{true, false, main_m * 256};
    return t;
}

// Effective reduction slicing: slice length is a multiple of 64.
void split_geometry(int64_t K, int split, int64_t* k_split, int* slices) {
    if (split <= 1) {
        *k_split = round_up(K, 64);
        *slices = 1;
        return;
    }
    int64_t ks = round_up((K + split - 1) / split, 64);
    *k_split = ks;
    *slices = (int)((K + ks - 1) / ks);
}

// A reduction that is not a multiple of 64 ends with a partial stage.
// Family 7 pads it: each reduction-contiguous operand is copied to rows of
// round_up(K, 64) values with zeros past K (its last 64-value stage then
// reads zeros there), while output-contiguous operands read zeros past row K
// through their buffer bounds. The rings (families 8 and 9) load the partial
// stage themselves, chunks past K reading zeros, and copy a
// reduction-contiguous operand to such padded rows only when the plan's copy
// bit for it is set: rows of K values then start part-way into a 128-byte
// line (every other row when K is an odd multiple of 32), so that a stage
// of them touches two lines, which the copy trades for its own traffic (the
// tuner weighs it). A plan does not combine padding with a transpose copy.
bool pads_a(const Problem& p, const Plan& pl) {
    if (p.K % 64 == 0 || p.a_oc) return false;
    return pl.family == kFamilyW4 + 1 || (pl.family >= kFamilyW4 + 2 && (pl.copy & 1));
}
bool pads_b(const Problem& p, const Plan& pl) {
    if (p.K % 64 == 0 || p.b_oc) return false;
    return pl.family == kFamilyW4 + 1 || (pl.family >= kFamilyW4 + 2 && (pl.copy & 2));
}
bool pads_reduction(const Problem& p, const Plan& pl) { return pads_a(p, pl) || pads_b(p, pl); }

struct WsLayout {
    int64_t a_off, b_off, p_off, total;
};

WsLayout ws_layout(const Problem& p, const Plan& pl) {
    WsLayout w{0, 0, 0, 0};
    int64_t off = 0;
    const bool pad_a = pads_a(p, pl), pad_b = pads_b(p, pl);
    const int64_t kp = round_up(p.K, 64);
    if (((pl.copy & 1) && p.a_oc) || pad_a) {
        w.a_off = off;
        off += round_up(p.M * (pad_a ? kp : p.K) * 2, 256);
    }
    if (((pl.copy & 2) && p.b_oc) || pad_b) {
        w.b_off = off;
        off += round_up(p.N * (pad_b ? kp : p.K) * 2, 256);
    }
    int64_t ks;
    int slices;
    split_geometry(p.K, pl.split, &ks, &slices);
    if (pl.tail) {  // partial planes of the tail part only
        const TailGeo t = tail_geometry(p, w4_bn(pl));
        const int64_t tail_elems = t.along_n ? p.M * (p.N - t.main) : (p.M - t.main) * p.N;
        w.p_off = off;
        off += round_up((int64_t)slices * tail_elems * 4, 256);
    } else if (slices > 1) {
        w.p_off = off;
        off += round_up((int64_t)slices * p.M * p.N * 4, 256);
    }
    w.total = off;
    return w;
}

// Is the plan meaningful for this problem?
bool plan_applies(const Problem& p, const Plan& pl) {
    // a copy bit transposes an output-contiguous operand, or (rings, a
    // reduction that is not a multiple of 64) pads a reduction-contiguous one
    const bool ring_pads = pl.family >= kFamilyW4 + 2 && p.K % 64 != 0;
    if ((pl.copy & 1) && !p.a_oc && !ring_pads) return false;
    if ((pl.copy & 2) && !p.b_oc && !ring_pads) return false;
    const bool aligned_after_copy = p.M % 8 == 0 && p.N % 8 == 0 && p.K % 8 == 0 &&
                                    (uintptr_t)p.C % 16 == 0 &&
                                    ((pl.copy & 1) || (uintptr_t)p.A % 16 == 0) &&
                                    ((pl.copy & 2) || (uintptr_t)p.B % 16 == 0);
    if (!aligned_after_copy && (pl.family != 1 || pl.tile != kUnalignedTile)) return false;
    if (pl.family >= 2 && pl.tile != 0 && !(w4_bn(pl) == 192)) return false;
    if (pl.family >= kFamilyW4) {
        int64_t ks;
        int slices;
        split_geometry(p.K, pl.split, &ks, &slices);
        if (pl.family == kFamilyW4) {  // 32-value stages in pairs: whole 64-value units, no padding
            if (p.K % 64 != 0 || ks % 64 != 0) return false;
        } else if (pl.family == kFamilyW4 + 1) {  // 64-value stages in pairs: even stage counts
            const int64_t first = (std::min(ks, p.K) + 63) / 64;
            const int64_t last = (p.K - (int64_t)(slices - 1) * ks + 63) / 64;
            if (first % 2 != 0 || last % 2 != 0) return false;
        }
        // family 7 pads every reduction-contiguous operand itself, a
        // transposed copy included, so it takes no copy then; a ring does not
        // combine a padded copy with a transposed one
        if (pl.family == kFamilyW4 + 1 && p.K % 64 != 0 && pl.copy != 0) return false;
        const bool transposes = ((pl.copy & 1) && p.a_oc) || ((pl.copy & 2) && p.b_oc);
        if (pads_reduction(p, pl) && transposes) return false;
        // a ring runs a partial last stage after at least one whole one (in
        // the slice that ends the reduction; a tail plan's main launch is
        // unsplit)
        if (pl.family >= kFamilyW4 + 2 && p.K % 64 != 0 && (p.K - (int64_t)(slices - 1) * ks < 64 || p.K < 64))
            return false;
    }
    if (pl.family != 1) {
        const int64_t k_a = pads_a(p, pl) ? round_up(p.K, 64) : p.K;
        const int64_t k_b = pads_b(p, pl) ? round_up(p.K, 64) : p.K;
        const int64_t a_bytes = ((pl.copy & 1) ? 0 : p.M * k_a * 2);
        const int64_t b_bytes = ((pl.copy & 2) ? 0 : p.N * k_b * 2);
        if (a_bytes >= kPipeMaxBytes || b_bytes >= kPipeMaxBytes || p.M * p.K * 2 >= kPipeMaxBytes ||
            p.N * p.K * 2 >= kPipeMaxBytes)
            return false;
    }
    if (pl.split > 1) {
        int64_t ks;
        int slices;
        split_geometry(p.K, pl.split, &ks, &slices);
        if (slices < 2) return false;
    }
    if (pl.tail) {  // the rings, no copies or padding, a tail to split
        if (pl.family < kFamilyW4 + 2 || pl.copy != 0 || pads_reduction(p, pl)) return false;
        if (!tail_geometry(p, w4_bn(pl)).ok) return false;
    }
    return true;
}

// ----------------------------------------------------------------- state

struct Key {
    int dev, op;
    int64_t M, K, N;
    int xo, wo, f32;
    bool operator<(const Key& o) const {
        return std::tie(dev, op, M, K, N, xo, wo, f32) < std::tie(o.dev, o.op, o.M, o.K, o.N, o.xo, o.wo, o.f32);
    }
};

// Device scratch of the no-allocation entry point (fc_bwd_weight_noalloc):
// split-K partial planes, transpose copies or padded operands of its plan.
// One copy per device, held from the library's load on that device to the
// end of the process. In host code `scratch` is a host-side stand-in, not
// the device address: host code only ever uses the address that
// hipGetSymbolAddress returns for the current device (DevState::scratch).
constexpr int64_t kNoallocScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

struct DevState {
    int checked = 0;  // 0 unknown, 1 gfx950, -1 other
    void* scratch = nullptr;  // this device's copy of `scratch`, once looked up
    char arch[64] = {0};
    void* ws = nullptr;
    int64_t ws_bytes = 0;
    // a hot call was captured into a graph while using the current workspace
    bool ws_captured = false;
    // workspaces superseded by a growth after such a capture: kept until
    // fc_release, because captured kernels keep the workspace address they
    // were captured with and may be replayed after the growth
    std::vector<void*> retired;
};

// A cached plan and, when fc_tune chose it, its measured time (median of the
// timed launches, ms); -1 when the plan was set or loaded without a time.
struct PlanEntry {
    int id;
    float ms;
};

// g_mu guards the plan cache and the device states. A hot call holds it from
// reading the workspace pointer until its kernels are enqueued, so a growth
// (which synchronizes the device before freeing) never frees a workspace that
// an enqueued or about-to-be-enqueued kernel uses. g_ws_mu is held by every
// call that may grow or free a workspace, or that runs the tuner's kernels on
// it, for its whole duration; it is taken before g_mu.
std::mutex g_mu;
std::mutex g_ws_mu;
std::map<Key, PlanEntry> g_plans;
DevState g_dev[kMaxDevices];

bool log_enabled() {
    static int v = -1;
    if (v < 0) {
        const char* e = std::getenv("FC_LOG");
        v = (e && *e && *e != '0') ? 1 : 0;
    }
    return v == 1;
}

fc_status check_device(int* dev_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FC_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FC_E_UNSUPPORTED;
    *dev_out = dev;
    DevState& d = g_dev[dev];
    if (d.checked == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FC_E_HIP;
        d.checked = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        std::snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
        for (char* c = d.arch; *c; ++c)
            if (*c == ' ' || *c == '\n') *c = '_';
    }
    return d.checked == 1 ? FC_OK : FC_E_UNSUPPORTED;
}

// default plan: no workspace, no split; the largest tile that still gives
// every CU work (every plan it returns has ws_layout(...).total == 0)
int default_plan(const Problem& p) {
    const int unaligned = encode_plan(kUnalignedTile, 0, 0, 1);
    if (!problem_aligned(p)) return unaligned;
    const int cus = 256;
    int tile = kUnalignedTile;  // 128x128
    for (int t = 0; t < kNumTiles; ++t) {
        const int64_t tiles = ((p.M + kTiles[t].bm - 1) / kTiles[t].bm) * ((p.N + kTiles[t].bn - 1) / kTiles[t].bn);
        if (tiles >= cus) {
            tile = t;
            break;
        }
    }
    // 256x256 tiles filling the chip: the ring kernel when its virtual (zero)
    // stages add at most 5 % to the reduction, else the two-slot kernel when
    // the reduction allows it without padding, else the ring if they add at
    // most 25 %, else the 8-wave ping-pong kernel; otherwise the 4-wave
    // pipelined kernel with the largest tile that still fills the chip (a
    // default plan never needs the workspace)
    const int ring = encode_plan(0, 0, 0, kFamilyW4 + 2);
    const bool ring_ok = tile == 0 && plan_applies(p, decode_plan(ring)) && ws_layout(p, decode_plan(ring)).total == 0;
    // the ring's virtual stages: none for a head form (stage count 2 or 4
    // mod 6 with a whole period after it), else those padding the count to
    // whole periods (a partial last stage takes one virtual stage's place)
    const int64_t whole = p.K / 64, stages = (p.K + 63) / 64;
    const int64_t virt = p.K % 64 != 0 ? 5 - whole % 6
                         : ((stages % 6 == 2 || stages % 6 == 4) && stages > 6) ? 0
                                                                               : (6 - stages % 6) % 6;
    if (ring_ok && virt * 20 <= stages) return ring;
    const int w64 = encode_plan(0, 0, 0, kFamilyW4 + 1);
    if (tile == 0 && plan_applies(p, decode_plan(w64)) && ws_layout(p, decode_plan(w64)).total == 0) return w64;
    if (ring_ok && virt * 4 <= stages) return ring;
    const int pp = encode_plan(0, 0, 0, 4);  // two-barrier ping-pong, 16x16x32
    if (tile == 0 && plan_applies(p, decode_plan(pp))) return pp;
    const int pipe = encode_plan(tile, 0, 0, 0);
    return plan_applies(p, decode_plan(pipe)) ? pipe : encode_plan(tile, 0, 0, 1);
}

// ------------------------------------------------------------- execution

// With `stamps`, the plan must be stampable (see stampable) and its GEMM
// runs the stamped ring instance, writing kStampSlots values per block.
hipError_t run_plan(const Problem& p0, const Plan& pl, void* ws, hipStream_t s,
                    unsigned long long* stamps = nullptr) {
    Problem p = p0;
    const WsLayout w = ws_layout(p0, pl);
    char* base = static_cast<char*>(ws);
    int64_t lda = p.a_oc ? p.M : p.K;
    int64_t ldb = p.b_oc ? p.N : p.K;
    hipError_t e;
    if ((pl.copy & 1) && p.a_oc) {  // A stored K x M -> M x K
        uint16_t* dst = reinterpret_cast<uint16_t*>(base + w.a_off);
        if ((e = launch_transpose_bf16(p.A, dst, p.K, p.M, s)) != hipSuccess) return e;
        p.A = dst;
        p.a_oc = false;
        lda = p.K;
    }
    if ((pl.copy & 2) && p.b_oc) {  // B stored K x N -> N x K
        uint16_t* dst = reinterpret_cast<uint16_t*>(base + w.b_off);
        if ((e = launch_transpose_bf16(p.B, dst, p.K, p.N, s)) != hipSuccess) return e;
        p.B = dst;
        p.b_oc = false;
        ldb = p.K;
    }
    if (pads_reduction(p0, pl)) {  // reduction-contiguous operands to rows of round_up(K, 64), zeros past K
        const int64_t kp = round_up(p.K, 64);
        if (pads_a(p0, pl)) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(base + w.a_off);
            if ((e = launch_pad_rows_bf16(p.A, dst, p.M, p.K, kp, s)) != hipSuccess) return e;
            p.A = dst;
            lda = kp;
        }
        if (pads_b(p0, pl)) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(base + w.b_off);
            if ((e = launch_pad_rows_bf16(p.B, dst, p.N, p.K, kp, s)) != hipSuccess) return e;
            p.B = dst;
            ldb = kp;
        }
    }
    int64_t ks;
    int slices;
    split_geometry(p.K, pl.split, &ks, &slices);
    const bool aligned = problem_aligned(p);
    GemmArgs g;
    g.A = p.A;
    g.B = p.B;
    g.M = p.M;
    g.N = p.N;
    g.K = p.K;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = p.N;
    g.k_split = ks;
    g.splits = slices;
    g.accumulate = 0;
    if (pl.tail) {  // whole waves unsplit, the tail split in two (see tail_geometry)
        const int bn = w4_bn(pl), variant = pl.family - kFamilyW4;
        const TailGeo t = tail_geometry(p, bn);
        const int64_t esz = p.out_f32 ? 4 : 2;
        GemmArgs gm = g, gt = g;
        gm.C = p.C;
        gm.k_split = round_up(p.K, 64);
        gm.splits = 1;
        gm.c_split_stride = 0;
        gm.accumulate = p.accumulate ? 1 : 0;
        char* ct = static_cast<char*>(p.C);
        if (t.along_n) {  // the tail is the output columns main .. N - 1
            gm.N = t.main;
            gt.N = p.N - t.main;
            gt.B = p.b_oc ? p.B + t.main : p.B + t.main * ldb;
            ct += t.main * esz;
        } else {  // the output rows main .. M - 1
            gm.M = t.main;
            gt.M = p.M - t.main;
            gt.A = p.a_oc ? p.A + t.main : p.A + t.main * lda;
            ct += t.main * p.N * esz;
        }
        if ((e = launch_gemm_w4(variant, bn, p.a_oc, p.b_oc, p.out_f32, gm, s)) != hipSuccess) return e;
        float* part = reinterpret_cast<float*>(base + w.p_off);
        gt.C = part;
        gt.ldc = gt.N;
        gt.c_split_stride = gt.M * gt.N;
        if ((e = launch_gemm_w4(variant, bn, p.a_oc, p.b_oc, true, gt, s)) != hipSuccess) return e;
        return launch_splitk_reduce_rect(part, ct, p.out_f32, p.accumulate, gt.M, gt.N, p.N, slices, gt.M * gt.N, s);
    }
    if (slices > 1) {  // partial planes, summed (and added to C) by the reduction
        float* part = reinterpret_cast<float*>(base + w.p_off);
        g.C = part;
        g.c_split_stride = p.M * p.N;
        e = pl.family == 0            ? launch_gemm_pipe(pl.tile, p.a_oc, p.b_oc, true, g, s)
            : pl.family >= kFamilyW4  ? launch_gemm_w4(pl.family - kFamilyW4, w4_bn(pl), p.a_oc, p.b_oc, true, g, s)
            : pl.family >= 2          ? launch_gemm_pingpong(pl.family - 2, p.a_oc, p.b_oc, true, g, s)
                             : launch_gemm(pl.tile, p.a_oc, p.b_oc, true, aligned, g, s);
        if (e != hipSuccess) return e;
        return launch_splitk_reduce(part, p.C, p.out_f32, p.accumulate, p.M * p.N, slices, p.M * p.N, s);
    }
    g.C = p.C;
    g.c_split_stride = 0;
    g.accumulate = p.accumulate ? 1 : 0;
    if (stamps) {
        g.stamps = stamps;
        return launch_gemm_w4_stamped(pl.family - kFamilyW4, p.a_oc, p.b_oc, g, s);
    }
    if (pl.family == 0) return launch_gemm_pipe(pl.tile, p.a_oc, p.b_oc, p.out_f32, g, s);
    if (pl.family >= kFamilyW4) return launch_gemm_w4(pl.family - kFamilyW4, w4_bn(pl), p.a_oc, p.b_oc, p.out_f32, g, s);
    if (pl.family >= 2) return launch_gemm_pingpong(pl.family - 2, p.a_oc, p.b_oc, p.out_f32, g, s);
    return launch_gemm(pl.tile, p.a_oc, p.b_oc, p.out_f32, aligned, g, s);
}

// ------------------------------------------------------------ validation

bool bad_order(int o) { return o != FC_ROW_MAJOR && o != FC_COL_MAJOR; }
bool bad_dtype(int d) { return d != FC_OUT_BF16 && d != FC_OUT_F32 && d != FC_OUT_F32_ACCUMULATE; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)abytes;
    const uintptr_t b0 = (uintptr_t)b, b1 = b0 + (uintptr_t)bbytes;
    return a0 < b1 && b0 < a1;
}

// Build the kernel-terms problem of one product (see the table at the top).
fc_status resolve(int op, const void* P, int p_order, const void* Q, int q_order, void* out, int dtype,
                  int64_t M, int64_t K, int64_t N, Problem* pr) {
    if (op < 0 || op > 2) return FC_E_INVALID;
    if (M < 1 || K < 1 || N < 1) return FC_E_INVALID;
    if (bad_order(p_order) || bad_order(q_order) || bad_dtype(dtype)) return FC_E_INVALID;
    if (M > kMaxDim || K > kMaxDim || N > kMaxDim) return FC_E_INVALID;
    // each matrix within kMaxElems elements (the products of two dimensions
    // fit 64 bits here), so that no byte count, offset or workspace size
    // derived from these sizes overflows
    if (M * K > kMaxElems || K * N > kMaxElems || M * N > kMaxElems) return FC_E_INVALID;
    Problem p;
    p.out_f32 = dtype != FC_OUT_BF16;
    p.accumulate = dtype == FC_OUT_F32_ACCUMULATE;
    p.A = static_cast<const uint16_t*>(P);
    p.B = static_cast<const uint16_t*>(Q);
    p.C = out;
    int64_t pbytes, qbytes, obytes;
    const int64_t esz = p.out_f32 ? 4 : 2;
    if (op == FC_OP_FWD) {  // P = X (M x K), Q = W (K x N)
        p.M = M, p.N = N, p.K = K;
        p.a_oc = p_order == FC_COL_MAJOR;
        p.b_oc = q_order == FC_ROW_MAJOR;
        pbytes = M * K * 2, qbytes = K * N * 2, obytes = M * N * esz;
    } else if (op == FC_OP_BWD_DATA) {  // P = dY (M x N, row-major), Q = W (K x N)
        p.M = M, p.N = K, p.K = N;
        p.a_oc = false;
        p.b_oc = q_order == FC_COL_MAJOR;
        pbytes = M * N * 2, qbytes = K * N * 2, obytes = M * K * esz;
    } else {  // P = X (M x K), Q = dY (M x N, row-major)
        p.M = K, p.N = N, p.K = M;
        p.a_oc = p_order == FC_ROW_MAJOR;
        p.b_oc = true;
        pbytes = M * K * 2, qbytes = M * N * 2, obytes = K * N * esz;
    }
    if (P != nullptr || Q != nullptr || out != nullptr) {
        if (!P || !Q || !out) return FC_E_INVALID;
        if ((uintptr_t)P % 2 || (uintptr_t)Q % 2 || (uintptr_t)out % esz) return FC_E_INVALID;
        if (overlaps(out, obytes, P, pbytes) || overlaps(out, obytes, Q, qbytes)) return FC_E_INVALID;
    }
    *pr = p;
    return FC_OK;
}

Key make_key(int dev, int op, int64_t M, int64_t K, int64_t N, int xo, int wo, int dtype) {
    // normalize the orders the product does not read
    if (op == FC_OP_BWD_DATA) xo = 0;
    if (op == FC_OP_BWD_WEIGHT) wo = 0;
    return Key{dev, op, M, K, N, xo, wo, dtype};
}

// Plans whose GEMM has a stamped instance: either ring (three A tiles or
// three B tiles) with 256-column block tiles, one reduction slice, no tail
// split or transpose copy (a padded reduction is fine), bf16 output.
bool stampable(const Problem& p, const Plan& pl) {
    int64_t ks;
    int slices;
    split_geometry(p.K, pl.split, &ks, &slices);
    return (pl.family == kFamilyW4 + 2 || pl.family == kFamilyW4 + 3) && w4_bn(pl) == 256 && !pl.tail &&
           slices == 1 && pl.copy == 0 && !p.out_f32;
}

// A hot call; with `stamps` (measurement aid) the plan must be stampable,
// else FC_E_UNSUPPORTED before anything is enqueued.
fc_status hot_call(int op, const void* P, int p_order, const void* Q, int q_order, void* out, int dtype,
                   int64_t M, int64_t K, int64_t N, void* stream, int xo, int wo,
                   unsigned long long* stamps = nullptr, int64_t stamp_bytes = 0, int64_t* blocks = nullptr) {
    if (!P || !Q || !out) return FC_E_INVALID;
    Problem p;
    fc_status st = resolve(op, P, p_order, Q, q_order, out, dtype, M, K, N, &p);
    if (st != FC_OK) return st;
    int dev;
    Plan pl;
    std::lock_guard<std::mutex> lk(g_mu);  // held until the kernels are enqueued
    if ((st = check_device(&dev)) != FC_OK) return st;
    int id = -1;
    auto it = g_plans.find(make_key(dev, op, M, K, N, xo, wo, dtype));
    if (it != g_plans.end()) id = it->second.id;
    if (id >= 0) {
        pl = decode_plan(id);
        // a plan that no longer applies (alignment) or lacks workspace falls back
        if (!plan_applies(p, pl) || ws_layout(p, pl).total > g_dev[dev].ws_bytes) id = -1;
    }
    if (id < 0) pl = decode_plan(default_plan(p));
    // never launch a plan whose workspace is not there
    const int64_t ws_need = ws_layout(p, pl).total;
    if (ws_need > g_dev[dev].ws_bytes) return FC_E_UNSUPPORTED;
    if (stamps) {
        if (!stampable(p, pl)) return FC_E_UNSUPPORTED;
        const int64_t nb = ((p.M + 255) / 256) * ((p.N + 255) / 256);
        if (stamp_bytes < nb * kStampSlots * 8) return FC_E_INVALID;
        if (blocks) *blocks = nb;
    }
    if (ws_need > 0 && !g_dev[dev].ws_captured) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) == hipSuccess &&
            cs != hipStreamCaptureStatusNone)
            g_dev[dev].ws_captured = true;
    }
    // the launchers report hipGetLastError(): drop an error that an earlier,
    // unrelated HIP call of this thread left behind
    (void)hipGetLastError();
    return run_plan(p, pl, g_dev[dev].ws, static_cast<hipStream_t>(stream), stamps) == hipSuccess ? FC_OK
                                                                                                : FC_E_HIP;
}

// A larger workspace replaces the current one. The old one is freed after a
// device synchronization (enqueued kernels may still use it), unless a hot
// call was captured into a graph while using it: then it is retired and kept
// until fc_release, so that replays of that graph stay valid.
// The address of this device's scratch array, looked up once per device
// with that device current (the caller holds g_mu).
fc_status scratch_of(int dev, void** out) {
    DevState& d = g_dev[dev];
    if (!d.scratch) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return FC_E_HIP;
        }
        d.scratch = ptr;
    }
    *out = d.scratch;
    return FC_OK;
}

fc_status grow_workspace(int dev, int64_t bytes) {
    DevState& d = g_dev[dev];
    if (bytes <= d.ws_bytes) return FC_OK;
    if (d.ws && d.ws_captured) {
        d.retired.push_back(d.ws);
    } else if (d.ws) {
        if (hipDeviceSynchronize() != hipSuccess) return FC_E_HIP;
        (void)hipFree(d.ws);
    }
    d.ws = nullptr;
    d.ws_bytes = 0;
    d.ws_captured = false;
    if (hipMalloc(&d.ws, (size_t)bytes) != hipSuccess) {
        d.ws = nullptr;
        (void)hipGetLastError();
        return FC_E_NOMEM;
    }
    d.ws_bytes = bytes;
    return FC_OK;
}

std::string describe(const Problem& p, int id) {
    const Plan pl = decode_plan(id);
    Problem q = p;
    if ((pl.copy & 1) && q.a_oc) q.a_oc = false, q.A = nullptr;
    if ((pl.copy & 2) && q.b_oc) q.b_oc = false, q.B = nullptr;
    int64_t ks;
    int slices;
    split_geometry(p.K, pl.split, &ks, &slices);
    const bool aligned = q.M % 8 == 0 && q.N % 8 == 0 && q.K % 8 == 0 &&
                         (uintptr_t)p.C % 16 == 0 && (q.A == nullptr || (uintptr_t)q.A % 16 == 0) &&
                         (q.B == nullptr || (uintptr_t)q.B % 16 == 0);
    // a tail plan is named by its main (unsplit) kernel
    const bool f32 = slices > 1 && !pl.tail ? true : p.out_f32;
    const int64_t ks_k = pl.tail ? round_up(p.K, 64) : ks;
    const int slices_k = pl.tail ? 1 : slices;
    const char* kname = pl.family == 0            ? pipe_kernel_name(pl.tile, q.a_oc, q.b_oc, f32)
                        : pl.family >= kFamilyW4  ? w4_kernel_name(pl.family - kFamilyW4, w4_bn(pl), q.a_oc, q.b_oc, f32, p.K, ks_k, slices_k)
                        : pl.family >= 2          ? pingpong_kernel_name(pl.family - 2, q.a_oc, q.b_oc, f32)
                                         : gemm_kernel_name(aligned ? pl.tile : kUnalignedTile, q.a_oc, q.b_oc, f32,
                                                            aligned);
    char buf[512];
    const char* tname = w4_bn(pl) == 192 ? "256x192" : kTiles[aligned ? pl.tile : kUnalignedTile].name;
    const long long pad = pads_reduction(p, pl) ? (long long)round_up(p.K, 64) : 0;
    // the values of a partial last stage that a ring kernel loads itself
    const long long ktail = pl.family >= kFamilyW4 + 2 ? (long long)(p.K % 64) : 0;
    std::snprintf(buf, sizeof buf, "plan=%d kernel=%s tile=%s split=%d copy=%d pad=%lld ktail=%lld ws=%lld", id, kname,
                  tname, slices, pl.copy, pad, ktail, (long long)ws_layout(p, pl).total);
    std::string d = buf;
    if (pl.tail) {  // the unsplit part's extent: tail=n<columns> or tail=m<rows>
        const TailGeo t = tail_geometry(p, w4_bn(pl));
        std::snprintf(buf, sizeof buf, " tail=%c%lld", t.along_n ? 'n' : 'm', (long long)t.main);
        d += buf;
    }
    return d;
}

// ------------------------------------------------------------ plan files

// One line of a plan file: "<arch> <op> <M> <K> <N> <x_order> <w_order>
// <out_dtype> <plan> [<tuned_ms>]", fields separated by blanks.
struct PlanLine {
    char arch[64];
    int op, xo, wo, f32, id;
    long long M, K, N;
    float ms;  // -1 when the line has no time
};

// a decimal integer within [lo, hi] that ends at a blank or the line's end
bool parse_int_field(const char** cur, long long lo, long long hi, long long* out) {
    const char* c = *cur;
    while (*c == ' ' || *c == '\t') ++c;
    char* end = nullptr;
    errno = 0;
    const long long v = std::strtoll(c, &end, 10);
    if (end == c || errno == ERANGE || v < lo || v > hi) return false;
    if (*end != '\0' && *end != ' ' && *end != '\t' && *end != '\n' && *end != '\r') return false;
    *out = v;
    *cur = end;
    return true;
}

// Parses one line of a plan file: 0 on success, 1 for a blank or comment
// line (skipped), -1 for a malformed line. Values are checked for range
// only; whether they name a valid problem and plan is set_plan's decision.
int parse_plan_line(const char* line, PlanLine* out) {
    const char* c = line;
    while (*c == ' ' || *c == '\t') ++c;
    if (*c == '\0' || *c == '\n' || *c == '\r' || *c == '#') return 1;
    size_t n = 0;
    while (c[n] && c[n] != ' ' && c[n] != '\t' && c[n] != '\n' && c[n] != '\r') ++n;
    if (n == 0 || n >= sizeof out->arch) return -1;
    std::memcpy(out->arch, c, n);
    out->arch[n] = '\0';
    c += n;
    long long v[8];
    const long long lim = (long long)1 << 40;
    const long long lo[8] = {-1000, -lim, -lim, -lim, -1000, -1000, -1000, -1000};
    const long long hi[8] = {1000, lim, lim, lim, 1000, 1000, 1000, 100000};
    for (int i = 0; i < 8; ++i)
        if (!parse_int_field(&c, lo[i], hi[i], &v[i])) return -1;
    out->op = (int)v[0], out->M = v[1], out->K = v[2], out->N = v[3];
    out->xo = (int)v[4], out->wo = (int)v[5], out->f32 = (int)v[6], out->id = (int)v[7];
    out->ms = -1.0f;
    while (*c == ' ' || *c == '\t') ++c;
    if (*c != '\0' && *c != '\n' && *c != '\r') {  // the optional time
        char* end = nullptr;
        errno = 0;
        const double ms = std::strtod(c, &end);
        if (end == c || errno == ERANGE || !(ms >= 0.0 && ms < 1e9)) return -1;
        out->ms = (float)ms;
        c = end;
        while (*c == ' ' || *c == '\t') ++c;
        if (*c != '\0' && *c != '\n' && *c != '\r') return -1;
    }
    return 0;
}

// --------------------------------------------------------------- tuning

struct TuneBuffers {
    void* X = nullptr;
    void* W = nullptr;
    void* dY = nullptr;
    void* out = nullptr;
    ~TuneBuffers() {
        if (X) (void)hipFree(X);
        if (W) (void)hipFree(W);
        if (dY) (void)hipFree(dY);
        if (out) (void)hipFree(out);
    }
};

// Two 256 MB buffers; a transpose of one into the other streams 512 MB through
// the L2s and the 256 MB MALL, so the GEMM timed after it reads its operands
// from HBM, as a training step does (each shard GEMM's operands were last
// touched several GEMMs earlier).
struct CacheFlush {
    static constexpr int64_t kRows = 16384, kCols = 8192;  // 2 B each: 256 MB
    uint16_t* a = nullptr;
    uint16_t* b = nullptr;
    bool init(hipStream_t s) {
        if (hipMalloc(&a, kRows * kCols * 2) != hipSuccess || hipMalloc(&b, kRows * kCols * 2) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        return launch_fill_bf16(a, kRows * kCols, 7u, s) == hipSuccess;
    }
    hipError_t run(hipStream_t s) const { return launch_transpose_bf16(a, b, kRows, kCols, s); }
    ~CacheFlush() {
        if (a) (void)hipFree(a);
        if (b) (void)hipFree(b);
    }
};

// Median of `reps` single-launch times after `warm` untimed launches; with
// `flush`, the caches are flushed before every timed launch.
float time_plan(const Problem& p, const Plan& pl, void* ws, hipStream_t s, int warm, int reps, hipEvent_t* ev,
                const CacheFlush* flush, bool* ok, std::vector<float>* samples = nullptr) {
    *ok = true;
    for (int i = 0; i < warm; ++i)
        if (run_plan(p, pl, ws, s) != hipSuccess) *ok = false;
    std::vector<float> t;
    for (int i = 0; i < reps && *ok; ++i) {
        if (flush && flush->run(s) != hipSuccess) *ok = false;
        if (hipEventRecord(ev[0], s) != hipSuccess) *ok = false;
        if (run_plan(p, pl, ws, s) != hipSuccess) *ok = false;
        if (hipEventRecord(ev[1], s) != hipSuccess) *ok = false;
        if (hipEventSynchronize(ev[1]) != hipSuccess) *ok = false;
        float ms = 0;
        if (hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) *ok = false;
        t.push_back(ms);
    }
    if (!*ok || t.empty()) return 1e30f;
    if (samples) samples->insert(samples->end(), t.begin(), t.end());
    std::sort(t.begin(), t.end());
    return t[t.size() / 2];
}

float median_of(std::vector<float> v) {
    std::sort(v.begin(), v.end());
    return v[v.size() / 2];
}

}  // namespace
}  // namespace fcs

using namespace fcs;

extern "C" {

fc_status fc_fwd(const void* X, fc_order x_order, const void* W, fc_order w_order, void* Y, fc_out_dtype y_dtype,
                 int64_t M, int64_t K, int64_t N, void* stream) {
    return hot_call(FC_OP_FWD, X, x_order, W, w_order, Y, y_dtype, M, K, N, stream, x_order, w_order);
}

fc_status fc_bwd_data(const void* dY, const void* W, fc_order w_order, void* dX, fc_out_dtype dx_dtype, int64_t M,
                      int64_t K, int64_t N, void* stream) {
    return hot_call(FC_OP_BWD_DATA, dY, FC_ROW_MAJOR, W, w_order, dX, dx_dtype, M, K, N, stream, FC_ROW_MAJOR,
                    w_order);
}

fc_status fc_bwd_weight(const void* X, fc_order x_order, const void* dY, void* dW, fc_out_dtype dw_dtype,
                        int64_t M, int64_t K, int64_t N, void* stream) {
    return hot_call(FC_OP_BWD_WEIGHT, X, x_order, dY, FC_ROW_MAJOR, dW, dw_dtype, M, K, N, stream, x_order,
                    FC_ROW_MAJOR);
}

fc_status fc_bwd_weight_noalloc(const void* X, fc_order x_order, const void* dY, void* dW, fc_out_dtype dw_dtype,
                                int64_t M, int64_t K, int64_t N, void* stream) {
    if (!X || !dY || !dW) return FC_E_INVALID;
    Problem p;
    fc_status st = resolve(FC_OP_BWD_WEIGHT, X, x_order, dY, FC_ROW_MAJOR, dW, dw_dtype, M, K, N, &p);
    if (st != FC_OK) return st;
    std::lock_guard<std::mutex> lk(g_mu);  // held until the kernels are enqueued
    int dev;
    if ((st = check_device(&dev)) != FC_OK) return st;
    void* scr = nullptr;
    if ((st = scratch_of(dev, &scr)) != FC_OK) return st;
    // the plan fc_bwd_weight would pick at this key, the scratch standing in
    // for the workspace
    Plan pl = decode_plan(default_plan(p));
    auto it = g_plans.find(make_key(dev, FC_OP_BWD_WEIGHT, M, K, N, x_order, FC_ROW_MAJOR, dw_dtype));
    if (it != g_plans.end() && plan_applies(p, decode_plan(it->second.id))) pl = decode_plan(it->second.id);
    if (ws_layout(p, pl).total > kNoallocScratchBytes) return FC_E_TOO_LARGE;
    (void)hipGetLastError();
    return run_plan(p, pl, scr, static_cast<hipStream_t>(stream)) == hipSuccess ? FC_OK : FC_E_HIP;
}

int64_t fc_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

fc_status fc_stamped_call(fc_op op, const void* P, fc_order p_order, const void* Q, fc_order q_order, void* out,
                          fc_out_dtype out_dtype, int64_t M, int64_t K, int64_t N, void* stamps,
                          int64_t stamp_bytes, int64_t* blocks, void* stream) {
    if (!stamps || !blocks || (uintptr_t)stamps % 8 || stamp_bytes < 0) return FC_E_INVALID;
    if (op != FC_OP_FWD && op != FC_OP_BWD_DATA && op != FC_OP_BWD_WEIGHT) return FC_E_INVALID;
    // the orders the product does not read are taken as row-major, as in the hot calls
    const int po = op == FC_OP_BWD_DATA ? FC_ROW_MAJOR : p_order;
    const int qo = op == FC_OP_BWD_WEIGHT ? FC_ROW_MAJOR : q_order;
    const int xo = op == FC_OP_BWD_DATA ? FC_ROW_MAJOR : p_order;
    const int wo = op == FC_OP_BWD_WEIGHT ? FC_ROW_MAJOR : q_order;
    *blocks = 0;
    return hot_call(op, P, po, Q, qo, out, out_dtype, M, K, N, stream, xo, wo,
                    static_cast<unsigned long long*>(stamps), stamp_bytes, blocks);
}

int fc_plan_count(void) { return kNumPlans; }

// fc_set_plan with g_ws_mu already held by the caller
static fc_status set_plan(fc_op op, int64_t M, int64_t K, int64_t N, fc_order x_order, fc_order w_order,
                          fc_out_dtype out_dtype, int plan_id) {
    if (bad_order(x_order) || bad_order(w_order) || bad_dtype(out_dtype)) return FC_E_INVALID;
    if (plan_id < -1 || plan_id >= kNumPlans) return FC_E_INVALID;
    int p_order = op == FC_OP_BWD_DATA ? FC_ROW_MAJOR : x_order;
    int q_order = op == FC_OP_BWD_WEIGHT ? FC_ROW_MAJOR : w_order;
    Problem p;
    fc_status st = resolve(op, nullptr, p_order, nullptr, q_order, nullptr, out_dtype, M, K, N, &p);
    if (st != FC_OK) return st;
    std::lock_guard<std::mutex> lk(g_mu);
    int dev;
    if ((st = check_device(&dev)) != FC_OK) return st;
    const Key key = make_key(dev, op, M, K, N, x_order, w_order, out_dtype);
    if (plan_id < 0) {
        g_plans.erase(key);
        return FC_OK;
    }
    // alignment of pointers is not known here: judge the shape only
    p.A = p.B = nullptr;
    p.C = nullptr;
    const Plan pl = decode_plan(plan_id);
    if (!plan_applies(p, pl)) return FC_E_UNSUPPORTED;
    if ((st = grow_workspace(dev, ws_layout(p, pl).total)) != FC_OK) return st;
    g_plans[key] = PlanEntry{plan_id, -1.0f};
    return FC_OK;
}

fc_status fc_set_plan(fc_op op, int64_t M, int64_t K, int64_t N, fc_order x_order, fc_order w_order,
                      fc_out_dtype out_dtype, int plan_id) {
    std::lock_guard<std::mutex> wl(g_ws_mu);
    return set_plan(op, M, K, N, x_order, w_order, out_dtype, plan_id);
}

fc_status fc_plan_describe(fc_op op, int64_t M, int64_t K, int64_t N, fc_order x_order, fc_order w_order,
                           fc_out_dtype out_dtype, char* buf, size_t len) {
    if (!buf || len == 0) return FC_E_INVALID;
    if (bad_order(x_order) || bad_order(w_order) || bad_dtype(out_dtype)) return FC_E_INVALID;
    int p_order = op == FC_OP_BWD_DATA ? FC_ROW_MAJOR : x_order;
    int q_order = op == FC_OP_BWD_WEIGHT ? FC_ROW_MAJOR : w_order;
    Problem p;
    fc_status st = resolve(op, nullptr, p_order, nullptr, q_order, nullptr, out_dtype, M, K, N, &p);
    if (st != FC_OK) return st;
    std::lock_guard<std::mutex> lk(g_mu);
    int dev;
    if ((st = check_device(&dev)) != FC_OK) return st;
    p.A = p.B = nullptr;
    p.C = nullptr;
    int id = -1;
    float ms = -1.0f;
    auto it = g_plans.find(make_key(dev, op, M, K, N, x_order, w_order, out_dtype));
    if (it != g_plans.end()) id = it->second.id, ms = it->second.ms;
    if (id >= 0 && ws_layout(p, decode_plan(id)).total > g_dev[dev].ws_bytes) id = -1, ms = -1.0f;
    if (id < 0) id = default_plan(p);
    std::string s = describe(p, id);
    if (ms >= 0.0f) {
        char t[48];
        std::snprintf(t, sizeof t, " tuned_ms=%.6f", ms);
        s += t;
    }
    std::snprintf(buf, len, "%s", s.c_str());
    return FC_OK;
}

fc_status fc_tune(int64_t M, int64_t K, int64_t N, fc_order x_order, fc_order w_order, fc_out_dtype out_dtype,
                  int flags, void* stream) {
    if (bad_order(x_order) || bad_order(w_order) || bad_dtype(out_dtype)) return FC_E_INVALID;
    if (M < 1 || K < 1 || N < 1) return FC_E_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> wl(g_ws_mu);  // no growth or release while timing on the workspace
    int dev;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        fc_status st = check_device(&dev);
        if (st != FC_OK) return st;
    }
    (void)hipGetLastError();  // as in hot_call: no stale error from an earlier HIP call
    TuneBuffers b;
    const int64_t esz = out_dtype == FC_OUT_BF16 ? 2 : 4;
    const int64_t out_elems = std::max(M * N, std::max(M * K, K * N));
    if (hipMalloc(&b.X, M * K * 2) != hipSuccess || hipMalloc(&b.W, K * N * 2) != hipSuccess ||
        hipMalloc(&b.dY, M * N * 2) != hipSuccess || hipMalloc(&b.out, out_elems * esz) != hipSuccess) {
        (void)hipGetLastError();
        return FC_E_NOMEM;
    }
    hipError_t fe = launch_fill_bf16((uint16_t*)b.X, M * K, 1u, s);
    if (fe == hipSuccess) fe = launch_fill_bf16((uint16_t*)b.W, K * N, 2u, s);
    if (fe == hipSuccess) fe = launch_fill_bf16((uint16_t*)b.dY, M * N, 3u, s);
    // an accumulating output starts from zeros (the timed calls add into it)
    if (fe == hipSuccess && out_dtype == FC_OUT_F32_ACCUMULATE) fe = hipMemsetAsync(b.out, 0, out_elems * esz, s);
    if (fe != hipSuccess) {
        if (log_enabled()) std::fprintf(stderr, "[fcshard] tune: filling the operands failed: %s\n", hipGetErrorString(fe));
        return FC_E_HIP;
    }
    hipEvent_t ev[2];
    if (hipEventCreate(&ev[0]) != hipSuccess) return FC_E_HIP;
    if (hipEventCreate(&ev[1]) != hipSuccess) {
        (void)hipEventDestroy(ev[0]);
        return FC_E_HIP;
    }
    const bool exhaustive = (flags & 1) != 0;
    const int warm = exhaustive ? 3 : 2, reps = exhaustive ? 10 : 5;
    CacheFlush flush_bufs;
    const CacheFlush* flush = nullptr;
    if (!(flags & 2)) {
        if (flush_bufs.init(s))
            flush = &flush_bufs;
        else if (log_enabled())
            std::fprintf(stderr, "[fcshard] tune: no memory for the cache flush; timing with warm caches\n");
    }
    fc_status result = FC_OK;

    for (int op = 0; op < 3; ++op) {
        const void* P = op == FC_OP_BWD_DATA ? b.dY : b.X;
        const void* Q = op == FC_OP_FWD ? b.W : (op == FC_OP_BWD_DATA ? b.W : b.dY);
        const int p_order = op == FC_OP_BWD_DATA ? FC_ROW_MAJOR : x_order;
        const int q_order = op == FC_OP_BWD_WEIGHT ? FC_ROW_MAJOR : w_order;
        Problem p;
        fc_status st = resolve(op, P, p_order, Q, q_order, b.out, out_dtype, M, K, N, &p);
        if (st != FC_OK) {
            result = st;
            break;
        }
        // candidate plans
        std::vector<int> cand;
        int64_t need = 0;
        for (int pass = 0; pass < 2 && cand.empty(); ++pass) {
            for (int id = 0; id < kNumPlans; ++id) {
                const Plan pl = decode_plan(id);
                if (!plan_applies(p, pl)) continue;
                if (!exhaustive && pl.split > 1 && pl.copy != 0) continue;
                // the simple kernels only win on unaligned shapes, or where no
                // other family applies (an operand of 2 GiB or more): second pass
                if (!exhaustive && pass == 0 && pl.family == 1 && problem_aligned(p)) continue;
                cand.push_back(id);
                need = std::max(need, ws_layout(p, pl).total);
            }
        }
        {
            std::lock_guard<std::mutex> lk(g_mu);
            if (grow_workspace(dev, need) != FC_OK) {
                // keep only the plans that fit what is there
                std::vector<int> keep;
                for (int id : cand)
                    if (ws_layout(p, decode_plan(id)).total <= g_dev[dev].ws_bytes) keep.push_back(id);
                cand.swap(keep);
            }
        }
        void* ws = g_dev[dev].ws;
        int best = -1;
        float best_ms = 1e30f;
        std::vector<std::pair<int, float>> times;
        std::vector<std::vector<float>> samples;  // per entry of times
        for (int id : cand) {
            bool ok;
            std::vector<float> t;
            const float ms = time_plan(p, decode_plan(id), ws, s, warm, reps, ev, flush, &ok, &t);
            if (!ok) {
                (void)hipGetLastError();
                continue;
            }
            times.push_back({id, ms});
            samples.push_back(t);
            if (ms < best_ms) best_ms = ms, best = id;
        }
        // The close candidates (within 3 % of the best, at most four) are timed
        // again in interleaved rounds and each keeps the median of all its
        // samples: five timed launches leave 2-4 % of noise, enough to flip a
        // pick, and the rounds spread any drift of the clock over all of them.
        {
            std::vector<size_t> close;
            for (size_t c = 0; c < times.size(); ++c)
                if (times[c].second <= best_ms * 1.03f) close.push_back(c);
            std::sort(close.begin(), close.end(),
                      [&](size_t a, size_t b) { return times[a].second < times[b].second; });
            if (close.size() > 4) close.resize(4);
            if (close.size() > 1) {
                constexpr int kRounds = 4, kRoundReps = 3;
                for (int r = 0; r < kRounds; ++r)
                    for (size_t c : close) {
                        bool ok;
                        time_plan(p, decode_plan(times[c].first), ws, s, 1, kRoundReps, ev, flush, &ok, &samples[c]);
                        if (!ok) (void)hipGetLastError();
                    }
                best_ms = 1e30f;
                for (size_t c = 0; c < times.size(); ++c) {
                    if (std::find(close.begin(), close.end(), c) != close.end())
                        times[c].second = median_of(samples[c]);
                    if (times[c].second < best_ms) best_ms = times[c].second, best = times[c].first;
                }
            }
        }
        // tie-break within 1%: no workspace, then no split, then the lower id
        int pick = best;
        for (auto& t : times) {
            if (t.second > best_ms * 1.01f) continue;
            const Plan a = decode_plan(t.first), c = decode_plan(pick);
            const int64_t wa = ws_layout(p, a).total, wc = ws_layout(p, c).total;
            const auto ka = std::make_tuple(wa > 0, a.split > 1, t.first);
            const auto kc = std::make_tuple(wc > 0, c.split > 1, pick);
            if (ka < kc) pick = t.first;
        }
        if (log_enabled()) {
            for (auto& t : times)
                std::fprintf(stderr, "[fcshard] tune op=%d M=%lld K=%lld N=%lld %s: %.4f ms\n", op, (long long)M,
                             (long long)K, (long long)N, describe(p, t.first).c_str(), t.second);
            std::fprintf(stderr, "[fcshard] tune op=%d pick %s\n", op, pick >= 0 ? describe(p, pick).c_str() : "none");
        }
        if (pick >= 0) {
            float pick_ms = -1.0f;
            for (auto& t : times)
                if (t.first == pick) pick_ms = t.second;
            std::lock_guard<std::mutex> lk(g_mu);
            g_plans[make_key(dev, op, M, K, N, x_order, w_order, out_dtype)] = PlanEntry{pick, pick_ms};
        }
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (hipStreamSynchronize(s) != hipSuccess) result = FC_E_HIP;
    return result;
}

fc_status fc_plans_save(const char* path) {
    if (!path) return FC_E_INVALID;
    std::lock_guard<std::mutex> lk(g_mu);
    int dev;
    fc_status st = check_device(&dev);
    if (st != FC_OK) return st;
    FILE* f = std::fopen(path, "w");
    if (!f) return FC_E_INVALID;
    for (const auto& kv : g_plans) {
        const Key& k = kv.first;
        if (k.dev != dev) continue;
        std::fprintf(f, "%s %d %lld %lld %lld %d %d %d %d", g_dev[dev].arch, k.op, (long long)k.M, (long long)k.K,
                     (long long)k.N, k.xo, k.wo, k.f32, kv.second.id);
        if (kv.second.ms >= 0.0f) std::fprintf(f, " %.6f", kv.second.ms);
        std::fputc('\n', f);
    }
    return std::fclose(f) == 0 ? FC_OK : FC_E_INVALID;
}

fc_status fc_plans_load(const char* path) {
    if (!path) return FC_E_INVALID;
    std::lock_guard<std::mutex> wl(g_ws_mu);
    int dev;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        fc_status st = check_device(&dev);
        if (st != FC_OK) return st;
    }
    FILE* f = std::fopen(path, "r");
    if (!f) return FC_E_INVALID;
    char line[512];
    fc_status result = FC_OK;
    while (std::fgets(line, sizeof line, f)) {
        // a line longer than the buffer is malformed (no plan line comes near it)
        if (!std::strchr(line, '\n') && !std::feof(f)) {
            result = FC_E_INVALID;
            break;
        }
        PlanLine pl;
        const int r = parse_plan_line(line, &pl);
        if (r == 1) continue;
        if (r != 0) {
            result = FC_E_INVALID;
            break;
        }
        if (std::strcmp(pl.arch, g_dev[dev].arch) != 0) continue;
        fc_status st = set_plan((fc_op)pl.op, pl.M, pl.K, pl.N, (fc_order)pl.xo, (fc_order)pl.wo,
                                (fc_out_dtype)pl.f32, pl.id);
        if (st != FC_OK) {
            result = st;
            break;
        }
        if (pl.ms >= 0.0f && pl.id >= 0) {
            std::lock_guard<std::mutex> lk(g_mu);
            auto it = g_plans.find(make_key(dev, (fc_op)pl.op, pl.M, pl.K, pl.N, pl.xo, pl.wo, pl.f32));
            if (it != g_plans.end()) it->second.ms = pl.ms;
        }
    }
    std::fclose(f);
    return result;
}

const char* fc_status_str(fc_status status) {
    switch (status) {
        case FC_OK: return "FC_OK: success";
        case FC_E_INVALID: return "FC_E_INVALID: invalid argument (NULL, dimension < 1, bad enum, misaligned or overlapping)";
        case FC_E_UNSUPPORTED: return "FC_E_UNSUPPORTED: device is not gfx950 or plan does not apply";
        case FC_E_HIP: return "FC_E_HIP: HIP runtime or launch error";
        case FC_E_NOMEM: return "FC_E_NOMEM: device allocation failed";
        case FC_E_TOO_LARGE:
            return "FC_E_TOO_LARGE: the plan needs more scratch than the no-allocation entry point's static "
                   "device buffer holds (fc_noalloc_scratch_bytes)";
    }
    return "unknown fc_status";
}

fc_status fc_release(void) {
    std::lock_guard<std::mutex> wl(g_ws_mu);
    std::lock_guard<std::mutex> lk(g_mu);
    g_plans.clear();
    fc_status st = FC_OK;
    for (int d = 0; d < kMaxDevices; ++d) {
        if (g_dev[d].ws || !g_dev[d].retired.empty()) {
            int cur = 0;
            if (hipGetDevice(&cur) != hipSuccess) return FC_E_HIP;
            if (hipSetDevice(d) != hipSuccess || hipDeviceSynchronize() != hipSuccess) st = FC_E_HIP;
            if (g_dev[d].ws) (void)hipFree(g_dev[d].ws);
            for (void* r : g_dev[d].retired) (void)hipFree(r);
            g_dev[d].retired.clear();
            g_dev[d].ws = nullptr;
            g_dev[d].ws_bytes = 0;
            g_dev[d].ws_captured = false;
            (void)hipSetDevice(cur);
        }
    }
    return st;
}

}  // extern "C"
