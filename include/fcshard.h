/*
 * fcshard.h - C ABI of the per-GPU shard GEMMs of a 3D-parallel FC layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation. One fully connected layer's matrix multiply is split over a
 * Gx x Gy x Gz virtual grid of GPUs with Agarwal's 3D parallel matrix
 * multiplication (sciencestack.ai/paper/2502.08145, Figure 1). After the
 * collectives that move shards around (pith.science/paper/2502.08145, "What
 * carries the argument": weight sharded along Z, all-gather, reduce-scatter,
 * all-reduce), each GPU runs three local bf16 matrix products on its shard:
 *
 *   forward          Y  = X . W      X: M x K, W: K x N, Y: M x N
 *   backward-data    dX = dY . W^T   dY: M x N, dX: M x K
 *   backward-weight  dW = X^T . dY   dW: K x N (the local, un-reduced block)
 *
 * M counts tokens of the shard, K input features, N output features. Inputs
 * are bf16 (mlsanity.com/paper/2502.08145, Abstract: bf16 training); products
 * are accumulated in fp32 and the output is rounded to bf16 (nearest-even) or
 * stored as fp32. Automated kernel tuning is one of the pages' named
 * optimisations (sciencestack.ai/paper/2502.08145, TL;DR); fc_tune is this
 * library's per-shape version of it.
 *
 * Layout. Every matrix is tightly packed (leading dimension = its column
 * count in its storage order). X and W take a storage order; dY, Y, dX and dW
 * are always row-major. A PyTorch nn.Linear weight (N x K, row-major) is W in
 * FC_COL_MAJOR.
 *
 * Ownership. All data pointers are DEVICE pointers owned by the caller. The
 * library owns only its plan cache and one workspace per device, which grow
 * only inside fc_tune / fc_set_plan / fc_plans_load and are freed by
 * fc_release.
 *
 * Hot calls (fc_fwd, fc_bwd_data, fc_bwd_weight) never allocate and never
 * synchronize: they validate, enqueue kernels on `stream` (a hipStream_t;
 * NULL is the null stream) and return. A shape that was never tuned runs a
 * default plan that needs no workspace; a hot call never launches a plan
 * whose workspace is missing. Errors are returned, never thrown; the library
 * never aborts. Device faults surface at the caller's next synchronization,
 * as for any asynchronous HIP call.
 *
 * Graph capture. Hot calls may be captured into a HIP graph (they launch
 * kernels only). A captured call that uses the workspace keeps its address:
 * a later growth then retires that workspace instead of freeing it, so the
 * graph stays valid until fc_release, which frees every workspace and so
 * invalidates such graphs.
 *
 * Threading: the plan cache is guarded by a mutex; hot calls may come from
 * several host threads. A workspace grows or is freed only while no other
 * thread is enqueuing a hot call, and is freed only after a device
 * synchronization, so no enqueued kernel loses its workspace. Streams: plans with split-K, a
 * transpose copy or a padded reduction (fc_plan_describe: ws > 0) stage data
 * in the device's one workspace, and so does fc_tune while it times them;
 * two such calls that can run at the same time on different streams race
 * on its contents. Order them (one stream, or events), or use plans without
 * workspace (fc_set_plan). Calls on one stream never race.
 * Determinism: the same plan on the same inputs gives bitwise-identical
 * output (split-K partials are summed in a fixed order, no atomics).
 */
#ifndef FCSHARD_H
#define FCSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * In C++ the enums below have int as their fixed underlying type, so that
 * every int a C caller passes is a value of the type and the library can
 * refuse the ones it does not know without undefined behaviour. In C they
 * are plain enums, also of int size.
 */
#ifdef __cplusplus
#define FC_INT_ENUM enum : int
#else
#define FC_INT_ENUM enum
#endif

typedef FC_INT_ENUM {
    FC_OK = 0,
    FC_E_INVALID = 1,     /* NULL pointer, dimension < 1, bad enum, misaligned or overlapping output */
    FC_E_UNSUPPORTED = 2, /* current device is not gfx950, or plan id not applicable */
    FC_E_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    FC_E_NOMEM = 4,       /* workspace or tuning buffers could not be allocated */
    FC_E_TOO_LARGE = 5    /* fc_bwd_weight_noalloc: the plan needs more than its static scratch */
} fc_status;

/* storage order of a LOGICAL matrix */
typedef FC_INT_ENUM { FC_ROW_MAJOR = 0, FC_COL_MAJOR = 1 } fc_order;

/*
 * output element type. FC_OUT_F32_ACCUMULATE: the output is fp32 and already
 * holds values; the product is added to them (C = C + product, one fp32 add
 * per element after the product's own fp32 sum), e.g. to accumulate dW over
 * micro-batches. The output must then be initialised by the caller.
 */
typedef FC_INT_ENUM { FC_OUT_BF16 = 0, FC_OUT_F32 = 1, FC_OUT_F32_ACCUMULATE = 2 } fc_out_dtype;

/* the three products, for the plan-control calls */
typedef FC_INT_ENUM { FC_OP_FWD = 0, FC_OP_BWD_DATA = 1, FC_OP_BWD_WEIGHT = 2 } fc_op;

/*
 * Y[M x N] = X[M x K] . W[K x N]   (forward; reduction over K).
 * X: bf16, x_order; W: bf16, w_order; Y: row-major, y_dtype.
 * Y must not overlap X or W. Base pointers need 2-byte (bf16) or 4-byte
 * (fp32) alignment; 16-byte-aligned bases with M, K, N multiples of 8 take
 * the vectorized kernels.
 */
fc_status fc_fwd(const void* X, fc_order x_order, const void* W, fc_order w_order,
                 void* Y, fc_out_dtype y_dtype, int64_t M, int64_t K, int64_t N, void* stream);

/*
 * dX[M x K] = dY[M x N] . W[K x N]^T   (backward-data; reduction over N).
 * dY: bf16 row-major; W: bf16, w_order; dX: row-major, dx_dtype.
 */
fc_status fc_bwd_data(const void* dY, const void* W, fc_order w_order,
                      void* dX, fc_out_dtype dx_dtype, int64_t M, int64_t K, int64_t N, void* stream);

/*
 * dW[K x N] = X[M x K]^T . dY[M x N]   (backward-weight; reduction over the
 * M tokens). X: bf16, x_order; dY: bf16 row-major; dW: row-major, dw_dtype.
 * dW is this GPU's local block; in the full method it would then be
 * reduce-scattered over Gz.
 */
fc_status fc_bwd_weight(const void* X, fc_order x_order, const void* dY,
                        void* dW, fc_out_dtype dw_dtype, int64_t M, int64_t K, int64_t N, void* stream);

/*
 * dW = X^T . dY exactly as fc_bwd_weight (same arguments, same plan, same
 * bits), for callers that cannot allocate or own no workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It calls no allocating routine: a plan's split-K partial planes, copies or
 * padded operands go to a static device array of fc_noalloc_scratch_bytes()
 * bytes (64 MiB) that each device holds from the library's load to the end
 * of the process, instead of the library's workspace. The plan is the one
 * fc_bwd_weight would take at this key (tuned, or forced by fc_set_plan,
 * else the default, which needs no scratch); FC_E_TOO_LARGE if it needs
 * more scratch than the array holds (e.g. a 4-way split of a dW over 16 Mi
 * elements). Every call on a device shares that device's array, which keeps
 * the last call's contents (nothing a plan reads there is left from an
 * earlier call): calls that can overlap on one device (streams not ordered
 * by the caller) race on it.
 */
fc_status fc_bwd_weight_noalloc(const void* X, fc_order x_order, const void* dY, void* dW,
                                fc_out_dtype dw_dtype, int64_t M, int64_t K, int64_t N, void* stream);

/* size in bytes of fc_bwd_weight_noalloc's static device scratch */
int64_t fc_noalloc_scratch_bytes(void);

/*
 * Times candidate plans of all three products at (M, K, N, x_order, w_order,
 * out_dtype) on `stream` and caches the fastest per product. flags bit 0:
 * exhaustive search (else quick); bit 1: time with warm caches. By default
 * every timed launch follows a 512 MB copy that evicts the L2s and the MALL,
 * so plans are ranked on operands read from HBM, as in a training step
 * (warm caches are used if those buffers cannot be allocated). Candidates
 * within 3 % of the fastest (at most four) are timed again in interleaved
 * rounds before the pick. Allocates temporary buffers and may grow the
 * workspace; synchronizes `stream`. Plans are kept until fc_release.
 */
fc_status fc_tune(int64_t M, int64_t K, int64_t N, fc_order x_order, fc_order w_order,
                  fc_out_dtype out_dtype, int flags, void* stream);

/* number of plan ids (plan ids are 0 .. fc_plan_count()-1) */
int fc_plan_count(void);

/*
 * Forces plan `plan_id` for one product at one key, as if tuned (grows the
 * workspace if the plan needs one). FC_E_UNSUPPORTED if the plan does not
 * apply to this shape (e.g. a vectorized tile on an unaligned shape).
 * plan_id = -1 removes the cache entry (back to the default plan).
 */
fc_status fc_set_plan(fc_op op, int64_t M, int64_t K, int64_t N, fc_order x_order, fc_order w_order,
                      fc_out_dtype out_dtype, int plan_id);

/*
 * Describes the plan a hot call at this key would run: writes a NUL-terminated
 * text "plan=<id> kernel=<name> tile=<BMxBN> split=<s> copy=<mask> pad=<k>
 * ktail=<t> ws=<bytes>" into buf (truncated to len); copy has bit 0 for the
 * first operand (X or dY) and bit 1 for the second (W or dY), each a copy in
 * the workspace: transposed if the operand is output-contiguous, else (ring
 * kernels, a reduction that is not a multiple of 64) with rows padded to
 * whole 64-value stages; pad is the length the reduction is zero-padded to
 * (reduction-contiguous operands copied into the workspace), 0 for none;
 * ktail is, for the ring kernels, the number of
 * reduction values past the last whole 64-value stage (the partial stage they
 * load themselves), else 0. A tail-split plan adds " tail=n<cols>" or
 * " tail=m<rows>", the extent of its unsplit part. The text is followed by
 * " tuned_ms=<t>" when fc_tune chose
 * the plan (or a loaded plan file recorded its time): the median time of one
 * launch, in ms, as fc_tune measured it. Returns FC_E_INVALID for bad
 * arguments.
 */
fc_status fc_plan_describe(fc_op op, int64_t M, int64_t K, int64_t N, fc_order x_order,
                           fc_order w_order, fc_out_dtype out_dtype, char* buf, size_t len);

/*
 * Writes every cached plan of the current device to a text file, one line
 * "<arch> <op> <M> <K> <N> <x_order> <w_order> <out_dtype> <plan_id>", plus
 * " <ms>" (fc_tune's measured time) for plans that fc_tune chose.
 * FC_E_INVALID if path is NULL or the file cannot be written.
 */
fc_status fc_plans_save(const char* path);

/*
 * Reads such a file (the time field is optional) and caches, for the current
 * device, every line whose arch matches it, with its time if the line has
 * one (growing the workspace as the plans need). Lines for other
 * archs, blank lines and lines starting with '#' are skipped. FC_E_INVALID if
 * the file cannot be read or a line is malformed: fields missing or extra,
 * a number that is not a plain decimal or is out of range, a time that is
 * not a non-negative number, or a line of 512 characters or more (entries
 * before it stay loaded).
 */
fc_status fc_plans_load(const char* path);

/*
 * Measurement aid, not part of the path: the empirical MFMA peak. The pages
 * quote efficiency against an empirically measured peak
 * (pith.science/paper/2502.08145, "Assumptions & free parameters"); this is
 * the one of this chip for the GEMM kernels' instruction stream. One block of
 * 4 waves per compute unit issues `iters` rounds of 64
 * v_mfma_f32_16x16x32_bf16 per wave into 256 AGPR accumulators (the 128 x 128
 * wave tile of the GEMMs), with no loads, LDS accesses or barriers. The
 * result: the launch time (HIP events on `stream`), the bf16 flops issued,
 * the compute-unit count, and the mean over blocks of the shader-clock
 * counter's ticks per tick of the constant-rate counter (s_memtime over
 * s_memrealtime; times wall_clock_mhz it is the engine clock in MHz when the
 * first counter runs at the engine clock). Allocates and frees small
 * buffers and synchronizes `stream`. FC_E_INVALID for a NULL result or iters
 * outside 1 .. 2^40.
 */
typedef struct {
    double ms;             /* kernel time */
    double flops;          /* 2 x 16 x 16 x 32 per MFMA, every MFMA of the launch */
    int compute_units;     /* blocks launched, one per compute unit */
    double counter_ratio;  /* shader-clock counter ticks per constant-rate tick */
    double wall_clock_mhz; /* rate of the constant-rate counter */
} fc_mfma_probe_result;

fc_status fc_mfma_probe(int64_t iters, fc_mfma_probe_result* out, void* stream);

/*
 * The same kernel, enqueued on `stream` without waiting: `blocks` blocks (0:
 * one per compute unit), `iters` rounds. Block b writes four uint64 values
 * to clocks[4 b .. 4 b + 3] (device memory owned by the caller, 8-byte
 * aligned, 4 x blocks values): the shader-clock counter at the start and end
 * of its loop, then the constant-rate counter at the same two points. A
 * short launch after a GEMM samples the engine clock the GEMM left the chip
 * at. FC_E_INVALID for a NULL or misaligned buffer or arguments out of range.
 */
fc_status fc_mfma_probe_launch(int64_t iters, int blocks, void* clocks, void* stream);

/*
 * Measurement aid: one product with cycle stamps. It runs `op` as the
 * matching hot call would, with the same plan, the same result and the same
 * instruction stream in the main loop. The ring kernel writes 8 uint64
 * values per block to `stamps`, which is device memory owned by the caller,
 * 8-byte aligned, and at least 64 x blocks bytes (stamp_bytes).
 *
 * The values of block b, at stamps[8 b .. 8 b + 7]:
 *   0  shader-clock counter (s_memtime) at entry
 *   1  constant-rate counter (s_memrealtime, wall_clock_mhz) at entry
 *   2  shader-clock counter before the first loads
 *   3  shader-clock counter once the first reduction stage has landed (the
 *      second, issued with it, may still be in flight)
 *   4  shader-clock counter after the last MFMA
 *   5  shader-clock counter at exit, after the output is stored
 *   6  constant-rate counter at exit
 *   7  the reduction stages (64 values each) the block ran
 * From these the caller derives the engine clock during the kernel, the
 * cycles per stage of its main loop, and its prologue and epilogue.
 *
 * Arguments are those of the hot call of `op`:
 *   FC_OP_FWD         P = X (p_order), Q = W (q_order)
 *   FC_OP_BWD_DATA    P = dY, Q = W (q_order); p_order is not read
 *   FC_OP_BWD_WEIGHT  P = X (p_order), Q = dY; q_order is not read
 * *blocks receives the number of blocks.
 *
 * Only plans whose product is one ring-kernel launch have a stamped form:
 * family 8 or 9, 256-column tiles, one reduction slice, no tail split, no
 * operand copy (transposed or padded), bf16 output. A reduction that is not a
 * multiple of 64 is allowed (the ring loads its partial stage). Any other plan
 * returns FC_E_UNSUPPORTED, and nothing is enqueued.
 * FC_E_INVALID: a NULL, misaligned or too small stamps buffer, or arguments
 * the hot call would refuse.
 */
fc_status fc_stamped_call(fc_op op, const void* P, fc_order p_order, const void* Q, fc_order q_order, void* out,
                          fc_out_dtype out_dtype, int64_t M, int64_t K, int64_t N, void* stamps,
                          int64_t stamp_bytes, int64_t* blocks, void* stream);

/* static text for a status; never NULL */
const char* fc_status_str(fc_status status);

/* frees the library-owned workspaces and clears the plan cache */
fc_status fc_release(void);

#ifdef __cplusplus
}
#endif

#endif /* FCSHARD_H */
