// Host sanitizer run of the C-ABI layer (sharded_fc_layer_amd/csrc/
// fcshard_api.hip), whose source this file includes so that its internal
// host logic can be driven directly. tests/test_sanitize_cpu.py builds it
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only
// (the device code is not instrumented) and links the library's other
// objects; it runs on a machine without a GPU.
//
// Driven here: argument resolution at the size limits, the whole plan space
// (decode, applicability, workspace layout, tail geometry, descriptions,
// default plans) over a table of problems, the pointer-overlap test, the
// plan-file line parser on valid, malformed and random lines, the status
// strings, and every entry point's refusal of malformed arguments.
#include "../../sharded_fc_layer_amd/csrc/fcshard_api.hip"

#include <cstdio>
#include <string>

namespace {

int failures = 0;

#define EXPECT(cond, ...)                     \
    do {                                      \
        if (!(cond)) {                        \
            std::fprintf(stderr, __VA_ARGS__); \
            std::fputc('\n', stderr);         \
            ++failures;                       \
        }                                     \
    } while (0)

uint64_t rng = 0x2545F4914F6CDD1Dull;
uint32_t next_u32() {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}

void resolve_limits() {
    using namespace fcs;
    Problem p;
    const int64_t big = (int64_t)1 << 31;
    for (int op = -1; op <= 3; ++op)
        for (int po = -1; po <= 2; ++po)
            for (int dt = -1; dt <= 3; ++dt) {
                const fc_status st = resolve(op, nullptr, po, nullptr, 0, nullptr, dt, 8, 8, 8, &p);
                const bool valid = op >= 0 && op <= 2 && (po == 0 || po == 1) && dt >= 0 && dt <= 2;
                EXPECT((st == FC_OK) == valid, "resolve op %d order %d dtype %d: %d", op, po, dt, (int)st);
            }
    // each dimension up to 2^31, each matrix up to 2^46 elements
    EXPECT(resolve(0, nullptr, 0, nullptr, 0, nullptr, 1, big, big, big, &p) == FC_E_INVALID, "2^31 cube accepted");
    EXPECT(resolve(0, nullptr, 0, nullptr, 0, nullptr, 1, big, (int64_t)1 << 15, 1, &p) == FC_OK, "2^46 X refused");
    EXPECT(resolve(0, nullptr, 0, nullptr, 0, nullptr, 1, big, ((int64_t)1 << 15) + 1, 1, &p) == FC_E_INVALID,
           "X past 2^46 accepted");
    EXPECT(resolve(2, nullptr, 0, nullptr, 0, nullptr, 2, 1, big, (int64_t)1 << 15, &p) == FC_OK, "2^46 dW refused");
    EXPECT(resolve(1, nullptr, 0, nullptr, 0, nullptr, 0, big + 1, 1, 1, &p) == FC_E_INVALID, "M > 2^31 accepted");
    EXPECT(resolve(1, nullptr, 0, nullptr, 0, nullptr, 0, 1, 0, 1, &p) == FC_E_INVALID, "K = 0 accepted");
    EXPECT(resolve(1, nullptr, 0, nullptr, 0, nullptr, 0, 1, 1, INT64_MIN, &p) == FC_E_INVALID, "N < 0 accepted");
    EXPECT(resolve(0, nullptr, 0, nullptr, 0, nullptr, 0, INT64_MAX, INT64_MAX, INT64_MAX, &p) == FC_E_INVALID,
           "INT64_MAX accepted");
    // pointer checks: all or none, aligned, output disjoint from the inputs
    alignas(16) static char buf[4096];
    EXPECT(resolve(0, buf, 0, nullptr, 0, buf + 2048, 0, 4, 4, 4, &p) == FC_E_INVALID, "missing pointer accepted");
    EXPECT(resolve(0, buf + 1, 0, buf + 512, 0, buf + 2048, 0, 4, 4, 4, &p) == FC_E_INVALID, "odd pointer accepted");
    EXPECT(resolve(0, buf, 0, buf + 512, 0, buf + 2050, 1, 4, 4, 4, &p) == FC_E_INVALID, "misaligned fp32 accepted");
    EXPECT(resolve(0, buf, 0, buf + 512, 0, buf + 16, 0, 4, 4, 4, &p) == FC_E_INVALID, "overlap accepted");
    EXPECT(resolve(0, buf, 0, buf + 512, 0, buf + 2048, 0, 4, 4, 4, &p) == FC_OK, "disjoint buffers refused");
    EXPECT(overlaps(buf, 32, buf + 31, 1) && !overlaps(buf, 32, buf + 32, 1) && !overlaps(buf, 0, buf, 8),
           "overlaps");
    EXPECT(!overlaps((void*)(~(uintptr_t)0 - 8), 4, buf, 16), "overlaps near the top of the address space");
}

void plan_space() {
    using namespace fcs;
    struct Shape {
        int64_t M, K, N;
    };
    // ragged, tiny, one-wave, multi-wave, tail-split, unaligned and huge shapes
    const Shape shapes[] = {{1, 1, 1},          {7, 5, 3},           {256, 512, 2048},    {8192, 2048, 2048},
                            {8192, 8192, 12288}, {8192, 16384, 16032}, {8192, 16032, 16384}, {8192, 26624, 4096},
                            {4096, 4096, 3584},  {2304, 4096, 2304},   {100, 64, 6000},     {(int64_t)1 << 31, 64, 1},
                            {1, (int64_t)1 << 31, 1}, {65536, 65536, 1024}, {8200, 8200, 8200}, {16, 2048, 16}};
    int described = 0;
    std::string text;
    for (const Shape& sh : shapes)
        for (int op = 0; op < 3; ++op)
            for (int xo = 0; xo < 2; ++xo)
                for (int wo = 0; wo < 2; ++wo)
                    for (int dt = 0; dt < 3; ++dt) {
                        Problem p;
                        const int po = op == FC_OP_BWD_DATA ? 0 : xo, qo = op == FC_OP_BWD_WEIGHT ? 0 : wo;
                        if (resolve(op, nullptr, po, nullptr, qo, nullptr, dt, sh.M, sh.K, sh.N, &p) != FC_OK) {
                            EXPECT(false, "resolve refused %lld %lld %lld", (long long)sh.M, (long long)sh.K,
                                   (long long)sh.N);
                            continue;
                        }
                        const int def = default_plan(p);
                        EXPECT(def >= 0 && def < kNumPlans && plan_applies(p, decode_plan(def)) &&
                                   ws_layout(p, decode_plan(def)).total == 0,
                               "default plan %d of %lld %lld %lld", def, (long long)sh.M, (long long)sh.K,
                               (long long)sh.N);
                        for (int id = 0; id < kNumPlans; ++id) {
                            const Plan pl = decode_plan(id);
                            EXPECT(encode_plan(pl.tile, pl.tail ? kTailSplit : (pl.split == 1 ? 0 : pl.split == 2 ? 1 : 2),
                                               pl.copy, pl.family) == id,
                                   "plan %d does not round-trip", id);
                            const bool applies = plan_applies(p, pl);
                            if (stampable(p, pl))
                                EXPECT(pl.family >= kFamilyW4 + 2 && !pl.tail && pl.copy == 0 && !p.out_f32,
                                       "stampable plan %d", id);
                            const WsLayout w = ws_layout(p, pl);
                            EXPECT(w.total >= 0 && w.total % 256 == 0 && w.a_off >= 0 && w.b_off >= 0 && w.p_off >= 0 &&
                                       w.a_off <= w.total && w.b_off <= w.total && w.p_off <= w.total,
                                   "workspace layout of plan %d", id);
                            if (pl.tail && applies) {
                                const TailGeo t = tail_geometry(p, w4_bn(pl));
                                const int64_t ext = t.along_n ? p.N : p.M;
                                EXPECT(t.ok && t.main > 0 && t.main < ext, "tail geometry of plan %d", id);
                            }
                            if (applies || (id % 7) == 0) {
                                text = describe(p, id);
                                EXPECT(text.rfind("plan=", 0) == 0 && text.find("kernel=") != std::string::npos,
                                       "description of plan %d: %s", id, text.c_str());
                                ++described;
                            }
                        }
                    }
    std::printf("plan space: %d descriptions\n", described);
}

void plan_lines() {
    using namespace fcs;
    PlanLine pl;
    EXPECT(parse_plan_line("gfx950:sramecc+:xnack- 0 8192 8192 4096 0 0 0 512 0.336760\n", &pl) == 0 &&
               pl.op == 0 && pl.M == 8192 && pl.K == 8192 && pl.N == 4096 && pl.id == 512 && pl.ms > 0.3367f &&
               pl.ms < 0.3368f && std::strcmp(pl.arch, "gfx950:sramecc+:xnack-") == 0,
           "a saved line");
    EXPECT(parse_plan_line("gfx950 2 1 2 3 1 0 2 -1", &pl) == 0 && pl.id == -1 && pl.ms < 0.0f, "a line without time");
    EXPECT(parse_plan_line("  \tgfx950 1 5 6 7 0 1 1 3 2.5  \r\n", &pl) == 0 && pl.ms == 2.5f, "blanks around fields");
    EXPECT(parse_plan_line("\n", &pl) == 1 && parse_plan_line("", &pl) == 1 && parse_plan_line("# x", &pl) == 1 &&
               parse_plan_line("   # indented", &pl) == 1,
           "blank and comment lines");
    const char* bad[] = {
        "gfx950 0 1 2 3 0 0 0",                     // a field short
        "gfx950 0 1 2 3 0 0 0 512 1.0 7",           // a field too many
        "gfx950 0 1 2 3 0 0 0 5x2",                 // trailing garbage in a number
        "gfx950 0 1 2 3 0 0 0 512 nan",             // not a time
        "gfx950 0 1 2 3 0 0 0 512 -3",              // negative time
        "gfx950 0 99999999999999999999 2 3 0 0 0 1",  // out of range
        "gfx950 0 1 2 3 0 0 4294967296 1",          // wraps an int
        "gfx950 0 1 2 3 0 0 0 100001",              // plan id out of range
        "gfx950 zero 1 2 3 0 0 0 1",                // not a number
        "gfx950 0 1 2 3 0 0 0 512 1e400",           // time overflows
    };
    for (const char* b : bad) EXPECT(parse_plan_line(b, &pl) == -1, "accepted: %s", b);
    std::string longarch(70, 'a');
    EXPECT(parse_plan_line((longarch + " 0 1 2 3 0 0 0 1").c_str(), &pl) == -1, "an over-long arch name");
    // random lines: printable characters, digits and blanks
    char line[600];
    int parsed = 0;
    for (int i = 0; i < 20000; ++i) {
        const int n = (int)(next_u32() % 580);
        for (int j = 0; j < n; ++j) {
            const uint32_t r = next_u32() % 4;
            line[j] = r == 0 ? ' ' : r == 1 ? (char)('0' + next_u32() % 10) : (char)(33 + next_u32() % 94);
        }
        line[n] = '\0';
        const int r = parse_plan_line(line, &pl);
        EXPECT(r >= -1 && r <= 1, "random line result %d", r);
        if (r == 0) {
            ++parsed;
            EXPECT(std::strlen(pl.arch) < sizeof pl.arch, "arch length");
        }
    }
    // random valid lines round-trip
    for (int i = 0; i < 2000; ++i) {
        const long long M = next_u32() % 100000, K = next_u32() % 100000, N = next_u32() % 100000;
        const int op = (int)(next_u32() % 3), id = (int)(next_u32() % 640);
        std::snprintf(line, sizeof line, "gfx950:x %d %lld %lld %lld %d %d %d %d %.6f\n", op, M, K, N, i & 1, 1 - (i & 1),
                      i % 3, id, (double)(next_u32() % 100000) / 1000.0);
        EXPECT(parse_plan_line(line, &pl) == 0 && pl.M == M && pl.K == K && pl.N == N && pl.op == op && pl.id == id,
               "round trip: %s", line);
    }
    std::printf("plan lines: %d random lines parsed as plan lines\n", parsed);
}

void entry_points() {
    int ndev = 0;
    const bool device = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;
    (void)hipGetLastError();
    for (int s = -3; s < 12; ++s) EXPECT(fc_status_str((fc_status)s) != nullptr, "status string %d", s);
    EXPECT(std::strcmp(fc_status_str((fc_status)99), "unknown fc_status") == 0, "unknown status");
    EXPECT(fc_plan_count() == 640 && fc_noalloc_scratch_bytes() == ((int64_t)64 << 20), "counts");
    // malformed arguments are refused before any device work
    alignas(16) static char buf[4096];
    void* a = buf;
    void* b = buf + 1024;
    void* c = buf + 2048;
    EXPECT(fc_fwd(nullptr, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, nullptr) == FC_E_INVALID, "fwd null");
    EXPECT(fc_fwd(a, (fc_order)7, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, nullptr) == FC_E_INVALID, "fwd order");
    EXPECT(fc_fwd(a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, (fc_out_dtype)9, 4, 4, 4, nullptr) == FC_E_INVALID, "fwd dtype");
    EXPECT(fc_fwd(a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 0, 4, 4, nullptr) == FC_E_INVALID, "fwd M = 0");
    EXPECT(fc_bwd_data(a, b, FC_COL_MAJOR, a, FC_OUT_BF16, 4, 4, 4, nullptr) == FC_E_INVALID, "bwd-data aliasing");
    EXPECT(fc_bwd_weight(a, FC_ROW_MAJOR, b, c, FC_OUT_F32, -4, 4, 4, nullptr) == FC_E_INVALID, "bwd-weight M < 0");
    EXPECT(fc_bwd_weight_noalloc(a, FC_ROW_MAJOR, nullptr, c, FC_OUT_F32, 4, 4, 4, nullptr) == FC_E_INVALID,
           "noalloc null");
    EXPECT(fc_tune(4, 4, 4, (fc_order)2, FC_ROW_MAJOR, FC_OUT_BF16, 0, nullptr) == FC_E_INVALID, "tune order");
    EXPECT(fc_tune(4, 0, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, 0, nullptr) == FC_E_INVALID, "tune K = 0");
    EXPECT(fc_set_plan(FC_OP_FWD, 4, 4, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, 640) == FC_E_INVALID, "plan 640");
    EXPECT(fc_set_plan(FC_OP_FWD, 4, 4, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, -2) == FC_E_INVALID, "plan -2");
    EXPECT(fc_set_plan((fc_op)5, 4, 4, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, 0) == FC_E_INVALID, "op 5");
    char text[8];
    EXPECT(fc_plan_describe(FC_OP_FWD, 4, 4, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, nullptr, 8) == FC_E_INVALID,
           "describe null buffer");
    EXPECT(fc_plan_describe(FC_OP_FWD, 4, 4, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, text, 0) == FC_E_INVALID,
           "describe empty buffer");
    EXPECT(fc_plans_save(nullptr) == FC_E_INVALID && fc_plans_load(nullptr) == FC_E_INVALID, "null plan file");
    EXPECT(fc_mfma_probe(0, nullptr, nullptr) == FC_E_INVALID, "probe iters 0");
    int64_t nb = -1;
    EXPECT(fc_stamped_call(FC_OP_FWD, a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, nullptr, 64, &nb,
                           nullptr) == FC_E_INVALID,
           "stamped call without a buffer");
    EXPECT(fc_stamped_call(FC_OP_FWD, a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, buf + 3000, 64,
                           nullptr, nullptr) == FC_E_INVALID,
           "stamped call without a block count");
    EXPECT(fc_stamped_call(FC_OP_FWD, a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, buf + 3001, 64, &nb,
                           nullptr) == FC_E_INVALID,
           "stamped call with a misaligned buffer");
    EXPECT(fc_stamped_call((fc_op)3, a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, buf + 3000, 64, &nb,
                           nullptr) == FC_E_INVALID,
           "stamped call with op 3");
    EXPECT(fc_stamped_call(FC_OP_BWD_WEIGHT, a, (fc_order)5, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, buf + 3000,
                           64, &nb, nullptr) == FC_E_INVALID,
           "stamped call with a bad order");
    EXPECT(fc_mfma_probe_launch(1, -1, buf, nullptr) == FC_E_INVALID, "probe launch blocks < 0");
    if (!device) {
        // with no device, calls that pass validation stop at the device check
        // (the pointers are never dereferenced on the host)
        const fc_status st = fc_fwd(a, FC_ROW_MAJOR, b, FC_ROW_MAJOR, c, FC_OUT_BF16, 4, 4, 4, nullptr);
        EXPECT(st == FC_E_HIP || st == FC_E_UNSUPPORTED, "fwd without a device: %d", (int)st);
        EXPECT(fc_plans_load("/nonexistent/plans.txt") != FC_OK, "plan file without a device");
        EXPECT(fc_plan_describe(FC_OP_FWD, 4, 4, 4, FC_ROW_MAJOR, FC_ROW_MAJOR, FC_OUT_BF16, text, sizeof text) !=
                   FC_OK,
               "describe without a device");
    }
    EXPECT(fc_release() == FC_OK, "release");
}

}  // namespace

int main() {
    resolve_limits();
    plan_space();
    plan_lines();
    entry_points();
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("sanitized ABI run: ok\n");
    return 0;
}
