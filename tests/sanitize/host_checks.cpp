// host_checks.cpp -- the host side of libfsdp_shard.so under sanitizers
// (tests/test_sanitizers.py builds every library source with this driver, once
// with AddressSanitizer + UndefinedBehaviorSanitizer and once with
// ThreadSanitizer).  No GPU is needed: with device pointers that are never
// dereferenced on the host, every device call runs its argument validation and
// its launch planning (the 2^26-element slicing, the unit, copy and segment
// tables) on the host and returns FSDP_E_HIP at its first kernel launch.  That
// part is skipped when a device is present, so the fake pointers never reach a
// kernel.  Host-memory paths run for real: CRC32C, the threaded host AdamW of
// the offloaded step, sharded-checkpoint save/load and the shard-file parser
// fed truncated and bit-flipped files.
//
// usage: host_checks all|threads <scratch directory>
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "fsdp_shard.h"

namespace {

const uintptr_t kFake = uintptr_t(1) << 40;   // device-looking addresses, never dereferenced on the host
int g_checks = 0;

#define CHECK(cond, what)                                                                                      \
    do {                                                                                                       \
        ++g_checks;                                                                                            \
        if (!(cond)) {                                                                                         \
            fprintf(stderr, "host check failed: %s (line %d); last error: %s\n", what, __LINE__,               \
                    fsdp_last_error());                                                                        \
            exit(1);                                                                                           \
        }                                                                                                      \
    } while (0)

void* fake(int k, uintptr_t off = 0) { return (void*)(kFake + (uintptr_t(k) << 36) + off); }

uint32_t g_rng = 2463534242u;
uint32_t rnd() {
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 17;
    g_rng ^= g_rng << 5;
    return g_rng;
}

// ------------------------------------------------------------------ host-only queries
void queries() {
    for (int trial = 0; trial < 300; ++trial) {
        const int T = (int)(rnd() % 9);
        std::vector<int64_t> n(T);
        int64_t sum = 0;
        for (auto& x : n) sum += x = (int64_t)(rnd() % 100000);
        const int world = 1 + (int)(rnd() % FSDP_MAX_WORLD);
        int64_t P = -1, Pp = -1, S = -1;
        CHECK(fsdp_layout(n.data(), T, world, &P, &Pp, &S) == FSDP_OK, "layout");
        CHECK(P == sum && Pp % world == 0 && Pp - P < world && S * world == Pp, "layout sizes");
        std::vector<fsdp_view> v(T + 1);
        CHECK(fsdp_unflatten_views(n.data(), T, Pp, v.data(), nullptr, FSDP_F32, nullptr, nullptr) == FSDP_OK,
              "views");
        int64_t off = 0;
        for (int k = 0; k < T; ++k) {
            CHECK(v[k].offset == off && v[k].numel == n[k], "view table");
            off += n[k];
        }
        std::vector<int64_t> shards(1 + rnd() % 50);
        for (auto& x : shards) x = (int64_t)(rnd() % (3u << 26));
        int64_t elems = -1;
        const int c = fsdp_units_in_launch(world, shards.data(), (int)shards.size(), &elems);
        CHECK(c >= 1 && c <= (int)shards.size() && elems > 0 && elems <= (int64_t(1) << 26), "units in launch");
        CHECK(fsdp_unit_gather_split(FSDP_F32, (int)(rnd() % 3), elems) >= 0, "gather split");
    }
    int64_t P;
    const int64_t bad[2] = {5, -1};
    CHECK(fsdp_layout(bad, 2, 2, &P, nullptr, nullptr) == FSDP_E_INVAL, "negative numel");
    const int64_t huge[2] = {INT64_MAX / 2, INT64_MAX / 2};
    CHECK(fsdp_layout(huge, 2, 2, &P, nullptr, nullptr) == FSDP_E_SIZE, "overflowing unit");
    CHECK(fsdp_units_in_launch(0, bad, 1, nullptr) == FSDP_E_INVAL, "units in launch world 0");
    CHECK(fsdp_units_in_launch(2, bad, 2, nullptr) == FSDP_E_INVAL, "units in launch negative");
}

// ------------------------------------------------------------------ validation
void validation() {
    fsdp_adamw_hp hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1};
    const void* g2[2] = {fake(1), fake(2)};
    const void* peers[2] = {nullptr, fake(3)};
    float* a = (float*)fake(4);
    float* b = (float*)fake(5);
    float* c = (float*)fake(6);
    // world / rank / dtype / hp / NULL / alias errors, every one before a launch
    CHECK(fsdp_sharded_adamw(a, b, c, g2, 0, 0, FSDP_F16, 1, fake(7), FSDP_F16, 100, &hp, nullptr) == FSDP_E_INVAL,
          "world 0");
    CHECK(fsdp_sharded_adamw(a, b, c, g2, 2, 2, FSDP_F16, 1, fake(7), FSDP_F16, 100, &hp, nullptr) == FSDP_E_INVAL,
          "rank 2");
    CHECK(fsdp_sharded_adamw(a, b, c, g2, 2, 0, (fsdp_dtype)9, 1, fake(7), FSDP_F16, 100, &hp, nullptr) ==
              FSDP_E_DTYPE, "grad dtype");
    CHECK(fsdp_sharded_adamw(a, a + 10, c, g2, 2, 0, FSDP_F16, 1, fake(7), FSDP_F16, 100, &hp, nullptr) ==
              FSDP_E_ALIAS, "master overlaps m");
    CHECK(fsdp_sharded_adamw(a, b, c, g2, 2, 0, FSDP_F16, 1, fake(7), FSDP_F16, -1, &hp, nullptr) == FSDP_E_INVAL,
          "negative shard");
    CHECK(fsdp_sharded_adamw(a, b, c, g2, 2, 0, FSDP_F16, 1, fake(7), FSDP_F16, 100, nullptr, nullptr) ==
              FSDP_E_INVAL, "hp NULL");
    for (int f = 0; f < 6; ++f) {
        fsdp_adamw_hp h = hp;
        const float badv = f < 3 ? -1.0f : NAN;
        if (f % 3 == 0) h.lr = badv;
        if (f % 3 == 1) h.eps = badv;
        if (f % 3 == 2) h.weight_decay = badv;
        CHECK(fsdp_sharded_adamw(a, b, c, g2, 2, 0, FSDP_F16, 1, fake(7), FSDP_F16, 100, &h, nullptr) ==
                  FSDP_E_INVAL, "bad hyper-parameter");
    }
    CHECK(fsdp_step_unit(a, b, c, g2, 2, 0, FSDP_BF16, 0, peers, fake(8, 2), FSDP_BF16, 100, fake(8), &hp,
                         nullptr) == FSDP_E_ALIAS, "persistent copy inside the full buffer");
    CHECK(fsdp_reduce_scatter_local(g2, 2, 1, 100, FSDP_F16, 0, (char*)fake(1) + 200, nullptr) == FSDP_E_ALIAS,
          "reduce-scatter output overlaps its input");
    const void* sh[2] = {(char*)fake(9) + 100, fake(10)};
    CHECK(fsdp_unshard_gather(sh, 2, 100, FSDP_F16, fake(9), nullptr) == FSDP_E_ALIAS, "gather alias");
    const int64_t n1[1] = {10};
    const void* src1[1] = {(char*)fake(11) + 8};
    CHECK(fsdp_flatten_pad(src1, n1, 1, FSDP_F32, 4, fake(11), 12, nullptr, nullptr) == FSDP_E_ALIAS,
          "flatten alias");
    CHECK(fsdp_flatten_pad(src1, n1, 1, FSDP_F32, 4, fake(12), 11, nullptr, nullptr) == FSDP_E_SIZE,
          "flatten capacity");
    fsdp_view v[2];
    const int64_t n2[2] = {5, 6};
    CHECK(fsdp_unflatten_views(n2, 2, 10, v, nullptr, FSDP_F32, nullptr, nullptr) == FSDP_E_SIZE, "views size");
    void* d2[2] = {fake(13), (char*)fake(13) + 8};
    CHECK(fsdp_unflatten_views(n2, 2, 11, v, fake(14), FSDP_F32, d2, nullptr) == FSDP_E_ALIAS, "views dsts alias");
    fsdp_unit u[2] = {};
    u[0] = fsdp_unit{fake(15), fake(16), fake(17), g2, peers, fake(18), nullptr, 100};
    u[1] = u[0];
    CHECK(fsdp_step_units(u, 2, 2, 0, FSDP_BF16, 0, FSDP_F32, FSDP_BF16, &hp, nullptr) == FSDP_E_ALIAS,
          "a unit twice");
    CHECK(fsdp_step_units(u, 1, 2, 0, FSDP_BF16, 0, FSDP_BF16, FSDP_F16, &hp, nullptr) == FSDP_E_DTYPE,
          "16-bit state with another compute dtype");
    fsdp_optim_hp o = {};
    o.kind = (fsdp_optimizer)7;
    o.step = 1;
    CHECK(fsdp_step_units_optim(u, 1, 2, 0, FSDP_BF16, 0, FSDP_F32, FSDP_BF16, &o, nullptr) == FSDP_E_INVAL,
          "unknown optimizer");
    // offload: validation only (these return before any HIP call)
    std::vector<float> hm(64), hv(64), hp2(64), hg(64), hc(64);
    fsdp_offload_unit ou = {hm.data(), hv.data(), hp2.data(), g2, fake(19), hg.data(), hc.data(), fake(20), 64};
    fsdp_offload_unit dup[2] = {ou, ou};
    CHECK(fsdp_offload_step_units(dup, 2, 2, 0, FSDP_F16, 1, FSDP_F16, 0, &hp, 2, nullptr, nullptr) == FSDP_E_ALIAS,
          "offload unit twice");
    CHECK(fsdp_offload_step_units_noalloc(&ou, 1, 2, 0, FSDP_F16, 1, FSDP_F16, 0, &hp, 2, nullptr, nullptr) ==
              FSDP_E_INVAL, "no-alloc offload with a device gradient shard");
    ou.grad_shard_dev = nullptr;
    CHECK(fsdp_offload_step_units_noalloc(&ou, 1, 2, 0, FSDP_F16, 1, FSDP_F16, (FSDP_OFFLOAD_SCRATCH_BYTES / 4) + 8,
                                          &hp, 2, nullptr, nullptr) == FSDP_E_SIZE, "no-alloc chunk too large");
}

// ------------------------------------------------------------------ launch planning (no device only)
int expect_launch(int rc, const char* what) {
    // without a device the planning ran to the first launch, which failed
    CHECK(rc == FSDP_E_HIP, what);
    return rc;
}

void launch_planning() {
    fsdp_adamw_hp hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 3};
    int k = 100;
    auto grads = [&](int world) {
        std::vector<const void*> g(world);
        for (auto& p : g) p = fake(k++);
        return g;
    };
    auto peers_of = [&](int world, int rank) {
        std::vector<const void*> p(world, nullptr);
        for (int q = 0; q < world; ++q)
            if (q != rank) p[q] = fake(k++);
        return p;
    };
    const int64_t cap = int64_t(1) << 26;
    struct Case {
        int world, rank;
        std::vector<int64_t> sizes;
        fsdp_dtype gdt, state, cdt;
        bool gather, persistent;
        uintptr_t misalign;
    };
    const std::vector<Case> cases = {
        {2, 1, {3 * cap + 1003}, FSDP_F16, FSDP_F32, FSDP_F16, true, false, 0},          // slices, split copies
        {2, 0, std::vector<int64_t>(40, 1000003), FSDP_F16, FSDP_F32, FSDP_F16, true, false, 0},   // packing
        {8, 7, {cap + 517, 12345, 2 * cap}, FSDP_BF16, FSDP_F32, FSDP_BF16, true, true, 0},
        {3, 2, {4099 + 7, 333}, FSDP_BF16, FSDP_F32, FSDP_BF16, true, false, 0},           // generic N
        {FSDP_MAX_WORLD, 127, {1000}, FSDP_F16, FSDP_F32, FSDP_F16, true, false, 0},     // the largest world
        {2, 1, {100003, cap + 9}, FSDP_BF16, FSDP_BF16, FSDP_BF16, true, false, 0},       // 16-bit state
        {4, 3, {777, 12345}, FSDP_F32, FSDP_F32, FSDP_F32, false, false, 0},              // no gather
        {2, 0, {12345}, FSDP_F16, FSDP_F32, FSDP_F16, true, true, 4},                     // unaligned
    };
    for (const Case& cs : cases) {
        std::vector<std::vector<const void*>> gs, ps;
        std::vector<fsdp_unit> units;
        for (int64_t S : cs.sizes) {
            gs.push_back(grads(cs.world));
            ps.push_back(peers_of(cs.world, cs.rank));
            fsdp_unit u = {};
            u.master = (char*)fake(k++) + cs.misalign;
            u.exp_avg = fake(k++);
            u.exp_avg_sq = fake(k++);
            u.rank_grads = gs.back().data();
            u.peer_shards = cs.gather ? ps.back().data() : nullptr;
            u.full_out = cs.gather ? fake(k++) : nullptr;
            u.compute_shard = cs.persistent || !cs.gather ? fake(k++) : nullptr;
            u.shard_numel = S;
            units.push_back(u);
        }
        expect_launch(fsdp_step_units(units.data(), (int)units.size(), cs.world, cs.rank, cs.gdt, 1, cs.state, cs.cdt,
                                      &hp, nullptr), "step_units planning");
        if (cs.state == FSDP_F32) {
            fsdp_optim_hp o = {};
            o.lr = 1e-2f;
            o.step = 2;
            o.kind = FSDP_OPT_SGD;
            expect_launch(fsdp_step_units_optim(units.data(), (int)units.size(), cs.world, cs.rank, cs.gdt, 1,
                                                cs.state, cs.cdt, &o, nullptr), "SGD planning");
            o.momentum = 0.9f;
            expect_launch(fsdp_step_units_optim(units.data(), (int)units.size(), cs.world, cs.rank, cs.gdt, 1,
                                                cs.state, cs.cdt, &o, nullptr), "SGD momentum planning");
            o.kind = FSDP_OPT_ADAMAX;
            o.beta1 = 0.9f;
            o.beta2 = 0.999f;
            o.eps = 1e-8f;
            expect_launch(fsdp_step_units_optim(units.data(), (int)units.size(), cs.world, cs.rank, cs.gdt, 1,
                                                cs.state, cs.cdt, &o, nullptr), "Adamax planning");
            o.kind = FSDP_OPT_ADADELTA;
            o.rho = 0.9f;
            expect_launch(fsdp_step_units_optim(units.data(), (int)units.size(), cs.world, cs.rank, cs.gdt, 1,
                                                cs.state, cs.cdt, &o, nullptr), "Adadelta planning");
        }
    }
    // single-unit entry points
    auto g8 = grads(8);
    auto p8 = peers_of(8, 3);
    float* st[3];
    for (auto& x : st) x = (float*)fake(k++);
    void* full8 = fake(k++);
    void* pers8 = fake(k++);
    expect_launch(fsdp_step_unit(st[0], st[1], st[2], g8.data(), 8, 3, FSDP_F16, 1, p8.data(), full8, FSDP_F16,
                                 2 * cap + 5, pers8, &hp, nullptr), "step_unit planning");
    for (auto& x : st) x = (float*)fake(k++);
    void* comp = fake(k++);
    expect_launch(fsdp_sharded_adamw((float*)((char*)st[0] + 4), st[1], st[2], g8.data(), 8, 0, FSDP_BF16, 0, comp,
                                     FSDP_BF16, 3 * cap + 1, &hp, nullptr), "sharded_adamw planning");
    auto gmax = grads(FSDP_MAX_WORLD);
    expect_launch(fsdp_reduce_scatter_local(gmax.data(), FSDP_MAX_WORLD, 5, 100003, FSDP_F16, 1, fake(k++), nullptr),
                  "reduce-scatter planning");
    std::vector<const void*> shards(FSDP_MAX_WORLD);
    void* full = fake(k++);
    for (int q = 0; q < FSDP_MAX_WORLD; ++q) shards[q] = q % 3 ? fake(k++) : (const char*)full + q * 2 * 1001;
    expect_launch(fsdp_unshard_gather(shards.data(), FSDP_MAX_WORLD, 1001, FSDP_F16, full, nullptr),
                  "gather planning");
    // flatten / unflatten over more tensors than one segment table holds
    const int T = 300;
    std::vector<int64_t> numels(T);
    std::vector<const void*> srcs(T);
    std::vector<void*> dsts(T);
    for (int t = 0; t < T; ++t) {
        numels[t] = (t * 7919) % 5000;
        srcs[t] = fake(k++);
        dsts[t] = fake(k++);
    }
    int64_t Pp = 0;
    void* flat = fake(k++);
    expect_launch(fsdp_flatten_pad(srcs.data(), numels.data(), T, FSDP_BF16, 7, flat, INT64_MAX / 4, &Pp, nullptr),
                  "flatten planning");
    CHECK(Pp % 7 == 0 && Pp > 0, "padded length reported before the launch");
    std::vector<fsdp_view> views(T);
    expect_launch(fsdp_unflatten_views(numels.data(), T, Pp, views.data(), fake(k++), FSDP_BF16, dsts.data(), nullptr),
                  "unflatten planning");
}

// ------------------------------------------------------------------ CRC32C
uint32_t crc_bitwise(const unsigned char* p, size_t n) {
    uint32_t c = 0xFFFFFFFFu;
    for (size_t i = 0; i < n; ++i) {
        c ^= p[i];
        for (int b = 0; b < 8; ++b) c = (c >> 1) ^ ((c & 1) ? 0x82F63B78u : 0u);
    }
    return c ^ 0xFFFFFFFFu;
}

void crc(bool threads) {
    // exact-size buffers at every start offset: no byte past the end may be read
    for (size_t n = 0; n < 1100; n += (n < 80 ? 1 : 37))
        for (size_t off = 0; off < 8; ++off) {
            unsigned char* buf = (unsigned char*)malloc(n + off ? n + off : 1);
            for (size_t i = 0; i < n + off; ++i) buf[i] = (unsigned char)rnd();
            CHECK(fsdp_crc32c(buf + off, (int64_t)n) == (n ? crc_bitwise(buf + off, n) : 0u), "crc32c");
            free(buf);
        }
    for (size_t n : {size_t(65535), size_t(65536), size_t(65536 + 23), size_t(3 * 65536 + 7), size_t(200003)}) {
        std::vector<unsigned char> v(n);
        for (auto& x : v) x = (unsigned char)rnd();
        unsigned char* buf = (unsigned char*)malloc(n);
        memcpy(buf, v.data(), n);
        const uint32_t want = crc_bitwise(buf, n);
        CHECK(fsdp_crc32c(buf, (int64_t)n) == want, "crc32c multi-lane");
        if (threads) {   // concurrent callers share the dispatch and keep their own lane maps
            std::vector<std::thread> ts;
            std::vector<uint32_t> got(8);
            for (int t = 0; t < 8; ++t)
                ts.emplace_back([&, t] {
                    for (int r = 0; r < 4; ++r) got[t] = fsdp_crc32c(buf + (t % 3), (int64_t)(n - 3));
                });
            for (auto& t : ts) t.join();
            const uint32_t ref = crc_bitwise(buf + 0, n - 3);
            CHECK(got[0] == ref && got[3] == ref && got[6] == ref, "crc32c from threads");
        }
        free(buf);
    }
}

// ------------------------------------------------------------------ host AdamW
uint16_t f2h_rne(float x) {   // only for building inputs: any 16-bit pattern will do
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

void host_adamw(bool threads) {
    const int64_t sizes[] = {0, 1, 7, 8, 9, 63, 64, 65, 4095, 4096, 8193, 65537, 100003};
    const int thread_counts[] = {1, 3, 16};
    const fsdp_dtype dts[] = {FSDP_F32, FSDP_F16, FSDP_BF16};
    fsdp_adamw_hp hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 3};
    for (int64_t n : sizes)
        for (fsdp_dtype gdt : dts)
            for (int cdt = -1; cdt < 3; ++cdt)
                for (int mis = 0; mis < 2; ++mis) {
                    if (threads && (n < 4096 || mis)) continue;
                    const int64_t gs = gdt == FSDP_F32 ? 4 : 2, cs = cdt == FSDP_F32 ? 4 : 2;
                    std::vector<float> p0(n), m0(n), v0(n);
                    std::vector<unsigned char> g0(n * gs);
                    for (int64_t i = 0; i < n; ++i) {
                        p0[i] = ((int32_t)rnd() / 2147483648.0f) * 0.02f;
                        m0[i] = ((rnd() % 1000) / 1000.0f) * 1e-4f;
                        v0[i] = ((rnd() % 1000) / 1000.0f) * 1e-6f;
                        const float g = ((int32_t)rnd() / 2147483648.0f) * 1e-3f;
                        if (gdt == FSDP_F32) memcpy(&g0[i * 4], &g, 4);
                        else {
                            const uint16_t h = f2h_rne(g);
                            memcpy(&g0[i * 2], &h, 2);
                        }
                    }
                    std::vector<std::vector<unsigned char>> ref;
                    for (int tc : thread_counts) {
                        // exact-size allocations, shifted by `mis` elements off the 32-byte grid
                        float* p = (float*)malloc(4 * (n + mis) + 1);
                        float* m = (float*)malloc(4 * (n + mis) + 1);
                        float* v = (float*)malloc(4 * (n + mis) + 1);
                        unsigned char* g = (unsigned char*)malloc(gs * (n + mis) + 1);
                        unsigned char* c = cdt >= 0 ? (unsigned char*)malloc(cs * (n + mis) + 1) : nullptr;
                        if (n > 0) {
                            memcpy(p + mis, p0.data(), 4 * n);
                            memcpy(m + mis, m0.data(), 4 * n);
                            memcpy(v + mis, v0.data(), 4 * n);
                            memcpy(g + gs * mis, g0.data(), gs * n);
                        }
                        const int rc = fsdp_host_adamw(p + mis, m + mis, v + mis, g + gs * mis, gdt,
                                                       c ? c + cs * mis : nullptr, (fsdp_dtype)(cdt < 0 ? 0 : cdt), n,
                                                       &hp, tc);
                        CHECK(rc == FSDP_OK, "host adamw");
                        std::vector<unsigned char> out(4 * n * 3 + (c ? cs * n : 0));
                        if (n > 0) {
                            memcpy(out.data(), p + mis, 4 * n);
                            memcpy(out.data() + 4 * n, m + mis, 4 * n);
                            memcpy(out.data() + 8 * n, v + mis, 4 * n);
                            if (c) memcpy(out.data() + 12 * n, c + cs * mis, cs * n);
                        }
                        ref.push_back(out);
                        free(p);
                        free(m);
                        free(v);
                        free(g);
                        free(c);
                    }
                    for (size_t r = 1; r < ref.size(); ++r)
                        CHECK(ref[r] == ref[0], "host adamw: every thread count gives the same bytes");
                }
}

// ------------------------------------------------------------------ checkpoint files
std::vector<unsigned char> read_file(const std::string& path) {
    std::vector<unsigned char> v;
    FILE* f = fopen(path.c_str(), "rb");
    if (!f) return v;
    int ch;
    while ((ch = fgetc(f)) != EOF) v.push_back((unsigned char)ch);
    fclose(f);
    return v;
}

void write_file(const std::string& path, const unsigned char* p, size_t n) {
    FILE* f = fopen(path.c_str(), "wb");
    CHECK(f != nullptr, "open scratch file");
    CHECK(fwrite(p, 1, n, f) == n, "write scratch file");
    fclose(f);
}

void checkpoint(const std::string& dir) {
    const int64_t S = 1031;
    const int64_t numels[2] = {2 * S - 9, 8};
    fsdp_ckpt_info info = {};
    info.world = 2;
    info.rank = 1;
    info.numel = 2 * S - 1;
    info.padded_numel = 2 * S;
    info.shard_numel = S;
    info.state_dt = FSDP_F32;
    info.compute_dt = FSDP_BF16;
    info.step = 7;
    info.hp = fsdp_adamw_hp{3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 7};
    info.n_tensors = 2;
    std::vector<float> st[3];
    for (auto& x : st) {
        x.resize(S);
        for (auto& y : x) y = (float)(int32_t)rnd();
    }
    const std::string path = dir + "/unit-shard1";
    CHECK(fsdp_save_shard(path.c_str(), &info, numels, st[0].data(), st[1].data(), st[2].data(), 0, nullptr) ==
              FSDP_OK, "save");
    const std::vector<unsigned char> raw = read_file(path);
    CHECK(raw.size() == 4096 + 12 * (size_t)S, "file size");
    auto load = [&](const unsigned char* bytes, size_t n) {
        write_file(path, bytes, n);
        float* d[3];
        for (auto& x : d) x = (float*)malloc(4 * S);   // exactly the capacity given
        fsdp_ckpt_info got;
        int64_t sizes[2];
        const int rc_info = fsdp_shard_info(path.c_str(), &got, sizes, 2);
        const int rc = fsdp_load_shard(path.c_str(), &got, d[0], d[1], d[2], S, 0, nullptr);
        bool same = rc == FSDP_OK;
        for (int k = 0; k < 3 && same; ++k) same = memcmp(d[k], st[k].data(), 4 * S) == 0;
        for (auto& x : d) free(x);
        CHECK(rc != FSDP_OK || same, "a load that succeeds returns the saved bytes");
        CHECK(rc != FSDP_OK || rc_info == FSDP_OK, "info agrees with load");
        return rc;
    };
    CHECK(load(raw.data(), raw.size()) == FSDP_OK, "clean load");
    for (size_t cut = 0; cut < raw.size(); cut += (cut < 4200 ? 1 : 97))
        CHECK(load(raw.data(), cut) == FSDP_E_FORMAT, "truncated file");
    std::vector<unsigned char> more(raw);
    more.push_back(0);
    CHECK(load(more.data(), more.size()) == FSDP_E_FORMAT, "trailing byte");
    const size_t table_end = 256 + 16;
    for (size_t at = 0; at < raw.size(); at += (at < table_end ? 1 : (at < 4096 ? 61 : 13))) {
        std::vector<unsigned char> bad(raw);
        bad[at] ^= (unsigned char)(1u << (at % 8));
        const int rc = load(bad.data(), bad.size());
        if (at < table_end || at >= 4096) CHECK(rc == FSDP_E_FORMAT, "flipped bit detected");
        else CHECK(rc == FSDP_OK, "the gap before the payload holds no data");
    }
    write_file(path, raw.data(), raw.size());
    float* small[3];
    for (auto& x : small) x = (float*)malloc(4 * (S - 1));
    CHECK(fsdp_load_shard(path.c_str(), nullptr, small[0], small[1], small[2], S - 1, 0, nullptr) == FSDP_E_SIZE,
          "capacity");
    for (auto& x : small) free(x);
    CHECK(fsdp_load_shard((dir + "/missing").c_str(), nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr) == FSDP_E_IO,
          "missing file");
    remove(path.c_str());
}

}  // namespace

int main(int argc, char** argv) {
    if (argc < 3) {
        fprintf(stderr, "usage: %s all|threads <scratch directory>\n", argv[0]);
        return 2;
    }
    const bool all = strcmp(argv[1], "all") == 0;
    const std::string dir = argv[2];
    int devices = 0;
    const bool device = hipGetDeviceCount(&devices) == hipSuccess && devices > 0;
    if (all) {
        queries();
        validation();
        if (!device) launch_planning();
        else printf("a device is present: launch planning with fake pointers skipped\n");
        checkpoint(dir);
    }
    crc(!all);
    host_adamw(!all);
    printf("host sanitizer checks (%s): %d checks ok\n", argv[1], g_checks);
    return 0;
}
