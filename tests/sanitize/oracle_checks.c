/*
 * oracle_checks.c -- every function of the CPU oracle (oracle/fsdp_oracle.c)
 * on buffers allocated to their exact size, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py
 * compiles the oracle source together with this file): any access past an
 * allocation or any undefined operation stops the run.  A few invariants are
 * checked so that the run is not vacuous; the oracle's values are pinned by
 * the oracle tests.  Test infrastructure, like the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} orc_hp;

typedef struct {
    float lr, weight_decay, momentum, dampening, beta1, beta2, eps, rho;
    int32_t nesterov;
    int64_t step;
} orc_opt;

uint16_t orc_f32_to_f16(float x);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float x);
float orc_bf16_to_f32(uint16_t h);
void orc_cast_from_f32(const float* src, int dt, void* dst, int64_t n);
void orc_cast_to_f32(const void* src, int dt, float* dst, int64_t n);
int64_t orc_padded_numel(int64_t total, int32_t world);
void orc_offsets(const int64_t* numels, int32_t n_tensors, int64_t* offsets);
void orc_flatten_pad(const void* const* srcs, const int64_t* numels, int32_t n_tensors, int64_t elem_size,
                     int64_t padded_numel, void* flat);
void orc_unflatten(const void* flat, const int64_t* numels, int32_t n_tensors, int64_t elem_size, void* const* dsts);
void orc_grad_average(const void* const* grads, int32_t world, int64_t begin, int64_t count, int grad_dt,
                      int fp32_reduce, void* out);
void orc_all_reduce(const void* const* grads, int32_t world, int64_t padded_numel, int grad_dt, int fp32_reduce,
                    void* out);
void orc_reduce_scatter(const void* const* grads, int32_t world, int32_t rank, int64_t shard_numel, int grad_dt,
                        int fp32_reduce, void* out);
void orc_adamw_scalars(const orc_hp* hp, float* out);
void orc_adamw(float* p, float* m, float* v, const float* g, int64_t n, const orc_hp* hp);
void orc_adamw16(uint16_t* p, uint16_t* m, uint16_t* v, int state_dt, const float* g, int64_t n, const orc_hp* hp);
void orc_sgd(float* p, float* buf, const float* g, int64_t n, const orc_opt* o);
void orc_adamax(float* p, float* m, float* u, const float* g, int64_t n, const orc_opt* o);
void orc_adadelta(float* p, float* v, float* acc, const float* g, int64_t n, const orc_opt* o);
void orc_cast(const float* master, int compute_dt, void* out, int64_t n);
void orc_gather(const void* const* shards, int32_t world, int64_t shard_numel, int64_t elem_size, void* full);
void orc_memory_per_worker(int64_t numel, int32_t world, int shard_params, int shard_grads, int shard_optim,
                           double param_bytes, double grad_bytes, double optim_bytes, double* out);

static uint32_t g_rng = 12345u;
static uint32_t rnd(void) {
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 17;
    g_rng ^= g_rng << 5;
    return g_rng;
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);   /* exact size: ASan's red zone starts right after it */
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void fail(const char* what) {
    fprintf(stderr, "oracle check failed: %s\n", what);
    exit(1);
}

static int64_t esize(int dt) { return dt == 0 ? 4 : 2; }

/* n values of format dt (fp32 or 16-bit patterns), scaled, with specials mixed in. */
static void* values(int64_t n, int dt, float scale) {
    float* f = (float*)xmalloc((size_t)n * 4);
    static const float specials[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 1e-40f, -3e-39f, 65504.0f, 7e4f};
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t r = rnd();
        f[i] = (r % 61 == 0) ? specials[r % 9] : ((float)(int32_t)rnd() / 2147483648.0f) * scale;
    }
    if (dt == 0) return f;
    void* h = xmalloc((size_t)n * 2);
    orc_cast_from_f32(f, dt, h, n);
    free(f);
    return h;
}

static void check_formats(void) {
    for (uint32_t u = 0; u < 0x10000u; ++u) {
        const float a = orc_f16_to_f32((uint16_t)u), b = orc_bf16_to_f32((uint16_t)u);
        if (a == a && orc_f32_to_f16(a) != (uint16_t)u) fail("binary16 round trip");
        if (b == b && orc_f32_to_bf16(b) != (uint16_t)u) fail("bfloat16 round trip");
    }
    for (int k = 0; k < 200000; ++k) {
        float x;
        const uint32_t bits = rnd();
        memcpy(&x, &bits, 4);
        (void)orc_f32_to_f16(x);
        (void)orc_f32_to_bf16(x);
    }
    for (int dt = 0; dt < 3; ++dt)
        for (int64_t n = 0; n < 40; ++n) {
            float* x = (float*)values(n, 0, 3.0f);
            void* y = xmalloc((size_t)n * esize(dt));
            float* z = (float*)xmalloc((size_t)n * 4);
            orc_cast_from_f32(x, dt, y, n);
            orc_cast_to_f32(y, dt, z, n);
            orc_cast(x, dt, y, n);
            free(x);
            free(y);
            free(z);
        }
}

static void check_layout(void) {
    for (int32_t world = 1; world <= 9; ++world)
        for (int trial = 0; trial < 40; ++trial) {
            const int32_t T = (int32_t)(rnd() % 7);
            int64_t* numels = (int64_t*)xmalloc(sizeof(int64_t) * (size_t)T);
            int64_t* offs = (int64_t*)xmalloc(sizeof(int64_t) * (size_t)T);
            int64_t total = 0;
            for (int32_t k = 0; k < T; ++k) total += numels[k] = (int64_t)(rnd() % 37);
            const int64_t padded = orc_padded_numel(total, world);
            if (padded < total || padded % world || padded - total >= world) fail("padded numel");
            orc_offsets(numels, T, offs);
            for (int dt = 0; dt < 3; ++dt) {
                const int64_t es = esize(dt);
                void** srcs = (void**)xmalloc(sizeof(void*) * (size_t)T);
                void** outs = (void**)xmalloc(sizeof(void*) * (size_t)T);
                for (int32_t k = 0; k < T; ++k) {
                    srcs[k] = values(numels[k], dt, 1.0f);
                    outs[k] = xmalloc((size_t)(numels[k] * es));
                }
                unsigned char* flat = (unsigned char*)xmalloc((size_t)(padded * es));
                orc_flatten_pad((const void* const*)srcs, numels, T, es, padded, flat);
                for (int64_t b = total * es; b < padded * es; ++b)
                    if (flat[b]) fail("padding is not +0");
                orc_unflatten(flat, numels, T, es, outs);
                for (int32_t k = 0; k < T; ++k) {
                    if (memcmp(srcs[k], outs[k], (size_t)(numels[k] * es))) fail("flatten / unflatten round trip");
                    free(srcs[k]);
                    free(outs[k]);
                }
                /* the gather of the shards is the flat buffer */
                const int64_t S = padded / world;
                void** shards = (void**)xmalloc(sizeof(void*) * (size_t)world);
                for (int32_t q = 0; q < world; ++q) {
                    shards[q] = xmalloc((size_t)(S * es));
                    memcpy(shards[q], flat + q * S * es, (size_t)(S * es));
                }
                unsigned char* full = (unsigned char*)xmalloc((size_t)(padded * es));
                orc_gather((const void* const*)shards, world, S, es, full);
                if (memcmp(full, flat, (size_t)(padded * es))) fail("gather");
                for (int32_t q = 0; q < world; ++q) free(shards[q]);
                free(shards);
                free(full);
                free(flat);
                free(srcs);
                free(outs);
            }
            free(numels);
            free(offs);
        }
}

static void check_reduction(void) {
    const int32_t worlds[] = {1, 2, 3, 8, 16};
    const int64_t shards[] = {0, 1, 7, 8, 9, 65, 1003};
    for (size_t wi = 0; wi < sizeof worlds / sizeof *worlds; ++wi)
        for (size_t si = 0; si < sizeof shards / sizeof *shards; ++si)
            for (int dt = 0; dt < 3; ++dt)
                for (int f32r = 0; f32r < 2; ++f32r) {
                    const int32_t N = worlds[wi];
                    const int64_t S = shards[si], P = (int64_t)N * S;
                    const int od = (f32r || dt == 0) ? 0 : dt;
                    void** g = (void**)xmalloc(sizeof(void*) * (size_t)N);
                    for (int32_t q = 0; q < N; ++q) g[q] = values(P, dt, 1e-3f);
                    unsigned char* ar = (unsigned char*)xmalloc((size_t)(P * esize(od)));
                    orc_all_reduce((const void* const*)g, N, P, dt, f32r, ar);
                    for (int32_t r = 0; r < N; ++r) {
                        unsigned char* rs = (unsigned char*)xmalloc((size_t)(S * esize(od)));
                        orc_reduce_scatter((const void* const*)g, N, r, S, dt, f32r, rs);
                        /* AG(RS) == AR on the bit patterns (NaN payloads included) */
                        if (memcmp(rs, ar + r * S * esize(od), (size_t)(S * esize(od)))) fail("RS != block of AR");
                        free(rs);
                    }
                    for (int32_t q = 0; q < N; ++q) free(g[q]);
                    free(g);
                    free(ar);
                }
}

static void check_optimizers(void) {
    const int64_t sizes[] = {0, 1, 7, 8, 9, 63, 1003};
    const int64_t steps[] = {1, 2, 10, 1000};
    float sc[8];
    for (size_t ni = 0; ni < sizeof sizes / sizeof *sizes; ++ni)
        for (size_t ti = 0; ti < sizeof steps / sizeof *steps; ++ti) {
            const int64_t n = sizes[ni];
            const orc_hp hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, steps[ti]};
            orc_adamw_scalars(&hp, sc);
            float* p = (float*)values(n, 0, 0.02f);
            float* m = (float*)values(n, 0, 1e-4f);
            float* v = (float*)values(n, 0, 1e-4f);
            float* g = (float*)values(n, 0, 1e-3f);
            orc_adamw(p, m, v, g, n, &hp);
            for (int dt = 1; dt < 3; ++dt) {
                uint16_t* p16 = (uint16_t*)values(n, dt, 0.02f);
                uint16_t* m16 = (uint16_t*)values(n, dt, 1e-4f);
                uint16_t* v16 = (uint16_t*)values(n, dt, 1e-4f);
                orc_adamw16(p16, m16, v16, dt, g, n, &hp);
                free(p16);
                free(m16);
                free(v16);
            }
            const orc_opt sgd = {1e-2f, 1e-4f, 0.9f, 0.1f, 0, 0, 0, 0, 0, steps[ti]};
            const orc_opt nes = {1e-2f, 0.0f, 0.9f, 0.0f, 0, 0, 0, 0, 1, steps[ti]};
            const orc_opt plain = {1e-2f, 1e-4f, 0.0f, 0.0f, 0, 0, 0, 0, 0, steps[ti]};
            const orc_opt amax = {2e-3f, 0.01f, 0, 0, 0.9f, 0.999f, 1e-8f, 0, 0, steps[ti]};
            const orc_opt adel = {1.0f, 0.01f, 0, 0, 0, 0, 1e-6f, 0.9f, 0, steps[ti]};
            orc_sgd(p, m, g, n, &sgd);
            orc_sgd(p, m, g, n, &nes);
            orc_sgd(p, NULL, g, n, &plain);   /* no momentum: the buffer is never touched */
            orc_adamax(p, m, v, g, n, &amax);
            orc_adadelta(p, m, v, g, n, &adel);
            free(p);
            free(m);
            free(v);
            free(g);
        }
    double out[3];
    orc_memory_per_worker(855638016, 8, 1, 1, 1, 2, 2, 12, out);
    if (!(out[0] > 0 && out[1] > 0 && out[2] > 0)) fail("memory per worker");
}

int main(void) {
    check_formats();
    check_layout();
    check_reduction();
    check_optimizers();
    printf("oracle sanitizer checks: ok\n");
    return 0;
}
