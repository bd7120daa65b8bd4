/*
 * fsdp_oracle.c -- plain, slow, single-threaded CPU oracle for the FSDP
 * flat-parameter shard pipeline.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no source, header, table or
 * helper with the HIP path.
 *
 * Sources (five web pages on FSDP; each function cites the passage it follows):
 *   [TR]  "Fully Sharded Data Parallel: faster AI training with fewer GPUs"
 *         (techreport.ngo)
 *   [P3]  "FSDP (Fully Sharded Data Parallel)" (vanos001 placement-prep notes)
 *   [P4]  "fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战指南" (zskr.cn)
 *   [P5]  "Data Parallelism" (vanos001 placement-prep notes)
 *
 * Arithmetic rules (the pages fix the precision of the master weights and of
 * the --fp32-reduce-scatter reduction as fp32, so fp32 is the working type):
 *   - every float operation below is ONE IEEE-754 binary32 operation with
 *     round-to-nearest-even; build with -O2 -ffp-contract=off (no FMA
 *     contraction), no -ffast-math, no flush-to-zero;
 *   - host scalars of the optimizer are computed in double and rounded once.
 *
 * Dtype codes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16 (bfloat16).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* ------------------------------------------------------------------------ */
/* Number formats.  Written from the IEEE-754 / bfloat16 encodings.          */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* m >> s rounded to nearest, ties to even (exact integer arithmetic). */
static uint64_t rne_shift(uint64_t m, int s)
{
    if (s <= 0) return m;
    if (s >= 64) return 0;
    uint64_t q = m >> s;
    uint64_t r = m & ((((uint64_t)1) << s) - 1);
    uint64_t half = ((uint64_t)1) << (s - 1);
    if (r > half || (r == half && (q & 1))) q += 1;
    return q;
}

/* fp32 -> IEEE binary16, round to nearest even, with subnormals, overflow to
 * infinity, and NaN kept a (quiet) NaN of the same sign. */
uint16_t orc_f32_to_f16(float x)
{
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
    if (a == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);
    int efield = (int)(a >> 23);
    uint64_t m24;   /* significand with the implicit bit, value = m24 * 2^(e-23) */
    int e;
    if (efield == 0) { m24 = a & 0x7fffffu; e = -126; }
    else { m24 = (a & 0x7fffffu) | 0x800000u; e = efield - 127; }
    if (m24 == 0) return sign;
    if (e >= -14) {
        /* binary16 normal range: keep 11 significant bits. */
        uint64_t q = rne_shift(m24, 13);          /* in [0x400, 0x800] */
        int64_t h = ((int64_t)(e + 15) << 10) + ((int64_t)q - 0x400);
        if (h >= 0x7c00) return (uint16_t)(sign | 0x7c00u);  /* overflow */
        return (uint16_t)(sign | (uint16_t)h);
    }
    /* binary16 subnormal: unit 2^-24, q = value / 2^-24 = m24 * 2^(e+1). */
    int s = -(e + 1);
    uint64_t q = rne_shift(m24, s);               /* q == 0x400 is the smallest normal */
    return (uint16_t)(sign | (uint16_t)q);
}

float orc_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t ef = ((uint32_t)h >> 10) & 0x1fu;
    uint32_t mf = (uint32_t)h & 0x3ffu;
    if (ef == 0x1f) return bits_f32(sign | 0x7f800000u | (mf << 13));
    if (ef == 0) {
        /* subnormal: mf * 2^-24, exact in fp32 */
        float v = (float)mf * 0x1p-24f;
        return sign ? -v : v;
    }
    return bits_f32(sign | ((ef - 15 + 127) << 23) | (mf << 13));
}

/* fp32 -> bfloat16, round to nearest even.  bfloat16 is the upper half of the
 * fp32 encoding and the fp32 magnitude encoding is monotone with uniform spacing
 * inside each binade, so rounding the 31-bit magnitude pattern at bit 16 is
 * rounding the value (the carry walks into the exponent, and past the largest
 * finite value into infinity). */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7fc0u | ((a >> 16) & 0x7fu));
    return (uint16_t)(sign | (uint16_t)rne_shift(a, 16));
}

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

static float load_as_f32(const void* base, int dt, int64_t i)
{
    if (dt == ORC_F32) return ((const float*)base)[i];
    if (dt == ORC_F16) return orc_f16_to_f32(((const uint16_t*)base)[i]);
    return orc_bf16_to_f32(((const uint16_t*)base)[i]);
}

/* round fp32 to 16-bit format dt, returned as fp32 */
static float round_to(int dt, float x)
{
    if (dt == ORC_F16) return orc_f16_to_f32(orc_f32_to_f16(x));
    if (dt == ORC_BF16) return orc_bf16_to_f32(orc_f32_to_bf16(x));
    return x;
}

static void store_from_f32(void* base, int dt, int64_t i, float x)
{
    if (dt == ORC_F32) ((float*)base)[i] = x;
    else if (dt == ORC_F16) ((uint16_t*)base)[i] = orc_f32_to_f16(x);
    else ((uint16_t*)base)[i] = orc_f32_to_bf16(x);
}

int64_t orc_dtype_size(int dt) { return dt == ORC_F32 ? 4 : 2; }

/* Bulk conversions (used to pin the converters exhaustively). */
void orc_cast_from_f32(const float* src, int dt, void* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) store_from_f32(dst, dt, i, src[i]);
}
void orc_cast_to_f32(const void* src, int dt, float* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = load_as_f32(src, dt, i);
}

/* ------------------------------------------------------------------------ */
/* Layout: flatten, pad, offsets, unflatten.                                 */
/* [TR] "Adoption paths for FSDP" (advanced concern 3): a wrapped module's   */
/* parameters become one flat tensor.  The flat buffer is padded at the tail */
/* with +0 to a multiple of the world size so it splits into N equal shards. */
/* ------------------------------------------------------------------------ */

int64_t orc_padded_numel(int64_t total, int32_t world)
{
    if (world <= 0) return -1;
    return ((total + world - 1) / world) * world;
}

/* offsets[k] = numel_0 + ... + numel_{k-1} */
void orc_offsets(const int64_t* numels, int32_t n_tensors, int64_t* offsets)
{
    int64_t off = 0;
    for (int32_t k = 0; k < n_tensors; ++k) { offsets[k] = off; off += numels[k]; }
}

/* flat[off_k + i] = T_k[i] for every tensor in caller order, then +0 up to
 * padded_numel.  Elements are copied as raw bytes of elem_size. */
void orc_flatten_pad(const void* const* srcs, const int64_t* numels, int32_t n_tensors,
                     int64_t elem_size, int64_t padded_numel, void* flat)
{
    unsigned char* out = (unsigned char*)flat;
    int64_t pos = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        const unsigned char* in = (const unsigned char*)srcs[k];
        for (int64_t b = 0; b < numels[k] * elem_size; ++b) out[pos * elem_size + b] = in[b];
        pos += numels[k];
    }
    for (int64_t b = pos * elem_size; b < padded_numel * elem_size; ++b) out[b] = 0;
}

/* tensor k = flat[off_k : off_k + numel_k], copied out into dsts[k]. */
void orc_unflatten(const void* flat, const int64_t* numels, int32_t n_tensors,
                   int64_t elem_size, void* const* dsts)
{
    const unsigned char* in = (const unsigned char*)flat;
    int64_t pos = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        unsigned char* out = (unsigned char*)dsts[k];
        for (int64_t b = 0; b < numels[k] * elem_size; ++b) out[b] = in[pos * elem_size + b];
        pos += numels[k];
    }
}

/* ------------------------------------------------------------------------ */
/* Gradient averaging.                                                       */
/* [P5] "The Basic Protocol": the all-reduce averages the workers' gradients */
/* as G_avg = (1/N) * sum_i G_i.  [TR] figure "All-reduce as a combination   */
/* of reduce-scatter and all-gather": the reduce-scatter sums equal blocks   */
/* by rank index, so rank r receives block r of the average.                 */
/* [P4] flag table: --fp32-reduce-scatter (default off) reduces in fp32.     */
/*                                                                           */
/* Element j, ranks summed left to right in rank order 0..N-1:               */
/*   fp32 mode:  acc = G_0[j]; acc = acc + G_q[j]; avg = acc / N   (fp32)    */
/*   16-bit mode (grad format d): a = G_0[j]; a = RNE_d(a + G_q[j]);         */
/*               avg = RNE_d(a / N)                                          */
/* The output covers elements [begin, begin + count).  out is fp32 in fp32   */
/* mode and format d in 16-bit mode.                                         */
/* ------------------------------------------------------------------------ */

void orc_grad_average(const void* const* grads, int32_t world, int64_t begin, int64_t count,
                      int grad_dt, int fp32_reduce, void* out)
{
    int fp32_mode = fp32_reduce || grad_dt == ORC_F32;
    for (int64_t i = 0; i < count; ++i) {
        int64_t j = begin + i;
        if (fp32_mode) {
            float acc = load_as_f32(grads[0], grad_dt, j);
            for (int32_t q = 1; q < world; ++q) acc = acc + load_as_f32(grads[q], grad_dt, j);
            ((float*)out)[i] = acc / (float)world;
        } else {
            float a = load_as_f32(grads[0], grad_dt, j);
            for (int32_t q = 1; q < world; ++q) a = round_to(grad_dt, a + load_as_f32(grads[q], grad_dt, j));
            store_from_f32(out, grad_dt, i, a / (float)world);
        }
    }
}

/* All-reduce: the average over the whole padded buffer. */
void orc_all_reduce(const void* const* grads, int32_t world, int64_t padded_numel,
                    int grad_dt, int fp32_reduce, void* out)
{
    orc_grad_average(grads, world, 0, padded_numel, grad_dt, fp32_reduce, out);
}

/* Reduce-scatter for one rank: block `rank` (S = padded_numel / world) of the
 * average. */
void orc_reduce_scatter(const void* const* grads, int32_t world, int32_t rank, int64_t shard_numel,
                        int grad_dt, int fp32_reduce, void* out)
{
    orc_grad_average(grads, world, (int64_t)rank * shard_numel, shard_numel, grad_dt, fp32_reduce, out);
}

/* ------------------------------------------------------------------------ */
/* AdamW on one shard.                                                       */
/* [P5] "The Basic Protocol" gives the update only as W = W - lr*Adam(G,m,v);*/
/* [P4] "限制与兼容性说明" lists AdamW among the pointwise optimizers FSDP   */
/* supports and "工作原理" says each rank updates only its own shard.        */
/* The update is the published AdamW: Adam with bias correction (Kingma &    */
/* Ba 2015, Algorithm 1) and weight decay decoupled from the gradient        */
/* (Loshchilov & Hutter 2019, Algorithm 2), eps added after the square root, */
/* decay factor (1 - lr*wd).  Reading fixed on these points because the      */
/* pages do not write the formula.                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} orc_hp;

/* out: [decay, beta1, 1-beta1, beta2, 1-beta2, step_size, sqrt(bias2), eps] */
void orc_adamw_scalars(const orc_hp* hp, float* out)
{
    double b1 = (double)hp->beta1, b2 = (double)hp->beta2, lr = (double)hp->lr;
    double t = (double)hp->step;
    double bias1 = 1.0 - pow(b1, t);     /* 1 - beta1^t */
    double bias2 = 1.0 - pow(b2, t);     /* 1 - beta2^t */
    out[0] = (float)(1.0 - lr * (double)hp->weight_decay);
    out[1] = hp->beta1;
    out[2] = 1.0f - hp->beta1;           /* exact (Sterbenz) for beta1 in [0.5, 1] */
    out[3] = hp->beta2;
    out[4] = 1.0f - hp->beta2;
    out[5] = (float)(lr / bias1);
    out[6] = (float)sqrt(bias2);
    out[7] = hp->eps;
}

/* One AdamW step over n elements: p, m, v updated in place from fp32 grads g.
 *   p <- p * (1 - lr*wd)
 *   m <- beta1*m + (1-beta1)*g
 *   v <- beta2*v + (1-beta2)*g*g
 *   p <- p - (lr / (1-beta1^t)) * m / (sqrt(v)/sqrt(1-beta2^t) + eps)          */
void orc_adamw(float* p, float* m, float* v, const float* g, int64_t n, const orc_hp* hp)
{
    float s[8];
    orc_adamw_scalars(hp, s);
    const float decay = s[0], b1 = s[1], omb1 = s[2], b2 = s[3], omb2 = s[4];
    const float step_size = s[5], bc2_sqrt = s[6], eps = s[7];
    for (int64_t i = 0; i < n; ++i) {
        float gi = g[i];
        float p1 = p[i] * decay;
        float m1 = (b1 * m[i]) + (omb1 * gi);
        float v1 = (b2 * v[i]) + (omb2 * (gi * gi));
        float den = (sqrtf(v1) / bc2_sqrt) + eps;
        float p2 = p1 - (step_size * (m1 / den));
        p[i] = p2;
        m[i] = m1;
        v[i] = v1;
    }
}

/* ------------------------------------------------------------------------ */
/* AdamW with 16-bit state.  [P3] "Mixed Precision and FSDP": without an fp32 */
/* master copy the parameters and the Adam state are kept in bf16; [TR]      */
/* "Adoption paths for FSDP", concern 4: FP16 master weights.  Reading: the  */
/* update is the fp32 AdamW above applied to the widened 16-bit values, and  */
/* each new value is rounded once to the state format; the rounded parameter */
/* is also the compute copy.  p, m, v are 16-bit patterns of format state_dt.*/
/* ------------------------------------------------------------------------ */

void orc_adamw16(uint16_t* p, uint16_t* m, uint16_t* v, int state_dt, const float* g, int64_t n,
                 const orc_hp* hp)
{
    float s[8];
    orc_adamw_scalars(hp, s);
    const float decay = s[0], b1 = s[1], omb1 = s[2], b2 = s[3], omb2 = s[4];
    const float step_size = s[5], bc2_sqrt = s[6], eps = s[7];
    for (int64_t i = 0; i < n; ++i) {
        float pi = load_as_f32(p, state_dt, i), mi = load_as_f32(m, state_dt, i), vi = load_as_f32(v, state_dt, i);
        float gi = g[i];
        float p1 = pi * decay;
        float m1 = (b1 * mi) + (omb1 * gi);
        float v1 = (b2 * vi) + (omb2 * (gi * gi));
        float den = (sqrtf(v1) / bc2_sqrt) + eps;
        float p2 = p1 - (step_size * (m1 / den));
        store_from_f32(p, state_dt, i, p2);
        store_from_f32(m, state_dt, i, m1);
        store_from_f32(v, state_dt, i, v1);
    }
}

/* ------------------------------------------------------------------------ */
/* Other pointwise optimizers.  [P4] "限制与兼容性说明": FSDP works with the  */
/* pointwise optimizers (Adam, AdamW, Adadelta, Adamax, SGD and the like)    */
/* and not with Adagrad, Adafactor or LAMB; the pages write none of their    */
/* updates.  Reading: the published algorithms in the form torch.optim       */
/* documents them (SGD with heavy-ball momentum, dampening and the Nesterov  */
/* variant, the buffer starting as the first gradient; Adamax, the infinity- */
/* norm Adam of Kingma & Ba 2015, section 7.1; Adadelta, Zeiler 2012,        */
/* Algorithm 1, with a learning-rate factor), their weight decay added to    */
/* the gradient (L2) and skipped when it is 0.  Scalars as for AdamW: fp32   */
/* hyper-parameters, 1 - beta etc. one fp32 operation, bias terms in double  */
/* rounded once.                                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    float lr, weight_decay;
    float momentum, dampening;   /* SGD */
    float beta1, beta2;          /* Adamax */
    float eps;                   /* Adamax, Adadelta */
    float rho;                   /* Adadelta */
    int32_t nesterov;            /* SGD */
    int64_t step;                /* t >= 1 */
} orc_opt;

/* The gradient with L2 weight decay: d = g + wd*p (just g when wd == 0). */
static float l2_grad(float g, float p, float wd)
{
    return wd != 0.0f ? g + (wd * p) : g;
}

/* SGD.  momentum == 0:  p <- p - lr*d.
 * momentum mu > 0:  b <- d at t = 1, else b <- mu*b + (1 - dampening)*d;
 *                   d <- d + mu*b (Nesterov) or d <- b;  p <- p - lr*d.
 * buf (n elements) is read and written only when mu > 0 (may be NULL else). */
void orc_sgd(float* p, float* buf, const float* g, int64_t n, const orc_opt* o)
{
    const float lr = o->lr, wd = o->weight_decay, mu = o->momentum;
    const float omd = 1.0f - o->dampening;
    for (int64_t i = 0; i < n; ++i) {
        float d = l2_grad(g[i], p[i], wd);
        if (mu != 0.0f) {
            float b = o->step == 1 ? d : (mu * buf[i]) + (omd * d);
            buf[i] = b;
            d = o->nesterov ? d + (mu * b) : b;
        }
        p[i] = p[i] - (lr * d);
    }
}

/* Adamax.  m <- beta1*m + (1-beta1)*d;  u <- max(beta2*u, |d| + eps) (NaN if
 * either is NaN);  p <- p - (lr / (1 - beta1^t)) * (m / u). */
void orc_adamax(float* p, float* m, float* u, const float* g, int64_t n, const orc_opt* o)
{
    const float b1 = o->beta1, omb1 = 1.0f - o->beta1, b2 = o->beta2, eps = o->eps, wd = o->weight_decay;
    const float clr = (float)((double)o->lr / (1.0 - pow((double)o->beta1, (double)o->step)));
    for (int64_t i = 0; i < n; ++i) {
        float d = l2_grad(g[i], p[i], wd);
        float m1 = (b1 * m[i]) + (omb1 * d);
        float a = b2 * u[i], b = fabsf(d) + eps;
        float u1 = (isnan(a) || isnan(b)) ? NAN : (b > a ? b : a);
        m[i] = m1;
        u[i] = u1;
        p[i] = p[i] - (clr * (m1 / u1));
    }
}

/* Adadelta.  v <- rho*v + (1-rho)*d*d;  delta = sqrt(acc + eps)/sqrt(v + eps) * d;
 * acc <- rho*acc + (1-rho)*delta*delta;  p <- p - lr*delta.
 * v is the running mean of squared gradients, acc that of squared updates. */
void orc_adadelta(float* p, float* v, float* acc, const float* g, int64_t n, const orc_opt* o)
{
    const float rho = o->rho, omr = 1.0f - o->rho, eps = o->eps, lr = o->lr, wd = o->weight_decay;
    for (int64_t i = 0; i < n; ++i) {
        float d = l2_grad(g[i], p[i], wd);
        float v1 = (rho * v[i]) + (omr * (d * d));
        float delta = (sqrtf(acc[i] + eps) / sqrtf(v1 + eps)) * d;
        float a1 = (rho * acc[i]) + (omr * (delta * delta));
        v[i] = v1;
        acc[i] = a1;
        p[i] = p[i] - (lr * delta);
    }
}

/* ------------------------------------------------------------------------ */
/* Cast to the compute dtype.  [P3] "Mixed Precision and FSDP": fp32 master  */
/* weights with a 16-bit compute copy; [P4] fsdp_config mapping:             */
/* compute_dtype is fp16 under --fp16 and fp32 otherwise.                    */
/* ------------------------------------------------------------------------ */

void orc_cast(const float* master, int compute_dt, void* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) store_from_f32(out, compute_dt, i, master[i]);
}

/* ------------------------------------------------------------------------ */
/* All-gather unshard.  [P3] "The Per-Layer Communication" and [TR] "From    */
/* all-reduce to sharded parameters": before compute every worker gathers    */
/* the full parameters from the shards; full[q*S + i] = shard_q[i].          */
/* ------------------------------------------------------------------------ */

void orc_gather(const void* const* shards, int32_t world, int64_t shard_numel, int64_t elem_size,
                void* full)
{
    unsigned char* out = (unsigned char*)full;
    for (int32_t q = 0; q < world; ++q) {
        const unsigned char* in = (const unsigned char*)shards[q];
        int64_t base = (int64_t)q * shard_numel * elem_size;
        for (int64_t b = 0; b < shard_numel * elem_size; ++b) out[base + b] = in[b];
    }
}

/* ------------------------------------------------------------------------ */
/* Per-worker memory.  [P3] "The Sharding Scheme": without sharding a worker */
/* holds parameters P, gradients P and optimizer state 4P (6P in total); with*/
/* full sharding each class is divided by N (6P/N).  [P5] "ZeRO Stages":     */
/* stage 1 shards only the optimizer state, stage 2 also the gradients,      */
/* stage 3 everything.  A sharded class holds one shard of the padded flat   */
/* buffer.  Byte weights per element are arguments; in the pages' units      */
/* (bf16 parameters) they are 2 : 2 : 8.                                     */
/* out[0..2] = parameter, gradient, optimizer-state bytes on one worker.     */
/* ------------------------------------------------------------------------ */

void orc_memory_per_worker(int64_t numel, int32_t world, int shard_params, int shard_grads,
                           int shard_optim, double param_bytes, double grad_bytes,
                           double optim_bytes, double* out)
{
    double full = (double)numel;
    double shard = (double)orc_padded_numel(numel, world) / (double)world;
    out[0] = (shard_params ? shard : full) * param_bytes;
    out[1] = (shard_grads ? shard : full) * grad_bytes;
    out[2] = (shard_optim ? shard : full) * optim_bytes;
}
