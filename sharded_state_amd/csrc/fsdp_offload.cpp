// fsdp_offload.cpp -- the CPU-offload optimizer step of libfsdp_shard.so.
//
// "Fully Sharded Data Parallel: faster AI training with fewer GPUs"
// (techreport.ngo), section "Adoption paths for FSDP", fairseq: --cpu-offload
// moves the optimizer state and the FP32 model copy to the CPU, where the Adam
// step runs.  "FSDP (Fully Sharded Data Parallel)" (vanos001 notes), section
// "CPU Offloading": parameters and optimizer state live in CPU RAM and cross
// PCIe every step.  "fairseq 中的 FSDP 实战指南", flag table (--cpu-offload) and
// the single-GPU example: the optimizer step (Adam) runs on the CPU.
//
// fsdp_host_adamw is the CPU kernel: the same fp32 operation sequence as the
// GPU kernels (separate multiply and add, correctly rounded divide and square
// root, no flush-to-zero), eight lanes at a time with AVX2 when the host has it
// (F16C for binary16), split over a pool of worker threads.
// fsdp_offload_step_units chains, for a batch of units, the device
// reduce-scatter, the device-to-host copy of each gradient shard, the host
// AdamW and the host-to-device copy of each compute shard.  All device work and
// device-to-host copies are enqueued first; the host threads then take
// (chunk, part) work items in order from one queue, each chunk as soon as its
// copy has landed, and whoever finishes a chunk's last part enqueues its copy
// back to the device (on a second stream when one is given, so the two copy
// directions run at once).  No barrier separates chunks or units.

#include <hip/hip_runtime.h>
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <memory>
#include <string>
#include <mutex>
#include <thread>
#include <vector>

#include "fsdp_internal.h"
#include "fsdp_kernels.h"
#include "fsdp_pool.h"
#include "fsdp_shard.h"

namespace {

using fsdp::Pool;

// ------------------------------------------------------------------ formats (host)
inline uint32_t fbits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
inline float bitsf(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

// binary16 <-> binary32, scalar (round to nearest even, subnormals, NaN kept NaN)
inline float h2f(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0x1f) return bitsf(sign | 0x7f800000u | (m << 13));
    if (e == 0) {
        if (m == 0) return bitsf(sign);
        const float v = std::ldexp((float)m, -24);   // exact
        return sign ? -v : v;
    }
    return bitsf(sign | ((e + 112u) << 23) | (m << 13));
}

inline uint16_t f2h(float x) {
    const uint32_t u = fbits(x), sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);        // rounds to infinity
    if (a >= 0x38800000u) {                                          // normal binary16
        const uint32_t mant = a + ((a >> 13) & 1u) + 0xfffu;         // RNE at bit 13
        return (uint16_t)(sign | ((mant - 0x38000000u) >> 13));
    }
    if (a < 0x33000001u) return (uint16_t)sign;                     // below half the smallest subnormal
    // subnormal binary16: value / 2^-24 rounded to nearest even
    const uint32_t e = a >> 23, m = (a & 0x7fffffu) | 0x800000u;
    const int shift = 126 - (int)e;                                  // 14 .. 24
    uint32_t q = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
}

inline float b2f(uint16_t h) { return bitsf((uint32_t)h << 16); }
inline uint16_t f2b(float x) {
    const uint32_t u = fbits(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

inline float load_g(const void* g, int dt, int64_t i) {
    if (dt == FSDP_F32) return ((const float*)g)[i];
    if (dt == FSDP_F16) return h2f(((const uint16_t*)g)[i]);
    return b2f(((const uint16_t*)g)[i]);
}

inline void store_c(void* c, int dt, int64_t i, float x) {
    if (dt == FSDP_F32) ((float*)c)[i] = x;
    else if (dt == FSDP_F16) ((uint16_t*)c)[i] = f2h(x);
    else ((uint16_t*)c)[i] = f2b(x);
}

using Scalars = fsdp::AdamScalars;

// ------------------------------------------------------------------ kernels (host)
void adamw_scalar(float* p, float* m, float* v, const void* g, int gdt, void* c, int cdt, int64_t lo, int64_t hi,
                  const Scalars& s) {
    for (int64_t i = lo; i < hi; ++i) {
        const float gi = load_g(g, gdt, i);
        const float p1 = p[i] * s.decay;
        const float m1 = (s.b1 * m[i]) + (s.omb1 * gi);
        const float v1 = (s.b2 * v[i]) + (s.omb2 * (gi * gi));
        const float den = (std::sqrt(v1) / s.bc2_sqrt) + s.eps;
        const float p2 = p1 - (s.step_size * (m1 / den));
        p[i] = p2;
        m[i] = m1;
        v[i] = v1;
        if (c) store_c(c, cdt, i, p2);
    }
}

__attribute__((target("avx2,f16c"))) inline __m256 load8_g(const void* g, int dt, int64_t i) {
    if (dt == FSDP_F32) return _mm256_loadu_ps((const float*)g + i);
    const __m128i h = _mm_loadu_si128((const __m128i*)((const uint16_t*)g + i));
    if (dt == FSDP_F16) return _mm256_cvtph_ps(h);                   // exact
    return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
}

// The compute copy is written once and read next by the device's copy engine,
// so with STREAM (8 elements aligned to their own size) it is written with
// non-temporal stores: no read-for-ownership of the destination lines.
template <bool STREAM>
__attribute__((target("avx2,f16c"))) inline void put16(void* dst, __m128i x) {
    if constexpr (STREAM) _mm_stream_si128((__m128i*)dst, x);
    else _mm_storeu_si128((__m128i*)dst, x);
}

template <bool STREAM>
__attribute__((target("avx2,f16c"))) inline void store8_c(void* c, int dt, int64_t i, __m256 x) {
    if (dt == FSDP_F32) {
        if constexpr (STREAM) _mm256_stream_ps((float*)c + i, x);
        else _mm256_storeu_ps((float*)c + i, x);
    } else if (dt == FSDP_F16) {
        put16<STREAM>((uint16_t*)c + i, _mm256_cvtps_ph(x, _MM_FROUND_TO_NEAREST_INT));
    } else {
        // bfloat16: round the encoding at bit 16 to nearest even; NaN -> quiet NaN
        const __m256i u = _mm256_castps_si256(x);
        const __m256i a = _mm256_and_si256(u, _mm256_set1_epi32(0x7fffffff));
        const __m256i nan = _mm256_cmpgt_epi32(a, _mm256_set1_epi32(0x7f800000));
        const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(1));
        __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, _mm256_set1_epi32(0x7fff)), lsb), 16);
        const __m256i q = _mm256_or_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(0x40));
        r = _mm256_blendv_epi8(r, q, nan);
        // pack the low 16 bits of the 8 lanes
        const __m128i lo = _mm256_castsi256_si128(r), hi = _mm256_extracti128_si256(r, 1);
        const __m128i shuf = _mm_setr_epi8(0, 1, 4, 5, 8, 9, 12, 13, -1, -1, -1, -1, -1, -1, -1, -1);
        const __m128i pl = _mm_shuffle_epi8(lo, shuf), ph = _mm_shuffle_epi8(hi, shuf);
        put16<STREAM>((uint16_t*)c + i, _mm_unpacklo_epi64(pl, ph));
    }
}

template <bool STREAM>
__attribute__((target("avx2,f16c"))) void adamw_avx2(float* p, float* m, float* v, const void* g, int gdt, void* c,
                                                      int cdt, int64_t lo, int64_t hi, const Scalars& s) {
    const __m256 decay = _mm256_set1_ps(s.decay), b1 = _mm256_set1_ps(s.b1), omb1 = _mm256_set1_ps(s.omb1);
    const __m256 b2 = _mm256_set1_ps(s.b2), omb2 = _mm256_set1_ps(s.omb2), step = _mm256_set1_ps(s.step_size);
    const __m256 bc2 = _mm256_set1_ps(s.bc2_sqrt), eps = _mm256_set1_ps(s.eps);
    int64_t i = lo;
    for (; i + 8 <= hi; i += 8) {
        const __m256 gi = load8_g(g, gdt, i);
        const __m256 p1 = _mm256_mul_ps(_mm256_loadu_ps(p + i), decay);
        const __m256 m1 = _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(m + i)), _mm256_mul_ps(omb1, gi));
        const __m256 v1 = _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(v + i)),
                                        _mm256_mul_ps(omb2, _mm256_mul_ps(gi, gi)));
        const __m256 den = _mm256_add_ps(_mm256_div_ps(_mm256_sqrt_ps(v1), bc2), eps);
        const __m256 p2 = _mm256_sub_ps(p1, _mm256_mul_ps(step, _mm256_div_ps(m1, den)));
        _mm256_storeu_ps(p + i, p2);
        _mm256_storeu_ps(m + i, m1);
        _mm256_storeu_ps(v + i, v1);
        if (c) store8_c<STREAM>(c, cdt, i, p2);
    }
    if constexpr (STREAM) _mm_sfence();   // the streamed lines are visible before anyone reads them
    adamw_scalar(p, m, v, g, gdt, c, cdt, i, hi, s);
}

void adamw_range(float* p, float* m, float* v, const void* g, int gdt, void* c, int cdt, int64_t lo, int64_t hi,
                 const Scalars& s) {
    // IEEE semantics for the whole range: no flush-to-zero, no denormals-are-zero
    const unsigned int csr = _mm_getcsr();
    _mm_setcsr(csr & ~0x8040u);
    static const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
    const uintptr_t c_lo = (uintptr_t)c + (uintptr_t)lo * (uintptr_t)fsdp::dt_size(cdt);
    const bool stream = c && c_lo % (8 * (uintptr_t)fsdp::dt_size(cdt)) == 0;
    if (avx2 && stream) adamw_avx2<true>(p, m, v, g, gdt, c, cdt, lo, hi, s);
    else if (avx2) adamw_avx2<false>(p, m, v, g, gdt, c, cdt, lo, hi, s);
    else adamw_scalar(p, m, v, g, gdt, c, cdt, lo, hi, s);
    _mm_setcsr(csr);
}

// ------------------------------------------------------------------ validation
struct Span {
    uintptr_t lo, hi;   // [lo, hi), non-empty
};

Span span(const void* p, int64_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }

// No two of the spans share a byte.
bool disjoint(std::vector<Span> v) {
    std::sort(v.begin(), v.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < v.size(); ++i)
        if (v[i].lo < v[i - 1].hi) return false;
    return true;
}

// No span of `ins` shares a byte with a span of `outs` (outs sorted by lo, disjoint).
bool apart(const std::vector<Span>& outs, const std::vector<Span>& ins) {
    for (const Span& x : ins) {
        auto it = std::upper_bound(outs.begin(), outs.end(), x.lo, [](uintptr_t a, const Span& b) { return a < b.lo; });
        if (it != outs.end() && it->lo < x.hi) return false;
        if (it != outs.begin() && std::prev(it)->hi > x.lo) return false;
    }
    return true;
}

int check_unit(const fsdp_offload_unit& u, int k, int32_t world, int32_t rank, int grad_dt, int64_t as, int64_t cs,
               bool scratch, std::vector<Span>& host, std::vector<Span>& dev_out, std::vector<Span>& dev_in) {
    if (u.shard_numel < 0) return fsdp::fail(FSDP_E_INVAL, "unit %d: shard_numel < 0", k);
    if (u.shard_numel > fsdp::kMaxElems / world)
        return fsdp::fail(FSDP_E_SIZE, "unit %d: shard_numel times world is too large", k);
    if (u.shard_numel == 0) return FSDP_OK;
    const int64_t S = u.shard_numel;
    if (scratch && u.grad_shard_dev)
        return fsdp::fail(FSDP_E_INVAL, "unit %d: grad_shard_dev must be NULL (the gradient chunks live in the "
                                        "library's scratch)", k);
    if (!u.master || !u.exp_avg || !u.exp_avg_sq || !u.rank_grads || (!scratch && !u.grad_shard_dev) ||
        !u.grad_shard_host || !u.compute_host || !u.compute_dev)
        return fsdp::fail(FSDP_E_INVAL, "unit %d: every buffer must be non-NULL", k);
    for (int q = 0; q < world; ++q) {
        if (!u.rank_grads[q]) return fsdp::fail(FSDP_E_INVAL, "unit %d: rank_grads[%d] is NULL", k, q);
        dev_in.push_back(span((const char*)u.rank_grads[q] + (int64_t)rank * S * fsdp::dt_size(grad_dt),
                              S * fsdp::dt_size(grad_dt)));
    }
    host.push_back(span(u.master, 4 * S));
    host.push_back(span(u.exp_avg, 4 * S));
    host.push_back(span(u.exp_avg_sq, 4 * S));
    host.push_back(span(u.grad_shard_host, as * S));
    host.push_back(span(u.compute_host, cs * S));
    if (!scratch) dev_out.push_back(span(u.grad_shard_dev, as * S));
    dev_out.push_back(span(u.compute_dev, cs * S));
    return FSDP_OK;
}

// ------------------------------------------------------------------ scratch
// The no-allocation variant (fsdp_offload_step_units_noalloc) reduces each
// chunk of a gradient shard into this file-scope device array and copies it to
// the host from there, instead of a caller's device gradient shard.  Every
// device holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels and copies take the
// address that scratch_setup obtained for the current device.
constexpr int64_t kScratchBytes = FSDP_OFFLOAD_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per device: the address of `scratch`, and events for the chunk copies (chunk
// c records ev[c % kScratchEvents]; a reused event only makes a worker wait for
// a later copy of the same stream) plus two that order the copy stream.
constexpr int kScratchEvents = 256;
constexpr int kMaxDevices = 64;
struct ScratchDevice {
    std::once_flag once;
    std::mutex mu;   // held for a whole call: calls on one device take the scratch in turn
    hipError_t err = hipSuccess;
    void* ptr = nullptr;
    hipEvent_t ev[kScratchEvents + 2] = {};
};
ScratchDevice g_scratch[kMaxDevices];

// Set-up, once per device with that device current (the first call of the
// variant on it): hipGetSymbolAddress for the device's copy of `scratch`, and
// the events.  Later calls create nothing.
int scratch_setup(ScratchDevice** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fsdp::hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fsdp::fail(FSDP_E_INVAL, "device %d: the scratch is kept for devices 0-%d only", dev, kMaxDevices - 1);
    ScratchDevice& d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
        for (int i = 0; i < kScratchEvents + 2 && d.err == hipSuccess; ++i)
            d.err = hipEventCreateWithFlags(&d.ev[i], hipEventDisableTiming);
    });
    if (d.err != hipSuccess) return fsdp::hip_fail(d.err, "scratch set-up (hipGetSymbolAddress / events)");
    *out = &d;
    return FSDP_OK;
}

// ------------------------------------------------------------------ the engine
struct Chunk {
    int unit;
    int64_t lo, n;         // elements [lo, lo + n) of the unit's shard
    int64_t first_item;    // work items [first_item, first_item + parts)
    int parts;
};

constexpr int64_t kPart = 1 << 15;   // elements per work item at most (128 KB of each fp32 stream)

int offload_units(const fsdp_offload_unit* units, int32_t n_units, int32_t world, int32_t rank, int grad_dt,
                  int32_t fp32_reduce, int compute_dt, int64_t chunk_numel, const fsdp_adamw_hp* hp,
                  int32_t n_threads, void* stream, void* copy_stream, const char* fn, bool use_scratch) {
    if (n_units < 0) return fsdp::fail(FSDP_E_INVAL, "%s: n_units < 0", fn);
    if (n_units > 0 && !units) return fsdp::fail(FSDP_E_INVAL, "%s: units is NULL", fn);
    if (world < 1 || world > FSDP_MAX_WORLD || rank < 0 || rank >= world)
        return fsdp::fail(FSDP_E_INVAL, "%s: world %d / rank %d out of range", fn, world, rank);
    if (!fsdp::valid_dtype(grad_dt) || !fsdp::valid_dtype(compute_dt))
        return fsdp::fail(FSDP_E_DTYPE, "%s: grad dtype %d / compute dtype %d unsupported", fn, grad_dt, compute_dt);
    int rc = fsdp::check_hp(fn, hp);
    if (rc) return rc;
    if (chunk_numel <= 0) chunk_numel = 4 << 20;
    if (chunk_numel > (int64_t(1) << 40)) return fsdp::fail(FSDP_E_INVAL, "%s: chunk_numel too large", fn);
    chunk_numel = (chunk_numel + 7) / 8 * 8;
    const int64_t part = std::min(kPart, chunk_numel);
    const int avg_dt = (fp32_reduce || grad_dt == FSDP_F32) ? FSDP_F32 : grad_dt;
    const int64_t as = fsdp::dt_size(avg_dt), cs = fsdp::dt_size(compute_dt);
    if (use_scratch && chunk_numel * as > kScratchBytes)
        return fsdp::fail(FSDP_E_SIZE, "%s: a chunk of %lld elements of %lld bytes exceeds the %lld-byte scratch "
                                       "(at most %lld elements per chunk)", fn, (long long)chunk_numel, (long long)as,
                          (long long)kScratchBytes, (long long)(kScratchBytes / as / 8 * 8));
    std::vector<Span> host, dev_out, dev_in;
    for (int k = 0; k < n_units; ++k) {
        rc = check_unit(units[k], k, world, rank, grad_dt, as, cs, use_scratch, host, dev_out, dev_in);
        if (rc) return rc;
    }
    if (!disjoint(host)) return fsdp::fail(FSDP_E_ALIAS, "%s: two host buffers overlap", fn);
    std::sort(dev_out.begin(), dev_out.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
    if (!disjoint(dev_out) || !apart(dev_out, dev_in))
        return fsdp::fail(FSDP_E_ALIAS, "%s: a device output overlaps another buffer", fn);

    // chunks and work items, in unit order
    std::vector<Chunk> chunks;
    int64_t items = 0;
    for (int k = 0; k < n_units; ++k)
        for (int64_t lo = 0; lo < units[k].shard_numel; lo += chunk_numel) {
            const int64_t n = std::min(chunk_numel, units[k].shard_numel - lo);
            const int parts = (int)((n + part - 1) / part);
            chunks.push_back(Chunk{k, lo, n, items, parts});
            items += parts;
        }
    if (chunks.empty()) return fsdp::ok();
    hipStream_t st = (hipStream_t)stream, cst = copy_stream ? (hipStream_t)copy_stream : st;

    std::vector<hipEvent_t> ready(chunks.size(), nullptr);
    hipEvent_t entry = nullptr, done = nullptr;
    ScratchDevice* sd = nullptr;
    std::unique_lock<std::mutex> scratch_lock;
    if (use_scratch) {
        // the device's scratch and its events: nothing is created after set-up.  The
        // lock is held until this call returns, by which time every chunk's copy out
        // of the scratch has landed (the host work waited for each), so a call from
        // another thread never finds the scratch or the events in use.
        rc = scratch_setup(&sd);
        if (rc) return rc;
        scratch_lock = std::unique_lock<std::mutex>(sd->mu);
        for (size_t c = 0; c < chunks.size(); ++c) ready[c] = sd->ev[c % kScratchEvents];
        if (cst != st) {
            entry = sd->ev[kScratchEvents];
            done = sd->ev[kScratchEvents + 1];
        }
    }
    struct Cleanup {
        std::vector<hipEvent_t>& ev;
        hipEvent_t& a;
        hipEvent_t& b;
        bool owned;
        hipStream_t st;
        bool finished = false;
        ~Cleanup() {
            if (!owned) {
                // the scratch's events stay with their device.  A call that ends in
                // an error may leave reduce-scatters into the scratch or copies out of
                // it on the stream: let them finish before the lock (released after
                // this) lets another call in
                if (!finished) (void)hipStreamSynchronize(st);
                return;
            }
            for (hipEvent_t x : ev)
                if (x) {
                    (void)hipEventSynchronize(x);
                    (void)hipEventDestroy(x);
                }
            if (a) (void)hipEventDestroy(a);
            if (b) (void)hipEventDestroy(b);
        }
    } cleanup{ready, entry, done, !use_scratch, st};
    hipError_t e = hipSuccess;
    if (!use_scratch) {
        for (size_t c = 0; c < chunks.size() && e == hipSuccess; ++c)
            e = hipEventCreateWithFlags(&ready[c], hipEventDisableTiming);
        if (e != hipSuccess) return fsdp::hip_fail(e, "event creation");
        if (cst != st && ((e = hipEventCreateWithFlags(&entry, hipEventDisableTiming)) != hipSuccess ||
                          (e = hipEventCreateWithFlags(&done, hipEventDisableTiming)) != hipSuccess))
            return fsdp::hip_fail(e, "event creation");
    }
    if (cst != st) {
        // the copy stream starts after the work already on `stream` (a reader of compute_dev)
        if ((e = hipEventRecord(entry, st)) != hipSuccess || (e = hipStreamWaitEvent(cst, entry, 0)) != hipSuccess)
            return fsdp::hip_fail(e, "copy stream ordering");
    }

    // 1. every unit's reduce-scatter and gradient copies to the host, in order
    size_t c = 0;
    const int64_t gs = fsdp::dt_size(grad_dt);
    std::vector<const void*> gp(world);
    (void)hipGetLastError();
    for (int k = 0; k < n_units; ++k) {
        const fsdp_offload_unit& u = units[k];
        if (u.shard_numel == 0) continue;
        if (!use_scratch) {
            rc = fsdp_reduce_scatter_local(u.rank_grads, world, rank, u.shard_numel, (fsdp_dtype)grad_dt,
                                           fp32_reduce, u.grad_shard_dev, stream);
            if (rc) return rc;
        }
        for (; c < chunks.size() && chunks[c].unit == k; ++c) {
            const Chunk& ch = chunks[c];
            const char* src = nullptr;
            if (!use_scratch) {
                src = (const char*)u.grad_shard_dev + ch.lo * as;
            } else {
                // this chunk's reduce-scatter into the scratch; stream order keeps
                // the next chunk's from overwriting it before its copy has run
                bool vec = true;
                for (int q = 0; q < world; ++q) {
                    gp[q] = (const char*)u.rank_grads[q] + ((int64_t)rank * u.shard_numel + ch.lo) * gs;
                    vec = vec && ((uintptr_t)gp[q] & 15) == 0;
                }
                fsdp::ReduceArgs a{};
                a.grads = gp.data();
                a.world = world;
                a.grad_dt = grad_dt;
                a.fp32_reduce = fp32_reduce != 0;
                a.S = ch.n;
                a.nvec = vec ? ch.n / 8 : 0;
                a.out = sd->ptr;
                a.rs = fsdp::reduce_scalars(world);
                a.cus = fsdp::cu_count();
                a.stream = stream;
                e = fsdp::launch_reduce_scatter(a);
                if (e != hipSuccess) return fsdp::hip_fail(e, "reduce-scatter launch");
                src = (const char*)sd->ptr;
            }
            e = hipMemcpyAsync((char*)u.grad_shard_host + ch.lo * as, src, ch.n * as, hipMemcpyDeviceToHost, st);
            if (e == hipSuccess) e = hipEventRecord(ready[c], st);
            if (e != hipSuccess) return fsdp::hip_fail(e, "device-to-host copy of a gradient shard");
        }
    }

    // 2. host AdamW over the work queue; a chunk's last part sends it back
    const fsdp::AdamScalars s = fsdp::adam_scalars(*hp);
    std::vector<int64_t> item_chunk(items);
    for (size_t j = 0; j < chunks.size(); ++j)
        for (int q = 0; q < chunks[j].parts; ++q) item_chunk[chunks[j].first_item + q] = (int64_t)j;
    std::unique_ptr<std::atomic<int>[]> left(new std::atomic<int>[chunks.size()]);
    std::unique_ptr<std::atomic<uint8_t>[]> landed(new std::atomic<uint8_t>[chunks.size()]);
    for (size_t j = 0; j < chunks.size(); ++j) {
        left[j].store(chunks[j].parts);
        landed[j].store(0);
    }
    std::atomic<int64_t> next{0};
    std::atomic<int> err{0};
    std::mutex err_mu;
    std::string err_msg;
    auto worker = [&](int) {
        for (;;) {
            if (err.load(std::memory_order_relaxed)) return;
            const int64_t it = next.fetch_add(1, std::memory_order_relaxed);
            if (it >= items) return;
            const int64_t j = item_chunk[it];
            const Chunk& ch = chunks[j];
            if (!landed[j].load(std::memory_order_acquire)) {
                const hipError_t we = hipEventSynchronize(ready[j]);
                if (we != hipSuccess) {
                    std::lock_guard<std::mutex> lk(err_mu);
                    err_msg = std::string("waiting for a gradient copy: ") + hipGetErrorString(we);
                    err.store(1);
                    return;
                }
                landed[j].store(1, std::memory_order_release);
            }
            const fsdp_offload_unit& u = units[ch.unit];
            const int64_t lo = ch.lo + (it - ch.first_item) * part, hi = std::min(ch.lo + ch.n, lo + part);
            adamw_range(u.master, u.exp_avg, u.exp_avg_sq, u.grad_shard_host, avg_dt, u.compute_host, compute_dt, lo,
                        hi, s);
            if (left[j].fetch_sub(1, std::memory_order_acq_rel) == 1) {
                const hipError_t we = hipMemcpyAsync((char*)u.compute_dev + ch.lo * cs,
                                                     (const char*)u.compute_host + ch.lo * cs, ch.n * cs,
                                                     hipMemcpyHostToDevice, cst);
                if (we != hipSuccess) {
                    std::lock_guard<std::mutex> lk(err_mu);
                    err_msg = std::string("host-to-device copy of a compute shard: ") + hipGetErrorString(we);
                    err.store(1);
                    return;
                }
            }
        }
    };
    const int workers = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)n_threads, (int64_t)256, items}));
    Pool::get().run_workers(workers, worker);
    if (err.load()) return fsdp::fail(FSDP_E_HIP, "%s: %s", fn, err_msg.c_str());
    if (cst != st) {
        // later work on `stream` sees the compute shards
        if ((e = hipEventRecord(done, cst)) != hipSuccess || (e = hipStreamWaitEvent(st, done, 0)) != hipSuccess)
            return fsdp::hip_fail(e, "copy stream ordering");
    }
    cleanup.finished = true;
    return fsdp::ok();
}

}  // namespace

extern "C" {

int fsdp_host_adamw(float* master, float* exp_avg, float* exp_avg_sq, const void* grad, fsdp_dtype grad_dt,
                    void* compute, fsdp_dtype compute_dt, int64_t n, const fsdp_adamw_hp* hp, int32_t n_threads) {
    if (n < 0) return fsdp::fail(FSDP_E_INVAL, "fsdp_host_adamw: n = %lld < 0", (long long)n);
    if (!fsdp::valid_dtype(grad_dt) || !fsdp::valid_dtype(compute_dt))
        return fsdp::fail(FSDP_E_DTYPE, "fsdp_host_adamw: grad dtype %d / compute dtype %d unsupported", (int)grad_dt,
                          (int)compute_dt);
    int rc = fsdp::check_hp("fsdp_host_adamw", hp);
    if (rc) return rc;
    if (n == 0) return fsdp::ok();
    if (!master || !exp_avg || !exp_avg_sq || !grad)
        return fsdp::fail(FSDP_E_INVAL, "fsdp_host_adamw: master, exp_avg, exp_avg_sq and grad must be non-NULL");
    std::vector<Span> v = {span(master, 4 * n), span(exp_avg, 4 * n), span(exp_avg_sq, 4 * n),
                           span(grad, n * fsdp::dt_size(grad_dt))};
    if (compute) v.push_back(span(compute, n * fsdp::dt_size(compute_dt)));
    if (!disjoint(v)) return fsdp::fail(FSDP_E_ALIAS, "fsdp_host_adamw: two of the buffers overlap");
    const fsdp::AdamScalars s = fsdp::adam_scalars(*hp);
    const int parts = std::max(1, std::min<int>(n_threads, 256));
    Pool::get().run(n, parts, [&](int64_t lo, int64_t hi) {
        adamw_range(master, exp_avg, exp_avg_sq, grad, grad_dt, compute, compute_dt, lo, hi, s);
    });
    return fsdp::ok();
}

int fsdp_offload_step_units(const fsdp_offload_unit* units, int32_t n_units, int32_t world, int32_t rank,
                            fsdp_dtype grad_dt, int32_t fp32_reduce, fsdp_dtype compute_dt, int64_t chunk_numel,
                            const fsdp_adamw_hp* hp, int32_t n_threads, void* stream, void* copy_stream) {
    return offload_units(units, n_units, world, rank, grad_dt, fp32_reduce, compute_dt, chunk_numel, hp, n_threads,
                         stream, copy_stream, "fsdp_offload_step_units", false);
}

int fsdp_offload_step_units_noalloc(const fsdp_offload_unit* units, int32_t n_units, int32_t world, int32_t rank,
                                    fsdp_dtype grad_dt, int32_t fp32_reduce, fsdp_dtype compute_dt,
                                    int64_t chunk_numel, const fsdp_adamw_hp* hp, int32_t n_threads, void* stream,
                                    void* copy_stream) {
    return offload_units(units, n_units, world, rank, grad_dt, fp32_reduce, compute_dt, chunk_numel, hp, n_threads,
                         stream, copy_stream, "fsdp_offload_step_units_noalloc", true);
}

int fsdp_offload_step(float* master, float* exp_avg, float* exp_avg_sq, const void* const* rank_grads,
                      int32_t world, int32_t rank, fsdp_dtype grad_dt, int32_t fp32_reduce, void* grad_shard_dev,
                      void* grad_shard_host, void* compute_host, void* compute_dev, fsdp_dtype compute_dt,
                      int64_t shard_numel, int64_t chunk_numel, const fsdp_adamw_hp* hp, int32_t n_threads,
                      void* stream, void* copy_stream) {
    const fsdp_offload_unit u{master, exp_avg, exp_avg_sq, rank_grads, grad_shard_dev, grad_shard_host,
                              compute_host, compute_dev, shard_numel};
    return offload_units(&u, 1, world, rank, grad_dt, fp32_reduce, compute_dt, chunk_numel, hp, n_threads, stream,
                         copy_stream, "fsdp_offload_step", false);
}

}  // extern "C"
