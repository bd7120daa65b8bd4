// fsdp_device.h -- device primitives shared by the gfx950 kernels of
// libfsdp_shard.so: 16-byte global accesses, number formats, the N-way
// rank reduction, and the launch helper.  Not installed.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "fsdp_kernels.h"

#pragma clang fp contract(off)

namespace fsdp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef FSDP_NT_STORE
#define FSDP_NT_STORE 1   // streamed outputs: non-temporal (measured +1-9% on the unit step)
#endif
// 16-byte global accesses; the streamed buffers are touched once per launch,
// so wide stores carry the non-temporal hint.  Loads carry it where it was
// measured to pay (NT = true): in the unit step at its residency cap (+1 to +3
// points of HBM peak on most workloads) and in the copies (+2%); the
// read-mostly reduce-scatter alone is faster with plain loads (-6% with the hint).
template <bool NT = false>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
#if FSDP_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool NT = false>
__device__ __forceinline__ u32x2 ld8(const u32x2* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
__device__ __forceinline__ void st8(u32x2* p, u32x2 v) {
#if FSDP_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

#ifndef FSDP_STORE_SC1
#define FSDP_STORE_SC1 1
#endif
// Streamed stores of one wave into one span of its outputs: every lane of the
// wave passes the same span start, and its own byte offset inside the span.
// With FSDP_STORE_SC1 (the default) the stores go through a buffer resource
// over the span, so that they carry the sc1 scope bit beside the non-temporal
// hint: measured on a 1 GiB copy, 82.0-82.3% of 8 TB/s with the hint alone
// and 84.0-84.2% with nt sc1 (load policy bits changed nothing); on the unit
// step, +1.0 to +4.0 points of the whole step on every workload, same box.
// The resource's range is the span, so an offset outside it is dropped, never
// written elsewhere.
__device__ __forceinline__ void* wave_uniform(void* p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (void*)(((uint64_t)hi << 32) | lo);
}
constexpr int kRsrcWord3 = 0x00020000;   // raw (unswizzled) buffer, 32-bit data format
constexpr int kStorePolicy = 2 | 16;     // nt sc1
template <unsigned SPAN>
__device__ __forceinline__ void st16_span(void* span, unsigned off, u32x4 v) {
#if FSDP_STORE_SC1
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(wave_uniform(span), 0, SPAN, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStorePolicy);
#else
    st16(reinterpret_cast<u32x4*>(static_cast<char*>(span) + off), v);
#endif
}
template <unsigned SPAN>
__device__ __forceinline__ void st8_span(void* span, unsigned off, u32x2 v) {
#if FSDP_STORE_SC1
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(wave_uniform(span), 0, SPAN, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStorePolicy);
#else
    st8(reinterpret_cast<u32x2*>(static_cast<char*>(span) + off), v);
#endif
}
// Lane l (= threadIdx.x % 64) of a wave stores 16 bytes at [16 l, 16 l + 16) of
// a 1 KB span.
__device__ __forceinline__ void st16_wave(void* span, int l, u32x4 v) { st16_span<1024>(span, 16u * l, v); }

// ----------------------------------------------------------------- formats
template <int F> __device__ __forceinline__ float to_f32(uint32_t bits);
template <> __device__ __forceinline__ float to_f32<FSDP_F32>(uint32_t bits) { return __uint_as_float(bits); }
template <> __device__ __forceinline__ float to_f32<FSDP_F16>(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);      // exact
}
template <> __device__ __forceinline__ float to_f32<FSDP_BF16>(uint32_t bits) {
    return __uint_as_float(bits << 16);                                // exact
}

template <int F> __device__ __forceinline__ uint32_t from_f32(float x);
template <> __device__ __forceinline__ uint32_t from_f32<FSDP_F32>(float x) { return __float_as_uint(x); }
template <> __device__ __forceinline__ uint32_t from_f32<FSDP_F16>(float x) {
    // v_cvt_f16_f32: round to nearest even, binary16 subnormals kept
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ uint32_t from_f32<FSDP_BF16>(float x) {
    // gfx950's conversion (v_cvt_pk_bf16_f32): round to nearest even, NaN kept
    // a quiet NaN with the high bits of its payload, subnormals kept -- the
    // same 16 bits as bf16_rne below on every one of the 2^32 fp32 encodings,
    // in one instruction instead of five and a branch.
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// The same rounding on the encoding: add 0x7fff plus the lowest kept bit and
// drop the low 16 bits (ties to even); a NaN is quieted and truncated.  The
// NaN test is one unordered compare and a branch that a wave skips when none
// of its lanes holds a NaN.  Used for the fold of a 16-bit reduce-scatter
// over more than two ranks (reduce_round below).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    if (__builtin_isnan(x)) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int F> __device__ __forceinline__ float round_to(float x) { return to_f32<F>(from_f32<F>(x)); }

// 8 consecutive elements of format F starting at element 8*vi (16-byte aligned).
template <int F, bool NT = false>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t vi, float (&x)[8]) {
    if constexpr (F == FSDP_F32) {
        const u32x4* q = reinterpret_cast<const u32x4*>(base) + 2 * vi;
        u32x4 a = ld16<NT>(q), b = ld16<NT>(q + 1);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    } else {
        u32x4 a = ld16<NT>(reinterpret_cast<const u32x4*>(base) + vi);
        uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = to_f32<F>(w[k] & 0xffffu);
            x[2 * k + 1] = to_f32<F>(w[k] >> 16);
        }
    }
}

// 8 consecutive elements per lane, stored by whole waves: lane l =
// threadIdx.x % 64 stores vector vi with vi % 64 == l, the wave the 64
// consecutive vectors from vi - l.  16-bit: one dwordx4 per lane, the wave's
// 1 KB span with the sc1 policy (the reduce-scatter's 16-bit output, the
// bf16-state unit step).  fp32 (two instructions, each one half of
// every 32-byte piece of the span) keeps plain non-temporal stores: with the
// sc1 policy that form measured 35% slower, so fp32 outputs take the group
// layout (store8g) instead.
template <int F>
__device__ __forceinline__ void store8(void* __restrict__ base, int64_t vi, const float (&x)[8]) {
    if constexpr (F == FSDP_F32) {
        u32x4* q = reinterpret_cast<u32x4*>(base) + 2 * vi;
        u32x4 a, b;
        a.x = __float_as_uint(x[0]); a.y = __float_as_uint(x[1]);
        a.z = __float_as_uint(x[2]); a.w = __float_as_uint(x[3]);
        b.x = __float_as_uint(x[4]); b.y = __float_as_uint(x[5]);
        b.z = __float_as_uint(x[6]); b.w = __float_as_uint(x[7]);
        st16(q, a);
        st16(q + 1, b);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = from_f32<F>(x[2 * k]) | (from_f32<F>(x[2 * k + 1]) << 16);
        u32x4 a;
        a.x = w[0]; a.y = w[1]; a.z = w[2]; a.w = w[3];
        const int l = (int)(threadIdx.x & 63);
        st16_wave(reinterpret_cast<u32x4*>(base) + (vi - l), l, a);
    }
}

// Group layout of the unit kernel.  A group is 64 vectors, one per lane of a
// wave: group g = vi / 64 holds elements [512 g, 512 g + 512), and lane
// l = vi % 64 owns elements 512 g + 4 l + k and 512 g + 256 + 4 l + k (k < 4).
// Each access instruction of the wave then covers one contiguous span (1 KB
// of fp32, 512 B of a 16-bit format), so no cache line is half-written by one
// instruction and completed by the next; with load8/store8 (8 consecutive
// elements per lane) an fp32 access is two instructions of 32-byte-strided
// halves.  Only for groups wholly inside the buffer, and only with the lanes
// of a wave on the 64 vectors of one group (vi % 64 == threadIdx.x % 64): the
// stores of a wave go to one span (st16_span).
template <int F, bool NT = false>
__device__ __forceinline__ void load8g(const void* __restrict__ base, int64_t vi, float (&x)[8]) {
    const int64_t g = vi >> 6, l = vi & 63;
    if constexpr (F == FSDP_F32) {
        const u32x4* q = reinterpret_cast<const u32x4*>(base) + g * 128 + l;
        u32x4 a = ld16<NT>(q), b = ld16<NT>(q + 64);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    } else {
        const u32x2* q = reinterpret_cast<const u32x2*>(base) + g * 128 + l;
        u32x2 a = ld8<NT>(q), b = ld8<NT>(q + 64);
        uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = to_f32<F>(w[k] & 0xffffu);
            x[2 * k + 1] = to_f32<F>(w[k] >> 16);
        }
    }
}

template <int F>
__device__ __forceinline__ void store8g(void* __restrict__ base, int64_t vi, const float (&x)[8]) {
    const int64_t g = vi >> 6, l = vi & 63;
    if constexpr (F == FSDP_F32) {
        u32x4* q = reinterpret_cast<u32x4*>(base) + g * 128;
        u32x4 a, b;
        a.x = __float_as_uint(x[0]); a.y = __float_as_uint(x[1]);
        a.z = __float_as_uint(x[2]); a.w = __float_as_uint(x[3]);
        b.x = __float_as_uint(x[4]); b.y = __float_as_uint(x[5]);
        b.z = __float_as_uint(x[6]); b.w = __float_as_uint(x[7]);
        st16_wave(q, (int)l, a);
        st16_wave(q + 64, (int)l, b);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = from_f32<F>(x[2 * k]) | (from_f32<F>(x[2 * k + 1]) << 16);
        u32x2* q = reinterpret_cast<u32x2*>(base) + g * 128;
        u32x2 a, b;
        a.x = w[0]; a.y = w[1];
        b.x = w[2]; b.y = w[3];
        st8_span<512>(q, 8u * (unsigned)l, a);
        st8_span<512>(q + 64, 8u * (unsigned)l, b);
    }
}

template <int F, bool GROUP>
__device__ __forceinline__ void store8x(void* __restrict__ base, int64_t vi, const float (&x)[8]) {
    if constexpr (GROUP) store8g<F>(base, vi, x);
    else store8<F>(base, vi, x);
}

// The 8 elements of vector vi: consecutive (GROUP = false) or in the group layout.
template <int F, bool NT, bool GROUP>
__device__ __forceinline__ void load8x(const void* __restrict__ base, int64_t vi, float (&x)[8]) {
    if constexpr (GROUP) load8g<F, NT>(base, vi, x);
    else load8<F, NT>(base, vi, x);
}

template <int F>
__device__ __forceinline__ float load1(const void* __restrict__ base, int64_t i) {
    if constexpr (F == FSDP_F32) return reinterpret_cast<const float*>(base)[i];
    else return to_f32<F>(reinterpret_cast<const uint16_t*>(base)[i]);
}

template <int F>
__device__ __forceinline__ void store1(void* __restrict__ base, int64_t i, float x) {
    if constexpr (F == FSDP_F32) reinterpret_cast<float*>(base)[i] = x;
    else reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)from_f32<F>(x);
}

// ----------------------------------------------------------------- reduction
// Whether the 16-bit fold of an N-rank reduce-scatter rounds to bf16 with the
// conversion instruction (N <= 2) or on the encoding (more ranks).  Same
// bits either way; measured on the whole step, same box, four repetitions:
// the instruction took GPT-2 XL (N = 2) from 78.7 to 79.8% of 8 TB/s and the
// 70B block (N = 8) from 81.2 to 80.5%; with the encoding form's branches the
// N = 8 fold keeps its loads ahead of the arithmetic without a fence.
template <int NW, int GF>
constexpr bool kHwFold = GF == FSDP_BF16 && NW >= 1 && NW <= 2;

template <int NW, int GF>
__device__ __forceinline__ float reduce_round(float x) {
    if constexpr (GF == FSDP_BF16 && !kHwFold<NW, GF>) return to_f32<GF>(bf16_rne(x));
    else return round_to<GF>(x);
}

// One step of the left fold over ranks.  fp32 mode: a single fp32 add.
// 16-bit mode: the sum rounded back to the gradient format.
template <int NW, int GF, bool FP32R>
__device__ __forceinline__ float fold(float acc, float x) {
    if constexpr (FP32R || GF == FSDP_F32) return acc + x;
    else return reduce_round<NW, GF>(acc + x);
}

// acc / N.  The specialised kernels (N in {1, 2, 4, 8}) multiply by 1/N: for a
// power of two that product is the same correctly rounded value as the
// quotient.  The generic kernel divides.  In 16-bit mode the quotient is then
// rounded to the gradient format.
template <int NW, int GF, bool FP32R>
__device__ __forceinline__ float finish(float acc, const ReduceScalars& r) {
    static_assert(NW == 0 || (NW & (NW - 1)) == 0, "specialised world sizes are powers of two");
    float q = NW > 0 ? acc * r.inv_n : acc / r.n;
    if constexpr (FP32R || GF == FSDP_F32) return q;
    else return reduce_round<NW, GF>(q);
}


// Gradient pointer accessors: gp(q) is rank q's block (shard-relative).
template <int NW>
struct GradsOf {                       // single-unit kernels: pointers by value
    const GradPtrs<NW>& g;
    __device__ __forceinline__ const void* operator()(int q) const { return g.p[q]; }
};
template <int NW>
struct UnitGrads {                     // batched kernel: unit u of the launch's table
    const UnitBatch<NW>& B;
    int u;
    __device__ __forceinline__ const void* operator()(int q) const { return B.g[u][q]; }
};

// Accumulate the N rank blocks of 8 elements into acc (all loads first).
template <int NW, int GF, bool FP32R, bool NT = false, bool GROUP = false, typename GP>
__device__ __forceinline__ void reduce8(const GP& gp, int world, int64_t vi, float (&acc)[8]) {
    if constexpr (NW > 0) {
        float x[NW][8];
#pragma unroll
        for (int q = 0; q < NW; ++q) load8x<GF, NT, GROUP>(gp(q), vi, x[q]);
        // every load issued before the fold: without this fence the scheduler
        // sinks gradient loads into a branch-free bf16 fold (fewer reads in flight)
        if constexpr (kHwFold<NW, GF> && !FP32R) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = x[0][k];
#pragma unroll
        for (int q = 1; q < NW; ++q)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = fold<NW, GF, FP32R>(acc[k], x[q][k]);
    } else {
        load8x<GF, NT, GROUP>(gp(0), vi, acc);
        int q = 1;
        for (; q + 4 <= world; q += 4) {
            float x[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) load8x<GF, NT, GROUP>(gp(q + j), vi, x[j]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = fold<NW, GF, FP32R>(acc[k], x[j][k]);
        }
        for (; q < world; ++q) {
            float x[8];
            load8x<GF, NT, GROUP>(gp(q), vi, x);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = fold<NW, GF, FP32R>(acc[k], x[k]);
        }
    }
}

template <int NW, int GF, bool FP32R, typename GP>
__device__ __forceinline__ float reduce1(const GP& gp, int world, int64_t i) {
    const int n = NW > 0 ? NW : world;
    float acc = load1<GF>(gp(0), i);
    for (int q = 1; q < n; ++q) acc = fold<NW, GF, FP32R>(acc, load1<GF>(gp(q), i));
    return acc;
}


// ----------------------------------------------------------------- launch
// Launch (with `lds` bytes of dynamic LDS per workgroup) with the events armed
// by set_launch_events(), if any, attached to the kernel's own dispatch packet
// (hipExtLaunchKernel); the pair is consumed.
void take_launch_events(hipEvent_t* start, hipEvent_t* stop);

template <typename K, typename... Args>
static void launch_lds(K kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t st, Args... args) {
    hipEvent_t a, b;
    take_launch_events(&a, &b);
    if (a || b)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, st, a, b, 0, args...);
    else
        kernel<<<grid, block, lds, st>>>(args...);
}

template <typename K, typename... Args>
static void launch(K kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    launch_lds(kernel, grid, block, 0u, st, args...);
}

static inline int64_t grid_for(int64_t work, int cus) {
    int64_t want = (work + kThreads - 1) / kThreads;
    int64_t cap = (int64_t)cus * kBlocksPerCU;
    if (want > cap) want = cap;
    return want < 1 ? 1 : want;
}

}  // namespace fsdp
