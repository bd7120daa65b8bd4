// fsdp_kernels.hip -- gfx950 (CDNA4) kernels of the FSDP flat-parameter shard
// pipeline.  Every kernel is an HBM stream: no contraction, so no MFMA.
//
// Design (MI355X, 256 CUs in 8 XCDs, 64-wide waves, HBM3E ~8 TB/s):
//  * 16-byte (dwordx4) global loads/stores per lane; a lane owns 8 consecutive
//    elements of the shard per step (one dwordx4 of 16-bit data, two of fp32);
//  * grid-stride loops over a grid sized to a multiple of the CU count, so a
//    launch is a few thousand workgroups regardless of the unit size;
//  * the N simulated ranks' gradient blocks are accumulated in registers, all N
//    loads issued before the first add (N is a template parameter for
//    N in {1, 2, 4, 8});
//  * reduce-scatter + AdamW + cast run in one pass over the shard (one read of
//    N gradient blocks and master/m/v, one write of master/m/v and the compute
//    copy);
//  * arithmetic matches the definition bit for bit: no FMA contraction,
//    correctly rounded divide and sqrt, fp32 subnormals preserved.
//
// Sources: "Fully Sharded Data Parallel: faster AI training with fewer GPUs"
// (techreport.ngo) -- figure on all-reduce as reduce-scatter + all-gather,
// section "From all-reduce to sharded parameters"; "Data Parallelism"
// (vanos001 notes) -- section "The Basic Protocol"; "FSDP (Fully Sharded Data
// Parallel)" (vanos001 notes) -- sections "The Per-Layer Communication" and
// "Mixed Precision and FSDP"; "fairseq 中的 Fully Sharded Data Parallel (FSDP)
// 实战指南" (zskr.cn) -- flag table (--fp32-reduce-scatter) and "工作原理".

#include "fsdp_kernels.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#pragma clang fp contract(off)

namespace fsdp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef FSDP_NT_LOAD
#define FSDP_NT_LOAD 0
#endif
#ifndef FSDP_NT_STORE
#define FSDP_NT_STORE 1   // streamed outputs: non-temporal (measured +1-9% on the unit step)
#endif
// 16-byte global accesses; the streamed buffers are touched once per launch,
// so wide stores carry the non-temporal hint.
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
#if FSDP_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
#if FSDP_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

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
    // Round the fp32 encoding at bit 16, ties to even; NaN stays a quiet NaN.
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int F> __device__ __forceinline__ float round_to(float x) { return to_f32<F>(from_f32<F>(x)); }

// 8 consecutive elements of format F starting at element 8*vi (16-byte aligned).
template <int F>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t vi, float (&x)[8]) {
    if constexpr (F == FSDP_F32) {
        const u32x4* q = reinterpret_cast<const u32x4*>(base) + 2 * vi;
        u32x4 a = ld16(q), b = ld16(q + 1);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    } else {
        u32x4 a = ld16(reinterpret_cast<const u32x4*>(base) + vi);
        uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = to_f32<F>(w[k] & 0xffffu);
            x[2 * k + 1] = to_f32<F>(w[k] >> 16);
        }
    }
}

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
        st16(reinterpret_cast<u32x4*>(base) + vi, a);
    }
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
// One step of the left fold over ranks.  fp32 mode: a single fp32 add.
// 16-bit mode: the sum rounded back to the gradient format.
template <int GF, bool FP32R>
__device__ __forceinline__ float fold(float acc, float x) {
    if constexpr (FP32R || GF == FSDP_F32) return acc + x;
    else return round_to<GF>(acc + x);
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
    else return round_to<GF>(q);
}

// ----------------------------------------------------------------- AdamW
__device__ __forceinline__ void adamw1(float g, float& p, float& m, float& v, const AdamScalars& s) {
    float p1 = p * s.decay;
    float m1 = (s.b1 * m) + (s.omb1 * g);
    float v1 = (s.b2 * v) + (s.omb2 * (g * g));
    float den = (__builtin_sqrtf(v1) / s.bc2_sqrt) + s.eps;
    float p2 = p1 - (s.step_size * (m1 / den));
    p = p2;
    m = m1;
    v = v1;
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
template <int NW, int GF, bool FP32R, typename GP>
__device__ __forceinline__ void reduce8(const GP& gp, int world, int64_t vi, float (&acc)[8]) {
    if constexpr (NW > 0) {
        float x[NW][8];
#pragma unroll
        for (int q = 0; q < NW; ++q) load8<GF>(gp(q), vi, x[q]);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = x[0][k];
#pragma unroll
        for (int q = 1; q < NW; ++q)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = fold<GF, FP32R>(acc[k], x[q][k]);
    } else {
        load8<GF>(gp(0), vi, acc);
        int q = 1;
        for (; q + 4 <= world; q += 4) {
            float x[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) load8<GF>(gp(q + j), vi, x[j]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = fold<GF, FP32R>(acc[k], x[j][k]);
        }
        for (; q < world; ++q) {
            float x[8];
            load8<GF>(gp(q), vi, x);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = fold<GF, FP32R>(acc[k], x[k]);
        }
    }
}

template <int NW, int GF, bool FP32R, typename GP>
__device__ __forceinline__ float reduce1(const GP& gp, int world, int64_t i) {
    const int n = NW > 0 ? NW : world;
    float acc = load1<GF>(gp(0), i);
    for (int q = 1; q < n; ++q) acc = fold<GF, FP32R>(acc, load1<GF>(gp(q), i));
    return acc;
}

// ----------------------------------------------------------------- kernels
// One unit's step on vector vi (8 elements): every load first (the N gradient
// blocks, master/m/v, the peers' compute vectors), then the math, then every
// store.  With GATHER, `out` is this rank's slot of the full buffer and the
// peers' vectors are copied into their slots.
template <int NW, int GF, bool FP32R, int CF, bool GATHER, int SF>
__device__ __forceinline__ void unit_vec(const UnitBatch<NW>& B, int u, int64_t vi, const ReduceScalars& rs,
                                         const AdamScalars& as) {
    constexpr int kW = CF == FSDP_F32 ? 2 : 1;      // dwordx4 per 8 compute elements
    constexpr int kP = NW > 1 ? NW - 1 : 1;
    void* __restrict__ p = B.p[u];
    void* __restrict__ m = B.m[u];
    void* __restrict__ v = B.v[u];
    float acc[8], pp[8], mm[8], vv[8];
    u32x4 peer[kP][kW];
    if constexpr (GATHER && NW > 1) {
#pragma unroll
        for (int j = 0; j < NW - 1; ++j)
#pragma unroll
            for (int w = 0; w < kW; ++w) peer[j][w] = ld16(reinterpret_cast<const u32x4*>(B.psrc[u][j]) + kW * vi + w);
    }
    load8<SF>(p, vi, pp);
    load8<SF>(m, vi, mm);
    load8<SF>(v, vi, vv);
    reduce8<NW, GF, FP32R>(UnitGrads<NW>{B, u}, B.world, vi, acc);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the math
#pragma unroll
    for (int k = 0; k < 8; ++k) adamw1(finish<NW, GF, FP32R>(acc[k], rs), pp[k], mm[k], vv[k], as);
    store8<SF>(p, vi, pp);
    store8<SF>(m, vi, mm);
    store8<SF>(v, vi, vv);
    void* out = B.out[u];
    void* out2 = B.out2[u];
    if constexpr (GATHER) {
        // the unit step always has its own slot; keep the peer stores in the
        // same basic block as their loads so they are not sunk past the math
        store8<CF>(out, vi, pp);
        if constexpr (NW > 1) {
#pragma unroll
            for (int j = 0; j < NW - 1; ++j)
#pragma unroll
                for (int w = 0; w < kW; ++w) st16(reinterpret_cast<u32x4*>(B.pdst[u][j]) + kW * vi + w, peer[j][w]);
        } else if constexpr (NW == 0) {
            for (int j = 0; j < B.npeers; ++j)
#pragma unroll
                for (int w = 0; w < kW; ++w)
                    st16(reinterpret_cast<u32x4*>(B.pdst[u][j]) + kW * vi + w,
                         ld16(reinterpret_cast<const u32x4*>(B.psrc[u][j]) + kW * vi + w));
        }
    } else {
        if (out) store8<CF>(out, vi, pp);
    }
    if (out2) store8<CF>(out2, vi, pp);
}

// Element i of unit u, one lane (the tail past the last full vector, or every
// element of a unit whose buffers are not 16-byte aligned).
template <int NW, int GF, bool FP32R, int CF, bool GATHER, int SF>
__device__ __forceinline__ void unit_elem(const UnitBatch<NW>& B, int u, int64_t i, const ReduceScalars& rs,
                                          const AdamScalars& as) {
    void* __restrict__ p = B.p[u];
    void* __restrict__ m = B.m[u];
    void* __restrict__ v = B.v[u];
    float pp = load1<SF>(p, i), mm = load1<SF>(m, i), vv = load1<SF>(v, i);
    adamw1(finish<NW, GF, FP32R>(reduce1<NW, GF, FP32R>(UnitGrads<NW>{B, u}, B.world, i), rs), pp, mm, vv, as);
    store1<SF>(p, i, pp);
    store1<SF>(m, i, mm);
    store1<SF>(v, i, vv);
    if (GATHER || B.out[u]) store1<CF>(B.out[u], i, pp);
    if (B.out2[u]) store1<CF>(B.out2[u], i, pp);
    if constexpr (GATHER) {
        const int n = NW > 0 ? NW - 1 : B.npeers;
        for (int j = 0; j < n; ++j) {
            if constexpr (CF == FSDP_F32)
                reinterpret_cast<uint32_t*>(B.pdst[u][j])[i] = reinterpret_cast<const uint32_t*>(B.psrc[u][j])[i];
            else
                reinterpret_cast<uint16_t*>(B.pdst[u][j])[i] = reinterpret_cast<const uint16_t*>(B.psrc[u][j])[i];
        }
    }
}

// Fused reduce-scatter + AdamW + cast (+ all-gather with GATHER) over the
// shards of up to UnitBatch<NW>::kMax units in one launch.  Workgroup b owns
// tile b: unit u holds tiles [tile_begin[u], tile_begin[u+1]); its first
// ceil(nvec/256) tiles are 256 vectors of 8 elements each, the rest 256
// single elements (the tail, or the whole unit when unaligned).  One launch
// pays the ramp-up and drain of the grid once for all its units.
// SF is the state format: FSDP_F32 for fp32 master/m/v with a separate compute
// copy of format CF, or a 16-bit format (CF == SF) where the parameter shard is
// itself the compute copy.
template <int NW, int GF, bool FP32R, int CF, bool GATHER, int SF>
__global__ __launch_bounds__(kThreads) void k_units(UnitBatch<NW> B, ReduceScalars rs, AdamScalars as) {
    const int64_t tile = blockIdx.x;
    int lo = 0, hi = B.count - 1;          // unit u with tile_begin[u] <= tile < tile_begin[u+1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (B.tile_begin[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    const int u = lo;
    const int64_t j = tile - B.tile_begin[u];
    const int64_t nvec = B.nvec[u];
    const int64_t tv = (nvec + kThreads - 1) / kThreads;
    if (j < tv) {
        const int64_t vi = j * kThreads + threadIdx.x;
        if (vi < nvec) unit_vec<NW, GF, FP32R, CF, GATHER, SF>(B, u, vi, rs, as);
    } else {
        const int64_t i = nvec * 8 + (j - tv) * kThreads + threadIdx.x;
        if (i < B.S[u]) unit_elem<NW, GF, FP32R, CF, GATHER, SF>(B, u, i, rs, as);
    }
}

// Reduce-scatter alone: averaged gradient shard in fp32 (fp32 mode) or in the
// gradient format (16-bit mode).
template <int NW, int GF, bool FP32R>
__global__ __launch_bounds__(kThreads) void k_reduce_scatter(
    GradPtrs<NW> g, int world, int64_t S, int64_t nvec, void* __restrict__ out, ReduceScalars rs) {
    constexpr int OF = (FP32R || GF == FSDP_F32) ? FSDP_F32 : GF;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const GradsOf<NW> gp{g};
    for (int64_t vi = t0; vi < nvec; vi += stride) {
        float acc[8];
        reduce8<NW, GF, FP32R>(gp, world, vi, acc);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = finish<NW, GF, FP32R>(acc[k], rs);
        store8<OF>(out, vi, acc);
    }
    for (int64_t i = nvec * 8 + t0; i < S; i += stride)
        store1<OF>(out, i, finish<NW, GF, FP32R>(reduce1<NW, GF, FP32R>(gp, world, i), rs));
}

// Copy `bytes` bytes from src to dst (or write zeros when src is null) with the
// widest access both addresses allow.  Called by every lane of a range of
// `nthreads` lanes, lane index `lane`.
__device__ __forceinline__ void copy_range(char* __restrict__ dst, const char* __restrict__ src,
                                           int64_t bytes, int64_t lane, int64_t nthreads) {
    const uintptr_t a = (uintptr_t)dst | (src ? (uintptr_t)src : 0);
    if ((a & 15) == 0) {
        const int64_t nv = bytes >> 4;
        u32x4* d = reinterpret_cast<u32x4*>(dst);
        const u32x4* s = reinterpret_cast<const u32x4*>(src);
        if (src) {
            for (int64_t i = lane; i < nv; i += nthreads) st16(d + i, ld16(s + i));
        } else {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int64_t i = lane; i < nv; i += nthreads) st16(d + i, z);
        }
        for (int64_t i = (nv << 4) + lane; i < bytes; i += nthreads) dst[i] = src ? src[i] : 0;
    } else if ((a & 3) == 0) {
        const int64_t nw = bytes >> 2;
        uint32_t* d = reinterpret_cast<uint32_t*>(dst);
        const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
        for (int64_t i = lane; i < nw; i += nthreads) d[i] = src ? s[i] : 0u;
        for (int64_t i = (nw << 2) + lane; i < bytes; i += nthreads) dst[i] = src ? src[i] : 0;
    } else if ((a & 1) == 0) {
        const int64_t nh = bytes >> 1;
        uint16_t* d = reinterpret_cast<uint16_t*>(dst);
        const uint16_t* s = reinterpret_cast<const uint16_t*>(src);
        for (int64_t i = lane; i < nh; i += nthreads) d[i] = src ? s[i] : (uint16_t)0;
        for (int64_t i = (nh << 1) + lane; i < bytes; i += nthreads) dst[i] = src ? src[i] : 0;
    } else {
        for (int64_t i = lane; i < bytes; i += nthreads) dst[i] = src ? src[i] : 0;
    }
}

// All-gather unshard: copy j of the list moves `bytes` bytes src[j] -> dst[j].
// blockIdx.y selects the copy; blocks along x stride over its bytes.
template <int MAXN>
__global__ __launch_bounds__(kThreads) void k_gather(CopyList<MAXN> L, int64_t bytes) {
    const int j = blockIdx.y;
    copy_range(L.dst[j], L.src[j], bytes, (int64_t)blockIdx.x * kThreads + threadIdx.x,
               (int64_t)gridDim.x * kThreads);
}

// Segmented copy for flatten/unflatten: workgroup b handles chunk b of the
// batch; segment k owns chunks [chunk_begin[k], chunk_begin[k+1]).
__global__ __launch_bounds__(kThreads) void k_segments(SegBatch B) {
    const int64_t c = blockIdx.x;
    int lo = 0, hi = B.count - 1;          // find k with chunk_begin[k] <= c < chunk_begin[k+1]
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (B.chunk_begin[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    const int k = lo;
    const int64_t start = (c - B.chunk_begin[k]) * kSegChunkBytes;
    int64_t n = B.bytes[k] - start;
    if (n > kSegChunkBytes) n = kSegChunkBytes;
    if (n <= 0) return;
    copy_range(B.dst[k] + start, B.src[k] ? B.src[k] + start : nullptr, n, threadIdx.x, kThreads);
}

// ----------------------------------------------------------------- launchers
// Optional timing of the next launch: the events ride on the kernel's own
// dispatch (hipExtLaunchKernel), so no marker packets enter the stream.
static thread_local hipEvent_t t_ev_start = nullptr;
static thread_local hipEvent_t t_ev_stop = nullptr;

void set_launch_events(void* start, void* stop) {
    t_ev_start = (hipEvent_t)start;
    t_ev_stop = (hipEvent_t)stop;
}

template <typename K, typename... Args>
static void launch(K kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    if (t_ev_start || t_ev_stop) {
        hipEvent_t a = t_ev_start, b = t_ev_stop;
        t_ev_start = t_ev_stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
    } else {
        kernel<<<grid, block, 0, st>>>(args...);
    }
}

static int64_t grid_for(int64_t work, int cus) {
    int64_t want = (work + kThreads - 1) / kThreads;
    int64_t cap = (int64_t)cus * kBlocksPerCU;
    if (want > cap) want = cap;
    return want < 1 ? 1 : want;
}

template <int NW, int GF, bool FP32R, int CF, int SF>
static hipError_t units_go(const UnitBatch<NW>& B, int64_t tiles, bool gather, const ReduceScalars& rs,
                           const AdamScalars& as, hipStream_t st) {
    if (gather)
        launch(k_units<NW, GF, FP32R, CF, true, SF>, dim3((unsigned)tiles), dim3(kThreads), st, B, rs, as);
    else
        launch(k_units<NW, GF, FP32R, CF, false, SF>, dim3((unsigned)tiles), dim3(kThreads), st, B, rs, as);
    return hipGetLastError();
}

template <int NW, int GF, bool FP32R>
static hipError_t units_cf(const UnitBatch<NW>& B, int64_t tiles, const UnitLaunch& L, hipStream_t st) {
    if (L.state_dt == FSDP_F16) return units_go<NW, GF, FP32R, FSDP_F16, FSDP_F16>(B, tiles, L.gather, L.rs, L.as, st);
    if (L.state_dt == FSDP_BF16) return units_go<NW, GF, FP32R, FSDP_BF16, FSDP_BF16>(B, tiles, L.gather, L.rs, L.as, st);
    switch (L.compute_dt) {
    case FSDP_F32: return units_go<NW, GF, FP32R, FSDP_F32, FSDP_F32>(B, tiles, L.gather, L.rs, L.as, st);
    case FSDP_F16: return units_go<NW, GF, FP32R, FSDP_F16, FSDP_F32>(B, tiles, L.gather, L.rs, L.as, st);
    default: return units_go<NW, GF, FP32R, FSDP_BF16, FSDP_F32>(B, tiles, L.gather, L.rs, L.as, st);
    }
}

template <int NW>
static hipError_t units_batch(const UnitBatch<NW>& B, int64_t tiles, const UnitLaunch& L) {
    hipStream_t st = (hipStream_t)L.stream;
    const bool f32r = L.fp32_reduce || L.grad_dt == FSDP_F32;
    if (L.grad_dt == FSDP_F32) return units_cf<NW, FSDP_F32, true>(B, tiles, L, st);
    if (L.grad_dt == FSDP_F16) {
        if (f32r) return units_cf<NW, FSDP_F16, true>(B, tiles, L, st);
        return units_cf<NW, FSDP_F16, false>(B, tiles, L, st);
    }
    if (f32r) return units_cf<NW, FSDP_BF16, true>(B, tiles, L, st);
    return units_cf<NW, FSDP_BF16, false>(B, tiles, L, st);
}

// Pack the units into tables of at most kMax and launch one grid per table.
template <int NW>
static hipError_t units_all(const UnitArgs* units, int n, const UnitLaunch& L) {
    constexpr int kMax = UnitBatch<NW>::kMax;
    int done = 0;
    while (done < n) {
        UnitBatch<NW> B{};
        B.world = L.world;
        B.npeers = L.gather ? L.world - 1 : 0;
        int64_t tiles = 0;
        int c = 0;
        for (; c < kMax && done + c < n; ++c) {
            const UnitArgs& a = units[done + c];
            B.tile_begin[c] = tiles;
            B.nvec[c] = a.nvec;
            B.S[c] = a.S;
            B.p[c] = a.p;
            B.m[c] = a.m;
            B.v[c] = a.v;
            B.out[c] = a.out;
            B.out2[c] = a.out2;
            for (int q = 0; q < L.world; ++q) B.g[c][q] = a.grads[q];
            for (int q = 0; q < B.npeers; ++q) {
                B.psrc[c][q] = (const char*)a.peer_src[q];
                B.pdst[c][q] = (char*)a.peer_dst[q];
            }
            tiles += (a.nvec + kThreads - 1) / kThreads + (a.S - 8 * a.nvec + kThreads - 1) / kThreads;
        }
        B.count = c;
        B.tile_begin[c] = tiles;
        done += c;
        if (tiles == 0) continue;
        hipError_t e = units_batch<NW>(B, tiles, L);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_units(const UnitArgs* units, int n, const UnitLaunch& L) {
    switch (L.world) {
    case 1: return units_all<1>(units, n, L);
    case 2: return units_all<2>(units, n, L);
    case 4: return units_all<4>(units, n, L);
    case 8: return units_all<8>(units, n, L);
    default: return units_all<0>(units, n, L);
    }
}

template <int NW, int GF, bool FP32R>
static hipError_t rs_only(const ReduceArgs& a, const GradPtrs<NW>& g) {
    const int64_t work = a.nvec > 0 ? a.nvec : a.S;
    dim3 grid((unsigned)grid_for(work, a.cus));
    launch(k_reduce_scatter<NW, GF, FP32R>, grid, dim3(kThreads), (hipStream_t)a.stream, g, a.world, a.S,
           a.nvec, a.out, a.rs);
    return hipGetLastError();
}

template <int NW>
static hipError_t rs_grad(const ReduceArgs& a) {
    GradPtrs<NW> g{};
    const int n = NW > 0 ? NW : a.world;
    for (int q = 0; q < n; ++q) g.p[q] = a.grads[q];
    const bool f32r = a.fp32_reduce || a.grad_dt == FSDP_F32;
    if (a.grad_dt == FSDP_F32) return rs_only<NW, FSDP_F32, true>(a, g);
    if (a.grad_dt == FSDP_F16) return f32r ? rs_only<NW, FSDP_F16, true>(a, g) : rs_only<NW, FSDP_F16, false>(a, g);
    return f32r ? rs_only<NW, FSDP_BF16, true>(a, g) : rs_only<NW, FSDP_BF16, false>(a, g);
}

hipError_t launch_reduce_scatter(const ReduceArgs& a) {
    switch (a.world) {
    case 1: return rs_grad<1>(a);
    case 2: return rs_grad<2>(a);
    case 4: return rs_grad<4>(a);
    case 8: return rs_grad<8>(a);
    default: return rs_grad<0>(a);
    }
}

hipError_t launch_gather(const void* const* srcs, void* const* dsts, int n, int64_t bytes, int cus,
                         void* stream) {
    if (n <= 0 || bytes <= 0) return hipSuccess;
    int64_t per = (bytes / 16 + kThreads - 1) / kThreads;
    int64_t cap = ((int64_t)cus * kBlocksPerCU + n - 1) / n;
    if (per > cap) per = cap;
    if (per < 1) per = 1;
    dim3 grid((unsigned)per, (unsigned)n);
    if (n <= 8) {
        CopyList<8> L;
        for (int j = 0; j < n; ++j) { L.src[j] = (const char*)srcs[j]; L.dst[j] = (char*)dsts[j]; }
        launch(k_gather<8>, grid, dim3(kThreads), (hipStream_t)stream, L, bytes);
    } else {
        CopyList<FSDP_MAX_WORLD> L;
        for (int j = 0; j < n; ++j) { L.src[j] = (const char*)srcs[j]; L.dst[j] = (char*)dsts[j]; }
        launch(k_gather<FSDP_MAX_WORLD>, grid, dim3(kThreads), (hipStream_t)stream, L, bytes);
    }
    return hipGetLastError();
}

hipError_t launch_segments(const SegBatch& b, int64_t chunks, void* stream) {
    if (chunks <= 0) return hipSuccess;
    launch(k_segments, dim3((unsigned)chunks), dim3(kThreads), (hipStream_t)stream, b);
    return hipGetLastError();
}

}  // namespace fsdp
