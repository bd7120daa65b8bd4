// fsdp_kernels.hip -- gfx950 (CDNA4) kernels of the FSDP flat-parameter shard
// pipeline.  Every kernel is an HBM stream: no contraction, so no MFMA.
//
// Design (MI355X, 256 CUs in 8 XCDs, 64-wide waves, HBM3E ~8 TB/s):
//  * 16-byte (dwordx4) global loads/stores per lane; a lane owns 8 consecutive
//    elements of the shard per step (one dwordx4 of 16-bit data, two of fp32),
//    except in the unit kernel, whose group layout (load8g in fsdp_device.h)
//    gives each wave access instruction one contiguous span;
//  * one-shot grids: a lane takes one 16-byte vector (8 elements) and the grid
//    has as many workgroups as that needs, up to 2048 per CU; the grid-stride
//    loops of the copy and reduce-scatter kernels make a second trip only
//    beyond that (about 1e9 elements), and the unit kernel, whose launches
//    hold at most 2^26 shard elements, has none (one-shot grids measured 3 to
//    9 points above grid-stride grids of 4 to 16 workgroups per CU);
//  * the N simulated ranks' gradient blocks are accumulated in registers, all N
//    loads issued before the first add (N is a template parameter for
//    N in {1, 2, 4, 8});
//  * reduce-scatter + optimizer step + cast run in one pass over the shard
//    (one read of N gradient blocks and the parameter/state, one write of the
//    parameter/state and the compute copy): the unit kernel, fsdp_units.h,
//    instantiated per optimizer family in fsdp_units_*.hip;
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

#include <algorithm>
#include <vector>

#include "fsdp_device.h"

#pragma clang fp contract(off)

namespace fsdp {

// Reduce-scatter alone: averaged gradient shard in fp32 (fp32 mode) or in the
// gradient format (16-bit mode).  fp32 output: vectors in the group layout
// (load8g / store8g; nvec a multiple of 64, so every wave of the grid-stride
// loop takes one whole group and each store instruction one contiguous span,
// stored with the sc1 policy).  16-bit output: 8 consecutive elements per lane,
// one dwordx4 per lane for every stream.  The gradient loads are non-temporal,
// as in the unit step (each byte is read once).  Measured on block shapes with
// unit pools larger than the last-level cache, TB/s: non-temporal loads +3 to
// +8% on eight shapes (70B N = 8 bf16 -> fp32 6.07-6.14 -> 6.48-6.54); fp32
// output in the group layout against 8 consecutive elements per lane, GPT-2
// Large N = 2 fp16 4.65-4.81 -> 5.42-5.65, 70B N = 8 6.03-6.07 -> 6.50-6.53,
// 13B N = 3 6.05-6.08 -> 6.46-6.51; 16-bit output tied (N = 8) or -2.5%
// (N = 2) in the group layout, so it keeps its own.
template <int NW, int GF, bool FP32R>
__global__ __launch_bounds__(kThreads) void k_reduce_scatter(
    GradPtrs<NW> g, int world, int64_t S, int64_t nvec, void* __restrict__ out, ReduceScalars rs) {
    constexpr int OF = (FP32R || GF == FSDP_F32) ? FSDP_F32 : GF;
    constexpr bool kGroup = OF == FSDP_F32;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const GradsOf<NW> gp{g};
    for (int64_t vi = t0; vi < nvec; vi += stride) {
        float acc[8];
        reduce8<NW, GF, FP32R, true, kGroup>(gp, world, vi, acc);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = finish<NW, GF, FP32R>(acc[k], rs);
        if constexpr (kGroup) store8g<OF>(out, vi, acc);
        else store8<OF>(out, vi, acc);
    }
    for (int64_t i = nvec * 8 + t0; i < S; i += stride)
        store1<OF>(out, i, finish<NW, GF, FP32R>(reduce1<NW, GF, FP32R>(gp, world, i), rs));
}

// Copy `bytes` bytes from src to dst (or write zeros when src is null) with the
// widest access both addresses allow.  Called by every lane of a range of
// `nthreads` lanes, lane index `lane`.  The 16-byte stores of a wave go out as
// one span with the sc1 policy (st16_wave): a 1 GiB copy +2.3%, the segmented
// flatten/unflatten copy +2 to +8% (with 4 KB chunks; with 8 KB chunks it had
// measured 1-3% slower).
__device__ __forceinline__ void copy_range(char* __restrict__ dst, const char* __restrict__ src,
                                           int64_t bytes, int64_t lane, int64_t nthreads) {
    const uintptr_t a = (uintptr_t)dst | (src ? (uintptr_t)src : 0);
    if ((a & 15) == 0) {
        const int64_t nv = bytes >> 4;
        u32x4* d = reinterpret_cast<u32x4*>(dst);
        const u32x4* s = reinterpret_cast<const u32x4*>(src);
        // lane and nthreads are multiples of 64 apart from threadIdx.x % 64, so
        // each wave's lanes cover one 1 KB span per trip
        const int l = (int)(threadIdx.x & 63);
        if (src) {
            for (int64_t i = lane; i < nv; i += nthreads) st16_wave(d + (i - l), l, ld16<true>(s + i));
        } else {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int64_t i = lane; i < nv; i += nthreads) st16_wave(d + (i - l), l, z);
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

// Batched copies: blockIdx.y selects copy j; blocks along x stride over its bytes
// (copies shorter than the longest leave their surplus blocks idle).
__global__ __launch_bounds__(kThreads) void k_copies(CopyBatch L) {
    const int j = blockIdx.y;
    copy_range(L.dst[j], L.src[j], L.bytes[j], (int64_t)blockIdx.x * kThreads + threadIdx.x,
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

void take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = t_ev_start;
    *stop = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
}

static hipError_t launch_units_policy(const UnitArgs* units, int n, const UnitLaunch& L) {
    switch (L.opt.kind) {
    case kOptAdamW: return launch_units_adamw(units, n, L);
    case kOptSgd:
    case kOptSgdMomentum: return launch_units_sgd(units, n, L);
    case kOptAdamax: return launch_units_adamax(units, n, L);
    case kOptAdadelta: return launch_units_adadelta(units, n, L);
    default: return hipErrorInvalidValue;
    }
}

// Units of more than kLaunchShardElems shard elements are stepped as slices
// of that many (a multiple of 512, so every slice keeps 16-byte alignment and
// whole groups): the step is pointwise, so a slice is a unit of its own whose
// pointers start lo elements in.  Measured: GPT-2 XL (one 778.8M-element
// shard) 75.2 -> 77.1% of 8 TB/s, 70B (106.9M) 77.7 -> 78.2% in 2^26-element
// slices; 2^25-element slices gained less and lost on 13B.
hipError_t launch_units(const UnitArgs* units, int n, const UnitLaunch& L) {
    int64_t pieces = 0;
    for (int k = 0; k < n; ++k) pieces += units[k].S > kLaunchShardElems ? slices_of(units[k].S) : 1;
    if (pieces == n) return launch_units_policy(units, n, L);
    const int64_t part = kLaunchShardElems;
    const int64_t gs = dt_bytes(L.grad_dt), ss = dt_bytes(L.state_dt), cs = dt_bytes(L.compute_dt);
    const int np = L.gather ? L.world - 1 : 0;
    std::vector<UnitArgs> out;
    std::vector<std::vector<const void*>> grads, srcs;   // per-slice pointer tables (stable: reserved)
    std::vector<std::vector<void*>> dsts;
    out.reserve(pieces);
    grads.reserve(pieces);
    srcs.reserve(pieces);
    dsts.reserve(pieces);
    for (int k = 0; k < n; ++k) {
        const UnitArgs& a = units[k];
        if (a.S <= part) {
            out.push_back(a);
            continue;
        }
        for (int64_t lo = 0; lo < a.S; lo += part) {
            const int64_t cnt = a.S - lo < part ? a.S - lo : part;
            UnitArgs b = a;
            grads.emplace_back(L.world);
            for (int q = 0; q < L.world; ++q) grads.back()[q] = (const char*)a.grads[q] + lo * gs;
            b.grads = grads.back().data();
            if (np > 0) {
                srcs.emplace_back(np);
                dsts.emplace_back(np);
                for (int q = 0; q < np; ++q) {
                    srcs.back()[q] = (const char*)a.peer_src[q] + lo * cs;
                    dsts.back()[q] = (char*)a.peer_dst[q] + lo * cs;
                }
                b.peer_src = srcs.back().data();
                b.peer_dst = dsts.back().data();
            }
            b.p = (char*)a.p + lo * ss;
            b.m = a.m ? (char*)a.m + lo * ss : nullptr;
            b.v = a.v ? (char*)a.v + lo * ss : nullptr;
            b.out = a.out ? (char*)a.out + lo * cs : nullptr;
            b.out2 = a.out2 ? (char*)a.out2 + lo * cs : nullptr;
            b.S = cnt;
            b.nvec = a.nvec > 0 ? std::min(a.nvec - lo / 8, cnt / 8) : 0;
            out.push_back(b);
        }
    }
    return launch_units_policy(out.data(), (int)out.size(), L);
}

// Dynamic LDS reserved per reduce-scatter workgroup (the kernel uses none), as
// for the unit kernel: with 4 or 8 gradient streams fewer resident workgroups
// stream them through the DRAM faster.  Measured at block shapes (two sweeps,
// separate processes): fp32 output with N = 4 or 8 at 2 workgroups per CU
// +5 to +7% over full occupancy, 16-bit output with N = 8 at 3 per CU +5 to
// +10%; N = 2, the generic kernel and 16-bit output with N = 4 lose with a cap
// (N = 2 16-bit output falls by half: its one-vector workgroups are too short
// for so few to keep the memory busy).
template <int NW, bool kGroup>
constexpr unsigned rs_lds_bytes() {
    if (kGroup && (NW == 4 || NW == 8)) return kUnitLdsBytes;
    if (!kGroup && NW == 8) return kUnitLdsBytes3;
    return 0u;
}

template <int NW, int GF, bool FP32R>
static hipError_t rs_only(const ReduceArgs& a, const GradPtrs<NW>& g) {
    constexpr bool kGroup = FP32R || GF == FSDP_F32;   // fp32 output: the group layout
    const int64_t nvec = kGroup ? a.nvec / 64 * 64 : a.nvec;   // whole groups; the rest is the element tail
    const int64_t work = nvec > 0 ? nvec : a.S;
    dim3 grid((unsigned)grid_for(work, a.cus));
    launch_lds(k_reduce_scatter<NW, GF, FP32R>, grid, dim3(kThreads), rs_lds_bytes<NW, kGroup>(),
               (hipStream_t)a.stream, g, a.world, a.S, nvec, a.out, a.rs);
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

hipError_t launch_copies(const CopyBatch& b, int cus, void* stream) {
    int64_t most = 0;
    for (int j = 0; j < b.count; ++j) most = b.bytes[j] > most ? b.bytes[j] : most;
    if (b.count <= 0 || most <= 0) return hipSuccess;
    int64_t per = (most / 16 + kThreads - 1) / kThreads;
    const int64_t cap = ((int64_t)cus * kBlocksPerCU + b.count - 1) / b.count;
    if (per > cap) per = cap;
    if (per < 1) per = 1;
    launch(k_copies, dim3((unsigned)per, (unsigned)b.count), dim3(kThreads), (hipStream_t)stream, b);
    return hipGetLastError();
}

hipError_t launch_segments(const SegBatch& b, int64_t chunks, void* stream) {
    if (chunks <= 0) return hipSuccess;
    launch(k_segments, dim3((unsigned)chunks), dim3(kThreads), (hipStream_t)stream, b);
    return hipGetLastError();
}

}  // namespace fsdp