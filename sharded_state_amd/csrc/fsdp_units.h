// fsdp_units.h -- the fused unit kernel of libfsdp_shard.so: reduce-scatter
// of the N ranks' gradient blocks, a pointwise optimizer step on the rank's
// shard, the cast to the compute format and the write of the own slot of the
// full buffer, for a table of units per launch; then the rest of the
// all-gather (the peers' slots): in the step's own trip, or as a batched copy
// launch of its own where that was measured faster (peer_copies).  Templated on the optimizer
// policy (fsdp_optim.h); each optimizer family is instantiated in a
// translation unit of its own (fsdp_units_*.hip).  Not installed.
//
// Sources: "Fully Sharded Data Parallel: faster AI training with fewer GPUs"
// (techreport.ngo), "From all-reduce to sharded parameters" (reduce-scatter
// and all-gather figure, forward/backward pseudo-code); "FSDP (Fully Sharded
// Data Parallel)" (vanos001 notes), "The Per-Layer Communication" and "Mixed
// Precision and FSDP"; "fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战
// 指南" (zskr.cn), "工作原理" and "限制与兼容性说明".
#pragma once

#include "fsdp_device.h"
#include "fsdp_optim.h"

#pragma clang fp contract(off)

namespace fsdp {

// ----------------------------------------------------------------- kernels
// One unit's step on vector vi (8 elements of a whole group in the group
// layout, load8g; for bf16 state, 8 consecutive elements, load8):
// every load first (the N gradient blocks, the parameter and
// the optimizer's state, the peers' compute vectors), then the math, then every
// store.  With GATHER, `out` is this rank's slot of the full buffer and the
// peers' vectors are copied into their slots (the copy moves the group's bytes
// in contiguous 1 KB spans per instruction whatever the format).
template <class OPT, int NW, int GF, bool FP32R, int CF, bool GATHER, int SF>
__device__ __forceinline__ void unit_vec(const UnitBatch<NW>& B, int u, int64_t vi, const ReduceScalars& rs,
                                         const OPT& op) {
    constexpr int kW = CF == FSDP_F32 ? 2 : 1;      // dwordx4 per 8 compute elements
    constexpr int kP = NW > 1 ? NW - 1 : 1;
    void* __restrict__ p = B.p[u];
    void* __restrict__ m = B.m[u];
    void* __restrict__ v = B.v[u];
    float acc[8], pp[8], mm[8] = {}, vv[8] = {};
    const int64_t g = vi >> 6, l = vi & 63;
    auto pv = [&](int w) -> int64_t { return g * (64 * kW) + w * 64 + l; };   // 16-byte index in the group
    u32x4 peer[kP][kW];
    if constexpr (GATHER && NW > 1) {
#pragma unroll
        for (int j = 0; j < NW - 1; ++j)
#pragma unroll
            for (int w = 0; w < kW; ++w) peer[j][w] = ld16<true>(reinterpret_cast<const u32x4*>(B.psrc[u][j]) + pv(w));
    }
    // parameter/state loads: non-temporal for fp32 state, and for 16-bit state
    // with more than two ranks; plain for 16-bit state with N <= 2 (+0.8 points
    // there; the hint gains 0.5 to 3 points on the fp32-state shapes and 0.7 on
    // the N = 8 bf16-state shape; same box, same bench)
    constexpr bool kNtState = SF == FSDP_F32 || NW == 0 || NW > 2;
    // bf16 state (every stream 16-bit): 8 consecutive elements per lane, one
    // dwordx4 per stream (+2.1 to +2.5 points against the group layout on GPT-2
    // Large and XL; with N = 8 once the peers' copies left the step's trip, 13B
    // +0.7 to +0.8 and 70B +0.5 to +1.1 on two boxes; fp16 state lost 2.2 with
    // N = 2, so it and fp32 state keep the group layout)
    constexpr bool kG = SF != FSDP_BF16;
    load8x<SF, kNtState, kG>(p, vi, pp);
    if constexpr (OPT::kStates >= 1) load8x<SF, kNtState, kG>(m, vi, mm);
    if constexpr (OPT::kStates >= 2) load8x<SF, kNtState, kG>(v, vi, vv);
    reduce8<NW, GF, FP32R, true, kG>(UnitGrads<NW>{B, u}, B.world, vi, acc);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the math
#pragma unroll
    for (int k = 0; k < 8; ++k) op(finish<NW, GF, FP32R>(acc[k], rs), pp[k], mm[k], vv[k]);
    if constexpr (OPT::kStorePace > 0 && NW >= 1 && NW <= 2) __builtin_amdgcn_s_sleep(OPT::kStorePace);
    store8x<SF, kG>(p, vi, pp);
    if constexpr (OPT::kStates >= 1) store8x<SF, kG>(m, vi, mm);
    if constexpr (OPT::kStates >= 2) store8x<SF, kG>(v, vi, vv);
    void* out = B.out[u];
    void* out2 = B.out2[u];
    if constexpr (GATHER) {
        // the unit step always has its own slot; keep the peer stores in the
        // same basic block as their loads so they are not sunk past the math
        store8x<CF, kG>(out, vi, pp);
        if constexpr (NW > 1) {
#pragma unroll
            for (int j = 0; j < NW - 1; ++j)
#pragma unroll
                for (int w = 0; w < kW; ++w)
                    st16_wave(reinterpret_cast<u32x4*>(B.pdst[u][j]) + (pv(w) - l), (int)l, peer[j][w]);
        } else if constexpr (NW == 0) {
            for (int j = 0; j < B.npeers; ++j)
#pragma unroll
                for (int w = 0; w < kW; ++w)
                    st16_wave(reinterpret_cast<u32x4*>(B.pdst[u][j]) + (pv(w) - l), (int)l,
                              ld16<true>(reinterpret_cast<const u32x4*>(B.psrc[u][j]) + pv(w)));
        }
    } else {
        if (out) store8x<CF, kG>(out, vi, pp);
    }
    // non-temporal like every other output: plain stores, which keep this
    // persistent copy in the caches, win only when the next all-gather follows
    // the step at once and lose when it comes after other units' work
    if (out2) store8x<CF, kG>(out2, vi, pp);
}

// Element i of unit u, one lane (the tail past the last full vector, or every
// element of a unit whose buffers are not 16-byte aligned).
template <class OPT, int NW, int GF, bool FP32R, int CF, bool GATHER, int SF>
__device__ __forceinline__ void unit_elem(const UnitBatch<NW>& B, int u, int64_t i, const ReduceScalars& rs,
                                          const OPT& op) {
    void* __restrict__ p = B.p[u];
    void* __restrict__ m = B.m[u];
    void* __restrict__ v = B.v[u];
    float pp = load1<SF>(p, i), mm = 0.0f, vv = 0.0f;
    if constexpr (OPT::kStates >= 1) mm = load1<SF>(m, i);
    if constexpr (OPT::kStates >= 2) vv = load1<SF>(v, i);
    op(finish<NW, GF, FP32R>(reduce1<NW, GF, FP32R>(UnitGrads<NW>{B, u}, B.world, i), rs), pp, mm, vv);
    store1<SF>(p, i, pp);
    if constexpr (OPT::kStates >= 1) store1<SF>(m, i, mm);
    if constexpr (OPT::kStates >= 2) store1<SF>(v, i, vv);
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

// Fused reduce-scatter + optimizer step + cast (+ all-gather with GATHER) over the
// shards of up to UnitBatch<NW>::kMax units in one launch.  Workgroup b owns
// tile b: unit u holds tiles [tile_begin[u], tile_begin[u+1]); its first
// ceil(nvec/256) tiles are 256 vectors of 8 elements each (nvec a multiple of
// 64: whole groups, so each wave is either wholly in range or wholly out), the
// rest 256 single elements (the tail of fewer than 520 elements, or the whole
// unit when unaligned).  One launch pays the ramp-up and drain of the grid once
// for all its units.
// SF is the state format: FSDP_F32 for fp32 master/m/v with a separate compute
// copy of format CF, or a 16-bit format (CF == SF) where the parameter shard is
// itself the compute copy.
template <class OPT, int NW, int GF, bool FP32R, int CF, bool GATHER, int SF>
__global__ __launch_bounds__(kThreads) void k_units(UnitBatch<NW> B, ReduceScalars rs, OPT op) {
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
        if (vi < nvec) unit_vec<OPT, NW, GF, FP32R, CF, GATHER, SF>(B, u, vi, rs, op);
    } else {
        const int64_t i = nvec * 8 + (j - tv) * kThreads + threadIdx.x;
        if (i < B.S[u]) unit_elem<OPT, NW, GF, FP32R, CF, GATHER, SF>(B, u, i, rs, op);
    }
}

// ----------------------------------------------------------------- launchers
template <class OPT, int NW, int GF, bool FP32R, int CF, int SF>
static hipError_t units_go(const UnitBatch<NW>& B, int64_t tiles, bool gather, const ReduceScalars& rs,
                           const OPT& op, hipStream_t st) {
    constexpr unsigned lds = (SF != FSDP_F32 && NW >= 1 && NW <= 2) ? kUnitLdsBytes3 : kUnitLdsBytes;
    if (gather)
        launch_lds(k_units<OPT, NW, GF, FP32R, CF, true, SF>, dim3((unsigned)tiles), dim3(kThreads), lds, st, B, rs,
                   op);
    else
        launch_lds(k_units<OPT, NW, GF, FP32R, CF, false, SF>, dim3((unsigned)tiles), dim3(kThreads), lds, st, B, rs,
                   op);
    return hipGetLastError();
}

template <class OPT, int NW, int GF, bool FP32R>
static hipError_t units_cf(const UnitBatch<NW>& B, int64_t tiles, const UnitLaunch& L, const OPT& op,
                           hipStream_t st) {
    if constexpr (OPT::kState16) {
        if (L.state_dt == FSDP_F16)
            return units_go<OPT, NW, GF, FP32R, FSDP_F16, FSDP_F16>(B, tiles, L.gather, L.rs, op, st);
        if (L.state_dt == FSDP_BF16)
            return units_go<OPT, NW, GF, FP32R, FSDP_BF16, FSDP_BF16>(B, tiles, L.gather, L.rs, op, st);
    } else if (L.state_dt != FSDP_F32) {
        return hipErrorInvalidValue;          // rejected by the host layer first
    }
    switch (L.compute_dt) {
    case FSDP_F32: return units_go<OPT, NW, GF, FP32R, FSDP_F32, FSDP_F32>(B, tiles, L.gather, L.rs, op, st);
    case FSDP_F16: return units_go<OPT, NW, GF, FP32R, FSDP_F16, FSDP_F32>(B, tiles, L.gather, L.rs, op, st);
    default: return units_go<OPT, NW, GF, FP32R, FSDP_BF16, FSDP_F32>(B, tiles, L.gather, L.rs, op, st);
    }
}

template <class OPT, int NW>
static hipError_t units_batch(const UnitBatch<NW>& B, int64_t tiles, const UnitLaunch& L, const OPT& op) {
    hipStream_t st = (hipStream_t)L.stream;
    const bool f32r = L.fp32_reduce || L.grad_dt == FSDP_F32;
    if (L.grad_dt == FSDP_F32) return units_cf<OPT, NW, FSDP_F32, true>(B, tiles, L, op, st);
    if (L.grad_dt == FSDP_F16) {
        if (f32r) return units_cf<OPT, NW, FSDP_F16, true>(B, tiles, L, op, st);
        return units_cf<OPT, NW, FSDP_F16, false>(B, tiles, L, op, st);
    }
    if (f32r) return units_cf<OPT, NW, FSDP_BF16, true>(B, tiles, L, op, st);
    return units_cf<OPT, NW, FSDP_BF16, false>(B, tiles, L, op, st);
}

// The all-gather of a table of units after their step: every unit's N-1 peer
// shards copied into their slots of its full buffer, batched into launches of
// up to CopyBatch::kMax copies.
//
// When split_gather() holds, the step and the copies run as two launches: the
// fused form (the peer copies in the step's own trip, GATHER = true) keeps 8 to
// 26 address streams in flight at once, and draining the step before the copies
// start was measured faster for fp32 state with an optimizer that keeps state
// (same box, two repetitions, % of 8 TB/s for the whole step: GPT-2 Large x36
// 73.1 -> 75.5, GPT-2 XL 74.7 -> 76.0, 13B x40 72.0 -> 78.7, 70B x96 69.9 ->
// 77.2; Adamax and SGD with momentum +1.7 and +2.2 points), and, once the bf16
// rounding became one conversion instruction, for 16-bit state too (70B x96
// with bf16 state 75.2-75.4 -> 77.8-78.5, 13B x40 +0.8).  The fused form stays
// where the second launch lost: SGD without momentum (1.9 points) and launches
// of fewer than 2^24 shard elements (GPT-2 Large, one 9.8M-element unit per
// launch: 2.1 points).  The copies as workgroups of the same launch, after the
// step's tiles, lost to both forms.
template <int NW>
static hipError_t peer_copies(const UnitBatch<NW>& B, int c, const UnitLaunch& L) {
    const int64_t cs = L.compute_dt == FSDP_F32 ? 4 : 2;
    CopyBatch cb;
    cb.count = 0;
    for (int k = 0; k < c; ++k)
        for (int q = 0; q < B.npeers; ++q) {
            if (cb.count == CopyBatch::kMax) {
                hipError_t e = launch_copies(cb, L.cus, L.stream);
                if (e != hipSuccess) return e;
                cb.count = 0;
            }
            cb.src[cb.count] = B.psrc[k][q];
            cb.dst[cb.count] = B.pdst[k][q];
            cb.bytes[cb.count] = B.S[k] * cs;
            ++cb.count;
        }
    return launch_copies(cb, L.cus, L.stream);
}

// Pack the units into tables (units_in_launch: at most kMax units and
// kLaunchShardElems shard elements) and launch one grid per table.
template <class OPT, int NW>
static hipError_t units_all(const UnitArgs* units, int n, const UnitLaunch& L, const OPT& op) {
    constexpr int kMax = UnitBatch<NW>::kMax;
    int done = 0;
    while (done < n) {
        UnitBatch<NW> B{};
        B.world = L.world;
        B.npeers = L.gather ? L.world - 1 : 0;
        int64_t tiles = 0;
        int c = 0;
        int64_t packed = 0;
        for (; c < kMax && done + c < n; ++c) {
            const UnitArgs& a = units[done + c];
            if (c > 0 && packed + a.S > kLaunchShardElems) break;   // as units_in_launch
            packed += a.S;
            B.tile_begin[c] = tiles;
            const int64_t nvec = a.nvec & ~int64_t(63);   // whole groups; the rest joins the tail
            B.nvec[c] = nvec;
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
            tiles += (nvec + kThreads - 1) / kThreads + (a.S - 8 * nvec + kThreads - 1) / kThreads;
        }
        B.count = c;
        B.tile_begin[c] = tiles;
        done += c;
        if (tiles == 0) continue;
        int64_t elems = 0;
        for (int k = 0; k < c; ++k) elems += B.S[k];
        if (L.gather && split_gather(L.state_dt, OPT::kStates, elems)) {
            // the step writes the own slot, then one launch copies every
            // unit's peer shards into their slots (peer_copies)
            UnitLaunch L1 = L;
            L1.gather = false;
            hipError_t e = units_batch<OPT, NW>(B, tiles, L1, op);
            if (e == hipSuccess) e = peer_copies(B, c, L);
            if (e != hipSuccess) return e;
            continue;
        }
        hipError_t e = units_batch<OPT, NW>(B, tiles, L, op);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Every unit of a launch with optimizer policy `op`.
template <class OPT>
static hipError_t launch_units_with(const UnitArgs* units, int n, const UnitLaunch& L, const OPT& op) {
    switch (L.world) {
    case 1: return units_all<OPT, 1>(units, n, L, op);
    case 2: return units_all<OPT, 2>(units, n, L, op);
    case 4: return units_all<OPT, 4>(units, n, L, op);
    case 8: return units_all<OPT, 8>(units, n, L, op);
    default: return units_all<OPT, 0>(units, n, L, op);
    }
}

}  // namespace fsdp
