// fsdp_kernels.h -- internal interface between the C ABI host layer
// (fsdp_abi.cpp, fsdp_offload.cpp) and the gfx950 kernels.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsdp_shard.h"

namespace fsdp {

#ifndef FSDP_BLOCKS_PER_CU
#define FSDP_BLOCKS_PER_CU 2048
#endif
constexpr int kThreads = 256;                          // 4 wave64 per workgroup
constexpr int kBlocksPerCU = FSDP_BLOCKS_PER_CU;       // grid cap = CUs * kBlocksPerCU (one trip per lane up to ~1e9 elements)
// Dynamic LDS reserved by every unit-kernel workgroup (the kernel uses none):
// with 160 KB of LDS per CU it holds residency at 2 workgroups (8 waves) per
// CU.  Fewer tiles in flight at once streams the unit step's 8-11 address
// streams through HBM measurably faster (+1.5 to +3 points of peak on every
// workload, same-process A/B); the copy kernels, with one load per lane, need
// full occupancy instead and reserve none, and the reduce-scatter alone
// reserves by its number of gradient streams (rs_lds_bytes).
#ifndef FSDP_UNIT_LDS
#define FSDP_UNIT_LDS 81920
#endif
constexpr unsigned kUnitLdsBytes = FSDP_UNIT_LDS;
// 3 per CU instead: measured faster for 16-bit state with N <= 2 (+1.5 to +3.7
// points; with N = 8 it loses 3.7), so those instantiations reserve this.
#ifndef FSDP_UNIT_LDS3
#define FSDP_UNIT_LDS3 53248
#endif
constexpr unsigned kUnitLdsBytes3 = FSDP_UNIT_LDS3;
constexpr int kSegMax = 64;             // segments per flatten/unflatten launch
// Bytes per flatten/unflatten workgroup: one 16-byte vector per lane.  With the
// sc1 store policy 4 KB chunks measured 6.05-6.60 TB/s on the four block shapes
// (70B block 6.61, 13B 6.60-6.62), against 5.90-6.54 with 8 KB chunks (with or
// without the policy); with global stores 8 KB had been best (32 KB 5.5-5.9).
constexpr int64_t kSegChunkBytes = 4096;

// Per-element AdamW constants, computed on the host (double, rounded once).
struct AdamScalars {
    float decay, b1, omb1, b2, omb2, step_size, bc2_sqrt, eps;
};

// The pointwise optimizer of a unit launch and its per-launch scalars
// (host-computed; each policy in fsdp_optim.h reads its own fields).
enum OptKind { kOptAdamW = 0, kOptSgd = 1, kOptSgdMomentum = 2, kOptAdamax = 3, kOptAdadelta = 4 };

struct OptParams {
    int kind;
    AdamScalars adam;                  // AdamW
    float lr, wd;                      // SGD, SGD with momentum, Adadelta (lr); all but AdamW (wd)
    float mu, omd;                     // SGD with momentum: momentum, 1 - dampening
    int first, nesterov;               // SGD with momentum: step == 1, Nesterov
    float clr, b1, omb1, b2;           // Adamax: lr / (1 - beta1^t), betas
    float eps;                         // Adamax, Adadelta
    float rho, omr;                    // Adadelta
};

// Division by N (n) or, for specialised power-of-two N, product with 1/N.
struct ReduceScalars {
    float n, inv_n;
};

template <int NW>
struct GradPtrs {
    const void* p[NW > 0 ? NW : FSDP_MAX_WORLD];
};

// Table of up to kMax units stepped by one launch of the unit kernel; it
// travels in the kernel arguments, so each table stays under 4000 bytes.  Gradient pointers are already offset to block
// `rank`; psrc/pdst are the peers' compute shards and their slots in the full
// buffer (unit step only).
template <int NW>
struct UnitBatch {
    static constexpr int kMax = NW == 0 ? 1 : (NW <= 2 ? 40 : (NW <= 4 ? 24 : 16));
    static constexpr int kG = NW > 0 ? NW : FSDP_MAX_WORLD;
    static constexpr int kP = NW > 1 ? NW - 1 : (NW == 1 ? 1 : FSDP_MAX_WORLD - 1);
    int32_t count;
    int32_t world;
    int32_t npeers;
    int64_t tile_begin[kMax + 1];
    int64_t nvec[kMax];            // vectors, whole 64-vector groups (the rest: single elements)
    int64_t S[kMax];
    void* p[kMax];                 // state: fp32 master/m/v, or 16-bit parameter/m/v
    void* m[kMax];
    void* v[kMax];
    void* out[kMax];
    void* out2[kMax];
    const void* g[kMax][kG];
    const char* psrc[kMax][kP];
    char* pdst[kMax][kP];
};
static_assert(sizeof(UnitBatch<1>) <= 4000 && sizeof(UnitBatch<2>) <= 4000 && sizeof(UnitBatch<4>) <= 4000 &&
                  sizeof(UnitBatch<8>) <= 4000 && sizeof(UnitBatch<0>) <= 4000,
              "unit tables travel in kernel arguments");

template <int MAXN>
struct CopyList {
    const char* src[MAXN];
    char* dst[MAXN];
};

// Batched copies (the peers' slots of the full buffers of a table of units):
// copy j moves bytes[j] bytes src[j] -> dst[j].
struct CopyBatch {
    static constexpr int kMax = 128;
    int32_t count;
    const char* src[kMax];
    char* dst[kMax];
    int64_t bytes[kMax];
};
static_assert(sizeof(CopyBatch) <= 4000, "copy tables travel in kernel arguments");

struct SegBatch {
    int32_t count;
    int64_t chunk_begin[kSegMax + 1];
    const char* src[kSegMax];   // null: zero fill
    char* dst[kSegMax];
    int64_t bytes[kSegMax];
};

// One unit of a unit-kernel launch (host side).
struct UnitArgs {
    const void* const* grads;      // world pointers, already offset to block `rank`
    const void* const* peer_src;   // world - 1 peer compute shards (gather only)
    void* const* peer_dst;         // their slots in the full buffer
    void* p;                       // state of format state_dt (UnitLaunch)
    void* m;
    void* v;
    void* out;                     // compute shard, or this rank's slot of the full buffer
    void* out2;                    // optional extra copy of the compute shard
    int64_t S;
    int64_t nvec;                  // 8-element vectors on the wide path (0: every element scalar)
};

// What every unit of one launch shares.
struct UnitLaunch {
    int world;
    int grad_dt;
    int fp32_reduce;
    int compute_dt;
    int state_dt;                  // FSDP_F32, or the 16-bit format shared with compute_dt
    bool gather;
    ReduceScalars rs;
    OptParams opt;
    int cus;                       // compute units of the device (grid caps)
    void* stream;
};

struct ReduceArgs {
    const void* const* grads;      // world pointers, already offset to block `rank`
    int world;
    int grad_dt;
    int fp32_reduce;
    int64_t S;
    int64_t nvec;
    void* out;
    ReduceScalars rs;
    int cus;
    void* stream;
};

hipError_t launch_units(const UnitArgs* units, int n, const UnitLaunch& L);
// per optimizer family (fsdp_units_*.hip)
hipError_t launch_units_adamw(const UnitArgs* units, int n, const UnitLaunch& L);
hipError_t launch_units_sgd(const UnitArgs* units, int n, const UnitLaunch& L);
hipError_t launch_units_adamax(const UnitArgs* units, int n, const UnitLaunch& L);
hipError_t launch_units_adadelta(const UnitArgs* units, int n, const UnitLaunch& L);
hipError_t launch_reduce_scatter(const ReduceArgs& a);
void set_launch_events(void* start, void* stop);
hipError_t launch_copies(const CopyBatch& b, int cus, void* stream);

// Packing of a unit-step call into launches: up to UnitBatch<NW>::kMax units
// (unit_table_max) and at most kLaunchShardElems shard elements in all per
// launch; a larger unit is stepped in slices of kLaunchShardElems elements, a
// launch each (launch_units).  The element cap was
// measured faster than one launch per table on every shape (same box, two
// repetitions, % of 8 TB/s: GPT-2 Large x36 75.3 -> 76.9 with AdamW, +1.4
// Adamax, +1.3 SGD, +0.6 bf16 state; 13B +0.3; 70B +1.0); a cap of 2^25 gained
// less, 5e7 about the same.
constexpr int64_t kLaunchShardElems = int64_t(1) << 26;
static_assert(kLaunchShardElems % 512 == 0, "slices keep whole groups");
inline int64_t slices_of(int64_t S) { return (S + kLaunchShardElems - 1) / kLaunchShardElems; }
inline int64_t dt_bytes(int dt) { return dt == FSDP_F32 ? 4 : 2; }
inline int unit_table_max(int world) {
    return world == 1 || world == 2 ? UnitBatch<2>::kMax : world == 4 ? UnitBatch<4>::kMax
         : world == 8 ? UnitBatch<8>::kMax : UnitBatch<0>::kMax;
}
// Units (of shard sizes S[0..n), n >= 1) the next launch takes, at least one,
// and the shard elements it covers (the first slice of a unit larger than the cap).
inline int units_in_launch(int world, const int64_t* S, int n, int64_t* elems) {
    if (S[0] > kLaunchShardElems) {
        *elems = kLaunchShardElems;
        return 1;
    }
    const int cap = unit_table_max(world);
    int64_t packed = 0;
    int c = 0;
    for (; c < cap && c < n; ++c) {
        if (S[c] > kLaunchShardElems || (c > 0 && packed + S[c] > kLaunchShardElems)) break;
        packed += S[c];
    }
    *elems = packed;
    return c;
}

// Whether a unit-step launch with a gather, over `elems` shard elements in
// all, leaves the peers' copies to a launch of their own (peer_copies in
// fsdp_units.h): an optimizer that keeps state and at least 2^24 shard
// elements, for fp32 and 16-bit state alike; otherwise the step's own trip
// copies them.  (16-bit state kept the fused form while its bf16 roundings
// were five instructions and a branch each: its step launch alone was bound by
// the VALU, 70% busy, and the split lost.)
constexpr int64_t kSplitGatherElems = int64_t(1) << 24;
inline bool split_gather(int state_dt, int n_states, int64_t elems) {
    (void)state_dt;
    return n_states >= 1 && elems >= kSplitGatherElems;
}
hipError_t launch_gather(const void* const* srcs, void* const* dsts, int n, int64_t bytes, int cus,
                         void* stream);
hipError_t launch_segments(const SegBatch& b, int64_t chunks, void* stream);

}  // namespace fsdp
