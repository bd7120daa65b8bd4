// fsdp_kernels.h -- internal interface between the C ABI host layer
// (fsdp_abi.cpp part of fsdp_shard.hip) and the gfx950 kernels.  Not installed.
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
constexpr int kSegMax = 64;             // segments per flatten/unflatten launch
constexpr int64_t kSegChunkBytes = 32768;

// Per-element AdamW constants, computed on the host (double, rounded once).
struct AdamScalars {
    float decay, b1, omb1, b2, omb2, step_size, bc2_sqrt, eps;
};

// Division by N (n) or, for specialised power-of-two N, product with 1/N.
struct ReduceScalars {
    float n, inv_n;
};

template <int NW>
struct GradPtrs {
    const void* p[NW > 0 ? NW : FSDP_MAX_WORLD];
};

// Peer compute shards copied into their slots of the full buffer by the
// one-launch unit step: world - 1 (src, dst) pairs.
template <int NW>
struct PeerPtrs {
    const char* src[NW > 1 ? NW - 1 : (NW == 1 ? 1 : FSDP_MAX_WORLD - 1)];
    char* dst[NW > 1 ? NW - 1 : (NW == 1 ? 1 : FSDP_MAX_WORLD - 1)];
};

template <int MAXN>
struct CopyList {
    const char* src[MAXN];
    char* dst[MAXN];
};

struct SegBatch {
    int32_t count;
    int64_t chunk_begin[kSegMax + 1];
    const char* src[kSegMax];   // null: zero fill
    char* dst[kSegMax];
    int64_t bytes[kSegMax];
};

struct FusedArgs {
    const void* const* grads;  // world pointers, already offset to block `rank`
    int world;
    int grad_dt;
    int fp32_reduce;
    int compute_dt;
    int64_t S;
    int64_t nvec;              // 8-element vectors taken by the wide path
    float* p;
    float* m;
    float* v;
    void* out;                 // compute shard (fused) or grad shard (reduce only)
    void* out2;                // optional second copy of the compute shard, or null
    const void* const* peer_src;  // world - 1 peer shards (unit step only)
    void* const* peer_dst;        // their slots in the full buffer
    int npeers;                // > 0 selects the unit-step kernel (fused + gather)
    ReduceScalars rs;
    AdamScalars as;
    int cus;
    void* stream;
};

hipError_t launch_fused(const FusedArgs& a, bool fused);
void set_launch_events(void* start, void* stop);
hipError_t launch_gather(const void* const* srcs, void* const* dsts, int n, int64_t bytes, int cus,
                         void* stream);
hipError_t launch_segments(const SegBatch& b, int64_t chunks, void* stream);

}  // namespace fsdp
