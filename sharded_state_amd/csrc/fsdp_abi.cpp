// fsdp_abi.cpp -- host layer of libfsdp_shard.so: argument validation, alias
// checks, host-side scalars, launch geometry and error reporting for the C ABI
// declared in include/fsdp_shard.h.  Every check runs before anything is
// enqueued; a negative status means nothing was launched.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fsdp_internal.h"
#include "fsdp_kernels.h"
#include "fsdp_shard.h"

namespace fsdp {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    set_launch_events(nullptr, nullptr);   // a failed call consumes pending timing events
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    set_launch_events(nullptr, nullptr);   // consumed even when nothing was launched
    g_err[0] = 0;
    return FSDP_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(FSDP_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(int dt) { return dt == FSDP_F32 || dt == FSDP_F16 || dt == FSDP_BF16; }
int64_t dt_size(int dt) { return dt == FSDP_F32 ? 4 : 2; }

const char* last_error() { return g_err; }

// AdamW constants: the per-element update uses these fp32 values.
AdamScalars adam_scalars(const fsdp_adamw_hp& hp) {
    const double b1 = hp.beta1, b2 = hp.beta2, lr = hp.lr, t = (double)hp.step;
    const double bias1 = 1.0 - std::pow(b1, t);
    const double bias2 = 1.0 - std::pow(b2, t);
    AdamScalars s;
    s.decay = (float)(1.0 - lr * (double)hp.weight_decay);
    s.b1 = hp.beta1;
    s.omb1 = 1.0f - hp.beta1;
    s.b2 = hp.beta2;
    s.omb2 = 1.0f - hp.beta2;
    s.step_size = (float)(lr / bias1);
    s.bc2_sqrt = (float)std::sqrt(bias2);
    s.eps = hp.eps;
    return s;
}

static std::atomic<int> g_cus[64];
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev >= 0 && dev < 64) g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

ReduceScalars reduce_scalars(int world) {
    ReduceScalars r;
    r.n = (float)world;
    r.inv_n = (float)(1.0 / (double)world);
    return r;
}

int check_hp(const char* fn, const fsdp_adamw_hp* hp) {
    if (!hp) return fail(FSDP_E_INVAL, "%s: hp is NULL", fn);
    if (hp->step < 1) return fail(FSDP_E_INVAL, "%s: hp->step = %lld < 1", fn, (long long)hp->step);
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(FSDP_E_INVAL, "%s: betas must lie in [0, 1)", fn);
    // the same ranges as fsdp_step_units_optim's AdamW; NaN fails every comparison
    if (!(hp->lr >= 0.0f) || !(hp->weight_decay >= 0.0f) || !(hp->eps >= 0.0f))
        return fail(FSDP_E_INVAL, "%s: lr, weight_decay and eps must be >= 0", fn);
    return FSDP_OK;
}

}  // namespace fsdp

namespace {

using fsdp::dt_size;
using fsdp::fail;
using fsdp::hip_fail;
using fsdp::ok;
using fsdp::valid_dtype;
using fsdp::adam_scalars;
using fsdp::check_hp;
using fsdp::cu_count;
using fsdp::reduce_scalars;

// Byte range [lo, lo + n) of device memory.
struct Range {
    uintptr_t lo;
    uint64_t n;
};
Range range(const void* p, int64_t elems, int64_t esize) {
    return Range{(uintptr_t)p, (uint64_t)elems * (uint64_t)esize};
}
bool overlaps(Range a, Range b) {
    if (a.n == 0 || b.n == 0) return false;
    return a.lo < b.lo + b.n && b.lo < a.lo + a.n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Shared validation of world / rank / shard size.
int check_world(int32_t world, int32_t rank, int64_t S) {
    if (world < 1 || world > FSDP_MAX_WORLD)
        return fail(FSDP_E_INVAL, "world = %d outside [1, %d]", world, FSDP_MAX_WORLD);
    if (rank < 0 || rank >= world) return fail(FSDP_E_INVAL, "rank = %d outside [0, %d)", rank, world);
    if (S < 0) return fail(FSDP_E_INVAL, "shard_numel = %lld < 0", (long long)S);
    if (S > fsdp::kMaxElems / world)
        return fail(FSDP_E_SIZE, "shard_numel = %lld times world = %d is too large", (long long)S, world);
    return FSDP_OK;
}

// Rank `rank`'s block of each rank's gradient, recorded as inputs.
int grad_blocks(const void* const* rank_grads, int32_t world, int32_t rank, int64_t S, int grad_dt,
                std::vector<const void*>& blocks, std::vector<Range>& ins) {
    if (!valid_dtype(grad_dt)) return fail(FSDP_E_DTYPE, "grad dtype %d unsupported", grad_dt);
    blocks.assign(world, nullptr);
    if (S == 0) return FSDP_OK;
    if (!rank_grads) return fail(FSDP_E_INVAL, "rank_grads is NULL");
    const int64_t g = dt_size(grad_dt);
    for (int q = 0; q < world; ++q) {
        if (!rank_grads[q]) return fail(FSDP_E_INVAL, "rank_grads[%d] is NULL", q);
        blocks[q] = (const char*)rank_grads[q] + (int64_t)rank * S * g;
        ins.push_back(range(blocks[q], S, g));
    }
    return FSDP_OK;
}

// No two outputs overlap and no output overlaps an input (all non-empty).
bool disjoint(std::vector<Range> outs, const std::vector<Range>& ins) {
    outs.erase(std::remove_if(outs.begin(), outs.end(), [](const Range& r) { return r.n == 0; }), outs.end());
    std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < outs.size(); ++i)
        if (outs[i].lo < outs[i - 1].lo + outs[i - 1].n) return false;
    for (const Range& r : ins) {
        if (r.n == 0) continue;
        // the last output starting below r's end is the only one that can reach into r
        auto it = std::lower_bound(outs.begin(), outs.end(), r.lo + r.n,
                                   [](const Range& a, uintptr_t v) { return a.lo < v; });
        if (it != outs.begin() && overlaps(*(it - 1), r)) return false;
    }
    return true;
}

// One unit of an AdamW launch: validated, with its pointer tables.
struct UnitBuild {
    std::vector<const void*> grads;
    std::vector<const void*> psrc;
    std::vector<void*> pdst;
    fsdp::UnitArgs a{};
};

// Validate unit `idx` (fused step; with full_out the all-gather too) and fill ub.
int build_unit(const char* fn, int idx, void* master, void* exp_avg, void* exp_avg_sq, int n_states, int state_dt,
               const void* const* rank_grads, int32_t world, int32_t rank, int grad_dt, int compute_dt,
               int64_t S, void* compute_shard, const void* const* peer_shards, void* full_out, bool gather,
               UnitBuild& ub, std::vector<Range>& ins, std::vector<Range>& outs) {
    int rc = check_world(world, rank, S);
    if (rc) return rc;
    rc = grad_blocks(rank_grads, world, rank, S, grad_dt, ub.grads, ins);
    if (rc) return rc;
    ub.a.grads = ub.grads.data();
    ub.a.S = S;
    if (S == 0) return FSDP_OK;
    if (!master) return fail(FSDP_E_INVAL, "%s: unit %d: master is NULL", fn, idx);
    if (n_states >= 1 && !exp_avg) return fail(FSDP_E_INVAL, "%s: unit %d: exp_avg is NULL", fn, idx);
    if (n_states >= 2 && !exp_avg_sq) return fail(FSDP_E_INVAL, "%s: unit %d: exp_avg_sq is NULL", fn, idx);
    if (n_states < 2) exp_avg_sq = nullptr;   // not kept by the optimizer: never touched
    if (n_states < 1) exp_avg = nullptr;
    const int64_t cs = dt_size(compute_dt);
    void* own = compute_shard;
    void* out2 = nullptr;
    if (gather) {
        if (!full_out) return fail(FSDP_E_INVAL, "%s: unit %d: full_out is NULL", fn, idx);
        if (world > 1 && !peer_shards) return fail(FSDP_E_INVAL, "%s: unit %d: peer_shards is NULL", fn, idx);
        const int64_t bytes = S * cs;
        for (int q = 0; q < world; ++q) {
            char* slot = (char*)full_out + (int64_t)q * bytes;
            outs.push_back(range(slot, S, cs));
            if (q == rank) continue;
            if (!peer_shards[q]) return fail(FSDP_E_INVAL, "%s: unit %d: peer_shards[%d] is NULL", fn, idx, q);
            ub.psrc.push_back(peer_shards[q]);
            ub.pdst.push_back(slot);
            ins.push_back(range(peer_shards[q], S, cs));
        }
        own = (char*)full_out + (int64_t)rank * bytes;
        out2 = compute_shard;
        if (out2) outs.push_back(range(out2, S, cs));
    } else if (own) {
        outs.push_back(range(own, S, cs));
    }
    const int64_t ss = dt_size(state_dt);
    outs.push_back(range(master, S, ss));
    if (exp_avg) outs.push_back(range(exp_avg, S, ss));
    if (exp_avg_sq) outs.push_back(range(exp_avg_sq, S, ss));

    bool vec = aligned16(master) && (!exp_avg || aligned16(exp_avg)) && (!exp_avg_sq || aligned16(exp_avg_sq)) &&
               (!own || aligned16(own)) && (!out2 || aligned16(out2));
    for (int q = 0; q < world; ++q) vec = vec && aligned16(ub.grads[q]);
    for (size_t j = 0; j < ub.psrc.size(); ++j) vec = vec && aligned16(ub.psrc[j]) && aligned16(ub.pdst[j]);
    ub.a.peer_src = ub.psrc.data();
    ub.a.peer_dst = ub.pdst.data();
    ub.a.p = master;
    ub.a.m = exp_avg;
    ub.a.v = exp_avg_sq;
    ub.a.out = own;
    ub.a.out2 = out2;
    ub.a.nvec = vec ? S / 8 : 0;
    return FSDP_OK;
}

// The AdamW policy's scalars (hp validated).
fsdp::OptParams adamw_params(const fsdp_adamw_hp& hp) {
    fsdp::OptParams op{};
    op.kind = fsdp::kOptAdamW;
    op.adam = adam_scalars(hp);
    return op;
}

// Validate an optimizer's hyper-parameters; fill its policy scalars and the
// number of state buffers it keeps.
int optim_params(const char* fn, const fsdp_optim_hp* hp, fsdp::OptParams& op, int& n_states) {
    if (!hp) return fail(FSDP_E_INVAL, "%s: hp is NULL", fn);
    if (hp->step < 1) return fail(FSDP_E_INVAL, "%s: hp->step = %lld < 1", fn, (long long)hp->step);
    if (!(hp->lr >= 0.0f) || !(hp->weight_decay >= 0.0f))
        return fail(FSDP_E_INVAL, "%s: lr and weight_decay must be >= 0", fn);
    const bool betas = hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f;
    op = fsdp::OptParams{};
    op.lr = hp->lr;
    op.wd = hp->weight_decay;
    op.eps = hp->eps;
    switch (hp->kind) {
    case FSDP_OPT_ADAMW: {
        if (!betas || !(hp->eps >= 0.0f)) return fail(FSDP_E_INVAL, "%s: AdamW needs betas in [0, 1), eps >= 0", fn);
        const fsdp_adamw_hp a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->step};
        op = adamw_params(a);
        n_states = 2;
        return FSDP_OK;
    }
    case FSDP_OPT_SGD:
        if (!(hp->momentum >= 0.0f) || !(hp->dampening == hp->dampening))
            return fail(FSDP_E_INVAL, "%s: SGD needs momentum >= 0 and a finite dampening", fn);
        if (hp->nesterov && (hp->momentum <= 0.0f || hp->dampening != 0.0f))
            return fail(FSDP_E_INVAL, "%s: Nesterov momentum needs momentum > 0 and dampening == 0", fn);
        op.kind = hp->momentum != 0.0f ? fsdp::kOptSgdMomentum : fsdp::kOptSgd;
        op.mu = hp->momentum;
        op.omd = 1.0f - hp->dampening;
        op.first = hp->step == 1;
        op.nesterov = hp->nesterov != 0;
        n_states = hp->momentum != 0.0f ? 1 : 0;
        return FSDP_OK;
    case FSDP_OPT_ADAMAX:
        if (!betas || !(hp->eps >= 0.0f)) return fail(FSDP_E_INVAL, "%s: Adamax needs betas in [0, 1), eps >= 0", fn);
        op.kind = fsdp::kOptAdamax;
        op.clr = (float)((double)hp->lr / (1.0 - std::pow((double)hp->beta1, (double)hp->step)));
        op.b1 = hp->beta1;
        op.omb1 = 1.0f - hp->beta1;
        op.b2 = hp->beta2;
        n_states = 2;
        return FSDP_OK;
    case FSDP_OPT_ADADELTA:
        if (!(hp->rho >= 0.0f && hp->rho <= 1.0f) || !(hp->eps >= 0.0f))
            return fail(FSDP_E_INVAL, "%s: Adadelta needs rho in [0, 1], eps >= 0", fn);
        op.kind = fsdp::kOptAdadelta;
        op.rho = hp->rho;
        op.omr = 1.0f - hp->rho;
        n_states = 2;
        return FSDP_OK;
    default:
        return fail(FSDP_E_INVAL, "%s: unknown optimizer %d", fn, (int)hp->kind);
    }
}

// Launch the validated units (one grid per table of units).
int launch_built(const char* fn, std::vector<UnitBuild>& units, int32_t world, int grad_dt,
                 int32_t fp32_reduce, int state_dt, int compute_dt, bool gather, const fsdp::OptParams& op,
                 const std::vector<Range>& ins, const std::vector<Range>& outs, void* stream) {
    if (!disjoint(outs, ins)) return fail(FSDP_E_ALIAS, "%s: an output overlaps an input or another output", fn);
    std::vector<fsdp::UnitArgs> args;
    args.reserve(units.size());
    for (UnitBuild& u : units) {
        u.a.grads = u.grads.data();
        u.a.peer_src = u.psrc.data();
        u.a.peer_dst = u.pdst.data();
        if (u.a.S > 0) args.push_back(u.a);
    }
    if (args.empty()) return ok();
    fsdp::UnitLaunch L;
    L.world = world;
    L.grad_dt = grad_dt;
    L.fp32_reduce = fp32_reduce != 0;
    L.compute_dt = compute_dt;
    L.state_dt = state_dt;
    L.gather = gather;
    L.rs = reduce_scalars(world);
    L.opt = op;
    L.cus = cu_count();
    L.stream = stream;
    (void)hipGetLastError();
    hipError_t e = fsdp::launch_units(args.data(), (int)args.size(), L);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return ok();
}

}  // namespace

extern "C" {

int fsdp_abi_version(void) { return FSDP_ABI_VERSION; }

const char* fsdp_last_error(void) { return fsdp::last_error(); }

int fsdp_unit_gather_split(fsdp_dtype state_dt, int32_t n_states, int64_t shard_elements) {
    if (!valid_dtype(state_dt)) return fail(FSDP_E_DTYPE, "fsdp_unit_gather_split: dtype %d unsupported", (int)state_dt);
    if (n_states < 0 || n_states > 2 || shard_elements < 0)
        return fail(FSDP_E_INVAL, "fsdp_unit_gather_split: n_states %d / shard_elements %lld out of range", n_states,
                    (long long)shard_elements);
    ok();
    return fsdp::split_gather(state_dt, n_states, shard_elements) ? 1 : 0;
}

int fsdp_units_in_launch(int32_t world, const int64_t* shard_numels, int32_t n_units, int64_t* shard_elements_out) {
    if (world < 1 || world > FSDP_MAX_WORLD || n_units < 0 || (n_units > 0 && !shard_numels))
        return fail(FSDP_E_INVAL, "fsdp_units_in_launch: world %d / n_units %d / shard_numels out of range", world,
                    n_units);
    for (int32_t k = 0; k < n_units; ++k)
        if (shard_numels[k] < 0) return fail(FSDP_E_INVAL, "fsdp_units_in_launch: shard_numels[%d] < 0", k);
    int64_t elems = 0;
    const int c = n_units == 0 ? 0 : fsdp::units_in_launch(world, shard_numels, n_units, &elems);
    if (shard_elements_out) *shard_elements_out = elems;
    ok();
    return c;
}

int fsdp_time_next_launch(void* start_event, void* stop_event) {
    fsdp::set_launch_events(start_event, stop_event);
    return FSDP_OK;
}

}  // extern "C"

namespace {

int layout_impl(const int64_t* numels, int32_t n_tensors, int32_t world, int64_t* numel_out,
                int64_t* padded_numel_out, int64_t* shard_numel_out) {
    if (world < 1) return fail(FSDP_E_INVAL, "world = %d < 1", world);
    if (n_tensors < 0) return fail(FSDP_E_INVAL, "n_tensors = %d < 0", n_tensors);
    if (n_tensors > 0 && !numels) return fail(FSDP_E_INVAL, "numels is NULL");
    int64_t total = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        if (numels[k] < 0) return fail(FSDP_E_INVAL, "numels[%d] < 0", k);
        if (total > fsdp::kMaxElems - numels[k]) return fail(FSDP_E_SIZE, "unit too large");
        total += numels[k];
    }
    const int64_t padded = (total + world - 1) / world * world;
    if (numel_out) *numel_out = total;
    if (padded_numel_out) *padded_numel_out = padded;
    if (shard_numel_out) *shard_numel_out = padded / world;
    return FSDP_OK;
}

}  // namespace

extern "C" {

int fsdp_layout(const int64_t* numels, int32_t n_tensors, int32_t world, int64_t* numel_out,
                int64_t* padded_numel_out, int64_t* shard_numel_out) {
    int rc = layout_impl(numels, n_tensors, world, numel_out, padded_numel_out, shard_numel_out);
    return rc ? rc : ok();
}

int fsdp_flatten_pad(const void* const* srcs, const int64_t* numels, int32_t n_tensors, fsdp_dtype dt,
                     int32_t world, void* flat, int64_t flat_capacity, int64_t* padded_numel_out,
                     void* stream) {
    int64_t total = 0, padded = 0;
    int rc = layout_impl(numels, n_tensors, world, &total, &padded, nullptr);
    if (rc) return rc;
    if (!valid_dtype(dt)) return fail(FSDP_E_DTYPE, "dtype %d unsupported", (int)dt);
    if (flat_capacity < padded)
        return fail(FSDP_E_SIZE, "flat_capacity %lld < padded numel %lld", (long long)flat_capacity,
                    (long long)padded);
    if (padded > 0 && !flat) return fail(FSDP_E_INVAL, "flat is NULL");
    if (n_tensors > 0 && !srcs) return fail(FSDP_E_INVAL, "srcs is NULL");
    const int64_t es = dt_size(dt);
    const Range out = range(flat, padded, es);
    for (int32_t k = 0; k < n_tensors; ++k) {
        if (numels[k] > 0 && !srcs[k]) return fail(FSDP_E_INVAL, "srcs[%d] is NULL", k);
        if (overlaps(range(srcs[k], numels[k], es), out))
            return fail(FSDP_E_ALIAS, "srcs[%d] overlaps the flat buffer", k);
    }
    if (padded_numel_out) *padded_numel_out = padded;

    // Segments: every non-empty tensor, then the zero tail; batched per launch.
    fsdp::SegBatch b;
    int nseg = 0;
    int64_t chunks = 0;
    auto flush = [&]() -> hipError_t {
        if (nseg == 0) return hipSuccess;
        b.count = nseg;
        b.chunk_begin[nseg] = chunks;
        hipError_t e = fsdp::launch_segments(b, chunks, stream);
        nseg = 0;
        chunks = 0;
        return e;
    };
    auto add = [&](const void* src, void* dst, int64_t bytes) -> hipError_t {
        if (bytes <= 0) return hipSuccess;
        b.src[nseg] = (const char*)src;
        b.dst[nseg] = (char*)dst;
        b.bytes[nseg] = bytes;
        b.chunk_begin[nseg] = chunks;
        chunks += (bytes + fsdp::kSegChunkBytes - 1) / fsdp::kSegChunkBytes;
        if (++nseg == fsdp::kSegMax) return flush();
        return hipSuccess;
    };
    (void)hipGetLastError();
    int64_t pos = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        hipError_t e = add(srcs[k], (char*)flat + pos * es, numels[k] * es);
        if (e != hipSuccess) return hip_fail(e, "flatten launch");
        pos += numels[k];
    }
    hipError_t e = add(nullptr, (char*)flat + total * es, (padded - total) * es);
    if (e == hipSuccess) e = flush();
    if (e != hipSuccess) return hip_fail(e, "flatten launch");
    return ok();
}

int fsdp_reduce_scatter_local(const void* const* rank_grads, int32_t world, int32_t rank,
                              int64_t shard_numel, fsdp_dtype grad_dt, int32_t fp32_reduce,
                              void* grad_shard_out, void* stream) {
    std::vector<const void*> blocks;
    std::vector<Range> ins;
    int rc = check_world(world, rank, shard_numel);
    if (rc) return rc;
    rc = grad_blocks(rank_grads, world, rank, shard_numel, grad_dt, blocks, ins);
    if (rc) return rc;
    const int out_dt = (fp32_reduce || grad_dt == FSDP_F32) ? FSDP_F32 : grad_dt;
    if (shard_numel == 0) return ok();
    if (!grad_shard_out) return fail(FSDP_E_INVAL, "grad_shard_out is NULL");
    const Range out = range(grad_shard_out, shard_numel, dt_size(out_dt));
    for (int q = 0; q < world; ++q)
        if (overlaps(out, ins[q])) return fail(FSDP_E_ALIAS, "grad_shard_out overlaps rank_grads[%d]", q);

    bool vec = aligned16(grad_shard_out);
    for (int q = 0; q < world; ++q) vec = vec && aligned16(blocks[q]);
    fsdp::ReduceArgs a{};
    a.grads = blocks.data();
    a.world = world;
    a.grad_dt = grad_dt;
    a.fp32_reduce = fp32_reduce != 0;
    a.S = shard_numel;
    a.nvec = vec ? shard_numel / 8 : 0;
    a.out = grad_shard_out;
    a.rs = reduce_scalars(world);
    a.cus = cu_count();
    a.stream = stream;
    (void)hipGetLastError();
    hipError_t e = fsdp::launch_reduce_scatter(a);
    if (e != hipSuccess) return hip_fail(e, "reduce-scatter launch");
    return ok();
}

int fsdp_sharded_adamw(float* master, float* exp_avg, float* exp_avg_sq, const void* const* rank_grads,
                       int32_t world, int32_t rank, fsdp_dtype grad_dt, int32_t fp32_reduce,
                       void* compute_shard, fsdp_dtype compute_dt, int64_t shard_numel,
                       const fsdp_adamw_hp* hp, void* stream) {
    const char* fn = "fsdp_sharded_adamw";
    if (!valid_dtype(compute_dt)) return fail(FSDP_E_DTYPE, "%s: compute dtype %d unsupported", fn, (int)compute_dt);
    int rc = check_hp(fn, hp);
    if (rc) return rc;
    std::vector<UnitBuild> units(1);
    std::vector<Range> ins, outs;
    rc = build_unit(fn, 0, master, exp_avg, exp_avg_sq, 2, FSDP_F32, rank_grads, world, rank, grad_dt, compute_dt,
                    shard_numel, compute_shard, nullptr, nullptr, false, units[0], ins, outs);
    if (rc) return rc;
    return launch_built(fn, units, world, grad_dt, fp32_reduce, FSDP_F32, compute_dt, false, adamw_params(*hp), ins,
                        outs, stream);
}

int fsdp_step_unit(float* master, float* exp_avg, float* exp_avg_sq, const void* const* rank_grads,
                   int32_t world, int32_t rank, fsdp_dtype grad_dt, int32_t fp32_reduce,
                   const void* const* peer_shards, void* full_out, fsdp_dtype compute_dt,
                   int64_t shard_numel, void* compute_shard, const fsdp_adamw_hp* hp, void* stream) {
    const char* fn = "fsdp_step_unit";
    if (!valid_dtype(compute_dt)) return fail(FSDP_E_DTYPE, "%s: compute dtype %d unsupported", fn, (int)compute_dt);
    int rc = check_hp(fn, hp);
    if (rc) return rc;
    std::vector<UnitBuild> units(1);
    std::vector<Range> ins, outs;
    rc = build_unit(fn, 0, master, exp_avg, exp_avg_sq, 2, FSDP_F32, rank_grads, world, rank, grad_dt, compute_dt,
                    shard_numel, compute_shard, peer_shards, full_out, true, units[0], ins, outs);
    if (rc) return rc;
    return launch_built(fn, units, world, grad_dt, fp32_reduce, FSDP_F32, compute_dt, true, adamw_params(*hp), ins,
                        outs, stream);
}

}  // extern "C"

namespace {

// The batched unit step of fsdp_step_units / fsdp_step_units_optim (hp checked).
int step_units_impl(const char* fn, const fsdp_unit* units, int32_t n_units, int32_t world, int32_t rank,
                    int grad_dt, int32_t fp32_reduce, int state_dt, int compute_dt, const fsdp::OptParams& op,
                    int n_states, bool state16_ok, void* stream) {
    if (n_units < 0) return fail(FSDP_E_INVAL, "%s: n_units = %d < 0", fn, n_units);
    if (n_units > 0 && !units) return fail(FSDP_E_INVAL, "%s: units is NULL", fn);
    if (!valid_dtype(state_dt)) return fail(FSDP_E_DTYPE, "%s: state dtype %d unsupported", fn, state_dt);
    if (!valid_dtype(compute_dt)) return fail(FSDP_E_DTYPE, "%s: compute dtype %d unsupported", fn, compute_dt);
    if (state_dt != FSDP_F32 && !state16_ok)
        return fail(FSDP_E_DTYPE, "%s: 16-bit state is supported for AdamW only", fn);
    if (state_dt != FSDP_F32 && compute_dt != state_dt)
        return fail(FSDP_E_DTYPE, "%s: with 16-bit state the parameter is the compute copy: compute dtype "
                                  "must equal the state dtype", fn);
    int rc = check_world(world, rank, 0);
    if (rc) return rc;
    if (n_units == 0) return ok();
    const bool gather = units[0].full_out != nullptr;
    std::vector<UnitBuild> built(n_units);
    std::vector<Range> ins, outs;
    for (int32_t k = 0; k < n_units; ++k) {
        const fsdp_unit& u = units[k];
        if ((u.full_out != nullptr) != gather)
            return fail(FSDP_E_INVAL, "%s: unit %d: either every unit has full_out or none", fn, k);
        if (state_dt != FSDP_F32 && u.compute_shard)
            return fail(FSDP_E_INVAL, "%s: unit %d: with 16-bit state the parameter shard is the compute shard; "
                                      "compute_shard must be NULL", fn, k);
        rc = build_unit(fn, k, u.master, u.exp_avg, u.exp_avg_sq, n_states, state_dt, u.rank_grads, world, rank,
                        grad_dt, compute_dt, u.shard_numel, u.compute_shard, u.peer_shards, u.full_out, gather,
                        built[k], ins, outs);
        if (rc) return rc;
    }
    return launch_built(fn, built, world, grad_dt, fp32_reduce, state_dt, compute_dt, gather, op, ins, outs,
                        stream);
}

}  // namespace

extern "C" {

int fsdp_step_units(const fsdp_unit* units, int32_t n_units, int32_t world, int32_t rank, fsdp_dtype grad_dt,
                    int32_t fp32_reduce, fsdp_dtype state_dt, fsdp_dtype compute_dt, const fsdp_adamw_hp* hp,
                    void* stream) {
    const char* fn = "fsdp_step_units";
    int rc = check_hp(fn, hp);
    if (rc) return rc;
    return step_units_impl(fn, units, n_units, world, rank, grad_dt, fp32_reduce, state_dt, compute_dt,
                           adamw_params(*hp), 2, true, stream);
}

int fsdp_step_units_optim(const fsdp_unit* units, int32_t n_units, int32_t world, int32_t rank,
                          fsdp_dtype grad_dt, int32_t fp32_reduce, fsdp_dtype state_dt, fsdp_dtype compute_dt,
                          const fsdp_optim_hp* hp, void* stream) {
    const char* fn = "fsdp_step_units_optim";
    fsdp::OptParams op;
    int n_states = 0;
    int rc = optim_params(fn, hp, op, n_states);
    if (rc) return rc;
    return step_units_impl(fn, units, n_units, world, rank, grad_dt, fp32_reduce, state_dt, compute_dt, op,
                           n_states, hp->kind == FSDP_OPT_ADAMW, stream);
}

int fsdp_unshard_gather(const void* const* shards, int32_t world, int64_t shard_numel, fsdp_dtype dt,
                        void* full_out, void* stream) {
    if (world < 1 || world > FSDP_MAX_WORLD)
        return fail(FSDP_E_INVAL, "world = %d outside [1, %d]", world, FSDP_MAX_WORLD);
    if (shard_numel < 0) return fail(FSDP_E_INVAL, "shard_numel = %lld < 0", (long long)shard_numel);
    if (shard_numel > fsdp::kMaxElems / world)
        return fail(FSDP_E_SIZE, "shard_numel = %lld times world = %d is too large", (long long)shard_numel, world);
    if (!valid_dtype(dt)) return fail(FSDP_E_DTYPE, "dtype %d unsupported", (int)dt);
    if (shard_numel == 0) return ok();
    if (!shards) return fail(FSDP_E_INVAL, "shards is NULL");
    if (!full_out) return fail(FSDP_E_INVAL, "full_out is NULL");
    const int64_t es = dt_size(dt);
    const int64_t bytes = shard_numel * es;
    const Range full = range(full_out, (int64_t)world * shard_numel, es);
    std::vector<const void*> src;
    std::vector<void*> dst;
    for (int q = 0; q < world; ++q) {
        if (!shards[q]) return fail(FSDP_E_INVAL, "shards[%d] is NULL", q);
        char* slot = (char*)full_out + (int64_t)q * bytes;
        if (shards[q] == slot) continue;  // already in place
        if (overlaps(range(shards[q], shard_numel, es), full))
            return fail(FSDP_E_ALIAS, "shards[%d] overlaps full_out outside its own slot", q);
        src.push_back(shards[q]);
        dst.push_back(slot);
    }
    (void)hipGetLastError();
    hipError_t e = fsdp::launch_gather(src.data(), dst.data(), (int)src.size(), bytes, cu_count(), stream);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
    return ok();
}

int fsdp_unflatten_views(const int64_t* numels, int32_t n_tensors, int64_t padded_numel,
                         fsdp_view* views_out, const void* full, fsdp_dtype dt, void* const* dsts,
                         void* stream) {
    int64_t total = 0;
    int rc = layout_impl(numels, n_tensors, 1, &total, nullptr, nullptr);
    if (rc) return rc;
    if (total > padded_numel || padded_numel > fsdp::kMaxElems)
        return fail(FSDP_E_SIZE, "tensors hold %lld elements; padded_numel %lld is smaller or too large",
                    (long long)total, (long long)padded_numel);
    if (n_tensors > 0 && !views_out) return fail(FSDP_E_INVAL, "views_out is NULL");
    if (dsts) {
        if (!valid_dtype(dt)) return fail(FSDP_E_DTYPE, "dtype %d unsupported", (int)dt);
        if (total > 0 && !full) return fail(FSDP_E_INVAL, "full is NULL");
        const int64_t es = dt_size(dt);
        const Range in = range(full, padded_numel, es);
        std::vector<Range> outs;
        for (int32_t k = 0; k < n_tensors; ++k) {
            if (numels[k] > 0 && !dsts[k]) return fail(FSDP_E_INVAL, "dsts[%d] is NULL", k);
            Range r = range(dsts[k], numels[k], es);
            if (overlaps(r, in)) return fail(FSDP_E_ALIAS, "dsts[%d] overlaps the full buffer", k);
            for (size_t j = 0; j < outs.size(); ++j)
                if (overlaps(r, outs[j])) return fail(FSDP_E_ALIAS, "dsts[%d] overlaps another output", k);
            outs.push_back(r);
        }
    }
    int64_t off = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        views_out[k].offset = off;
        views_out[k].numel = numels[k];
        off += numels[k];
    }
    if (!dsts) return ok();

    const int64_t es = dt_size(dt);
    fsdp::SegBatch b;
    int nseg = 0;
    int64_t chunks = 0;
    (void)hipGetLastError();
    for (int32_t k = 0; k <= n_tensors; ++k) {
        const bool last = k == n_tensors;
        if (!last && numels[k] > 0) {
            const int64_t bytes = numels[k] * es;
            b.src[nseg] = (const char*)full + views_out[k].offset * es;
            b.dst[nseg] = (char*)dsts[k];
            b.bytes[nseg] = bytes;
            b.chunk_begin[nseg] = chunks;
            chunks += (bytes + fsdp::kSegChunkBytes - 1) / fsdp::kSegChunkBytes;
            ++nseg;
        }
        if (nseg > 0 && (nseg == fsdp::kSegMax || last)) {
            b.count = nseg;
            b.chunk_begin[nseg] = chunks;
            hipError_t e = fsdp::launch_segments(b, chunks, stream);
            if (e != hipSuccess) return hip_fail(e, "unflatten launch");
            nseg = 0;
            chunks = 0;
        }
    }
    return ok();
}

}  // extern "C"
