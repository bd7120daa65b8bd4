/*
 * fsdp_shard.h -- C ABI of libfsdp_shard.so: the one-device data-parallel hot
 * path of Fully Sharded Data Parallel (ZeRO stage 3) on AMD Instinct MI355X
 * (gfx950).
 *
 * One training step of one FSDP unit, as the pages state the problem:
 *   flatten + pad   the unit's tensors become one flat buffer, padded at the
 *                   tail with +0 to a multiple of the world size N;
 *   reduce-scatter  N ranks' flat gradients are averaged, (1/N) * sum_i G_i,
 *                   and rank r keeps block r;
 *   sharded AdamW   each rank updates only its own fp32 master/m/v shard;
 *   cast            the master shard is rounded to the compute dtype;
 *   all-gather      the N compute shards are concatenated into the full buffer;
 *   views           each tensor is a slice of the full buffer.
 * Sources (cited per call below):
 *   [TR] "Fully Sharded Data Parallel: faster AI training with fewer GPUs"
 *        (techreport.ngo)
 *   [P3] "FSDP (Fully Sharded Data Parallel)" (vanos001 placement-prep notes)
 *   [P4] "fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战指南" (zskr.cn)
 *   [P5] "Data Parallelism" (vanos001 placement-prep notes)
 *
 * Conventions shared by every call:
 *  - Memory.  The caller owns every buffer.  "device" pointers are HIP device
 *    memory on the current device; arrays of pointers (srcs, rank_grads,
 *    shards, dsts) are HOST arrays holding device pointers; numels, views_out
 *    and *_out scalars are host memory.  The library keeps no pointer after a
 *    call returns and allocates no device memory.
 *  - Streams.  `stream` is a hipStream_t (NULL = the null stream).  Work is
 *    enqueued asynchronously; nothing synchronizes.  Any pointer alignment is
 *    accepted; 16-byte-aligned buffers take the wide (dwordx4) path.
 *  - Errors.  Every argument is validated on the host before anything is
 *    enqueued; on a negative status nothing was launched and
 *    fsdp_last_error() returns a message (thread-local).  Nothing throws or
 *    aborts across the ABI.  FSDP_E_HIP reports a HIP runtime error at enqueue.
 *  - Aliasing.  No output may overlap an input or another output, except the
 *    in-place master/m/v of fsdp_sharded_adamw and a shard already sitting in
 *    its slot of the full buffer in fsdp_unshard_gather; overlaps are reported
 *    as FSDP_E_ALIAS.
 *  - Arithmetic.  fp32 operations are single IEEE-754 operations with round to
 *    nearest even (no FMA contraction, correctly rounded divide and square
 *    root, subnormals kept); 16-bit outputs are rounded to nearest even.
 */
#ifndef FSDP_SHARD_H
#define FSDP_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSDP_API __attribute__((visibility("default")))

#define FSDP_ABI_VERSION 9
#define FSDP_MAX_WORLD 128
/* Bytes of the device scratch of fsdp_offload_step_units_noalloc (per device). */
#define FSDP_OFFLOAD_SCRATCH_BYTES (32 << 20)

/* Element formats.  A plain 32-bit integer rather than an enum type, so that
 * any value a caller passes is well defined; values other than these three
 * are refused with FSDP_E_DTYPE. */
typedef int32_t fsdp_dtype;
enum {
    FSDP_F32 = 0,   /* IEEE binary32 */
    FSDP_F16 = 1,   /* IEEE binary16 */
    FSDP_BF16 = 2   /* bfloat16 */
};

enum {
    FSDP_OK = 0,
    FSDP_E_INVAL = -1,  /* null pointer, world/rank out of range, negative size, bad step */
    FSDP_E_DTYPE = -2,  /* unsupported dtype or dtype combination */
    FSDP_E_SIZE = -3,   /* output capacity too small, inconsistent sizes, or an element count
                           (unit, shard x world, buffer) above INT64_MAX / 16 */
    FSDP_E_ALIAS = -4,  /* an output overlaps an input or another output */
    FSDP_E_HIP = -5,    /* HIP runtime error while enqueueing */
    FSDP_E_IO = -6,     /* a file could not be opened, written or renamed */
    FSDP_E_FORMAT = -7  /* a file is not a shard file, is truncated or fails its checksum */
};

/* AdamW hyper-parameters of one flat unit.  Flattening puts the whole unit in
 * one parameter group, so one set applies to every element, biases and norm
 * weights included ([TR] "Adoption paths for FSDP", advanced concern 3).
 * step is t >= 1, the index of the step being taken. */
typedef struct fsdp_adamw_hp {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    int64_t step;
} fsdp_adamw_hp;

/* Tensor k of a flat unit is elements [offset, offset + numel). */
typedef struct fsdp_view {
    int64_t offset;
    int64_t numel;
} fsdp_view;

/* Version of this ABI (FSDP_ABI_VERSION). */
FSDP_API int fsdp_abi_version(void);

/* Message for the last negative status returned on this thread ("" if none). */
FSDP_API const char* fsdp_last_error(void);

/* Profiling hook.  The next kernel that this thread enqueues through this
 * library is launched with start_event / stop_event (hipEvent_t created by the
 * caller, either may be NULL) attached to its own dispatch packet
 * (hipExtLaunchKernel), so timing it adds nothing to the stream.  The pair is
 * consumed by the next entry point that returns, whether it launched a kernel
 * or not; an entry point that enqueues several kernels times its first. */
FSDP_API int fsdp_time_next_launch(void* start_event, void* stop_event);

/* Sizes of a flat unit (host only, no device work).
 * numels[n_tensors]: element counts of the unit's tensors, in flat order.
 * Outputs: total P = sum numels; padded P_pad = smallest multiple of world
 * >= P; shard S = P_pad / world.  Padding follows from the tail-padding rule
 * of fsdp_flatten_pad. */
FSDP_API int fsdp_layout(const int64_t* numels, int32_t n_tensors, int32_t world,
                         int64_t* numel_out, int64_t* padded_numel_out,
                         int64_t* shard_numel_out);

/* Flatten + pad.  [TR] "Adoption paths for FSDP" (advanced concern 3) and
 * [P4] flag table (flatten_parameters): a wrapped unit's parameters become one
 * flat tensor.  flat[off_k + i] = srcs[k][i] with off_k = numel_0 + ... +
 * numel_{k-1} (tensors in caller order, each contiguous row-major, no padding
 * between tensors), then flat[P .. P_pad) = +0 so the buffer splits into
 * `world` equal shards.
 *   srcs[n_tensors]   host array of device pointers, each numels[k] elements of dt
 *                     (may be NULL where numels[k] == 0)
 *   flat              device, flat_capacity elements of dt; must not overlap a source
 *   padded_numel_out  host, receives P_pad (may be NULL)
 * FSDP_E_SIZE if flat_capacity < P_pad. */
FSDP_API int fsdp_flatten_pad(const void* const* srcs, const int64_t* numels, int32_t n_tensors,
                              fsdp_dtype dt, int32_t world, void* flat, int64_t flat_capacity,
                              int64_t* padded_numel_out, void* stream);

/* Reduce-scatter, emulated on one device.  [TR] figure on the decomposition of
 * all-reduce into reduce-scatter and all-gather: blocks are reduced by rank
 * index, rank r keeping block r; [P5] "The Basic Protocol": the average is
 * (1/N) * sum_i G_i; [P4] flag table: --fp32-reduce-scatter reduces in fp32.
 *   rank_grads[world]  host array of device pointers; rank q's flat gradient,
 *                      world * shard_numel elements of grad_dt (only block
 *                      `rank` is read)
 *   grad_shard_out     device, shard_numel elements: fp32 when fp32_reduce != 0
 *                      or grad_dt == FSDP_F32, else grad_dt
 * Element i (j = rank * shard_numel + i), ranks folded left to right:
 *   fp32 mode:   acc = G_0[j]; acc = acc + G_q[j] (q = 1..N-1); out = acc / N
 *   16-bit mode: a = G_0[j]; a = round16(a + G_q[j]); out = round16(a / N)
 * 1 <= world <= FSDP_MAX_WORLD, 0 <= rank < world. */
FSDP_API int fsdp_reduce_scatter_local(const void* const* rank_grads, int32_t world, int32_t rank,
                                       int64_t shard_numel, fsdp_dtype grad_dt, int32_t fp32_reduce,
                                       void* grad_shard_out, void* stream);

/* Sharded AdamW, fused with the reduce-scatter and the cast, one pass over the
 * shard (a shard above 2^26 elements in 2^26-element slices, a launch each;
 * see fsdp_units_in_launch).  [P4] "工作原理" and "限制与兼容性说明": each rank runs the pointwise
 * optimizer on its own shard only (AdamW is among the supported pointwise
 * optimizers); [P5] "The Basic Protocol": W = W - lr * Adam(G_avg, m, v);
 * [P3] "Mixed Precision and FSDP": fp32 master with a 16-bit compute copy.
 * The gradient of element i is the reduce-scatter average defined above,
 * converted to fp32.  Passing world = 1, rank = 0 and rank_grads = {g} is the
 * unfused form: AdamW + cast over an already reduced gradient shard g of
 * dtype grad_dt (for instance the output of fsdp_reduce_scatter_local; a
 * 16-bit g is taken as the 16-bit average, an fp32 g as the fp32 average).
 * Update (the published AdamW; t = hp->step; host scalars computed in double
 * and rounded once to fp32: decay = 1 - lr*wd, step_size = lr / (1 - beta1^t),
 * bc2 = sqrt(1 - beta2^t)):
 *   p1 = p * decay;  m1 = beta1*m + (1-beta1)*g;  v1 = beta2*v + (1-beta2)*(g*g)
 *   p2 = p1 - step_size * (m1 / (sqrt(v1) / bc2 + eps))
 *   master = p2, exp_avg = m1, exp_avg_sq = v1, compute_shard = round(p2)
 *   master, exp_avg, exp_avg_sq  device fp32, shard_numel each, updated in place
 *   compute_shard                device, shard_numel of compute_dt, or NULL (no cast)
 *   hp                           host; hp->step >= 1, betas in [0, 1), lr,
 *                                weight_decay and eps >= 0 (FSDP_E_INVAL otherwise;
 *                                every AdamW entry point checks the same) */
FSDP_API int fsdp_sharded_adamw(float* master, float* exp_avg, float* exp_avg_sq,
                                const void* const* rank_grads, int32_t world, int32_t rank,
                                fsdp_dtype grad_dt, int32_t fp32_reduce,
                                void* compute_shard, fsdp_dtype compute_dt, int64_t shard_numel,
                                const fsdp_adamw_hp* hp, void* stream);

/* All-gather unshard.  [P3] "The Per-Layer Communication" and [TR] "From
 * all-reduce to sharded parameters": the full parameters are gathered from the
 * N shards before compute; full[q * S + i] = shards[q][i].
 *   shards[world]  host array of device pointers, shard_numel elements of dt each
 *   full_out       device, world * shard_numel elements of dt
 * A shard that already sits at its slot (shards[q] == full_out + q*S) is not
 * copied; any other overlap with full_out is FSDP_E_ALIAS.  Call it twice per
 * step when parameters are resharded after the forward ([TR] pseudo-code). */
FSDP_API int fsdp_unshard_gather(const void* const* shards, int32_t world, int64_t shard_numel,
                                 fsdp_dtype dt, void* full_out, void* stream);

/* One FSDP unit's step: the fused reduce-scatter + AdamW + cast of
 * fsdp_sharded_adamw followed by the all-gather of fsdp_unshard_gather, with
 * this rank's compute shard written straight into its slot of the full buffer
 * (the all-gather then moves only the peers' shards).  The peers' shards are
 * copied in the step's own trip (one launch), or, where fsdp_unit_gather_split
 * says so, by a second launch after the step (fsdp_time_next_launch times the
 * step); a shard above 2^26 elements is stepped in 2^26-element slices, each
 * so.  Sources as for
 * those two calls; [TR] "From all-reduce to sharded parameters": after the
 * reduce-scatter each rank updates its own shard, and the full weights are
 * gathered from every rank's shard before the next compute.
 *   master, exp_avg, exp_avg_sq, rank_grads, world, rank, grad_dt, fp32_reduce,
 *   hp, shard_numel   as in fsdp_sharded_adamw
 *   peer_shards[world]  host array of device pointers: the other ranks'
 *                       compute shards (shard_numel elements of compute_dt);
 *                       entry `rank` is ignored and may be NULL
 *   full_out            device, world * shard_numel elements of compute_dt:
 *                       full_out[rank*S + i] = round(master_new[i]) and
 *                       full_out[q*S + i] = peer_shards[q][i] for q != rank
 *   compute_shard       device, shard_numel of compute_dt, or NULL: an extra
 *                       persistent copy of this rank's compute shard (needed
 *                       when the unit is gathered again, e.g. before backward
 *                       with parameters resharded after the forward)
 * No output may overlap an input or another output (FSDP_E_ALIAS). */
FSDP_API int fsdp_step_unit(float* master, float* exp_avg, float* exp_avg_sq,
                            const void* const* rank_grads, int32_t world, int32_t rank,
                            fsdp_dtype grad_dt, int32_t fp32_reduce,
                            const void* const* peer_shards, void* full_out, fsdp_dtype compute_dt,
                            int64_t shard_numel, void* compute_shard, const fsdp_adamw_hp* hp,
                            void* stream);

/* One unit of a batched step (fsdp_step_units).  The state buffers have the
 * call's state dtype: fp32 master / m / v, or with 16-bit state the 16-bit
 * parameter shard (also the compute shard) and 16-bit m / v. */
typedef struct fsdp_unit {
    void* master;                    /* device, shard_numel of state_dt, updated in place */
    void* exp_avg;                   /* device, shard_numel of state_dt, updated in place */
    void* exp_avg_sq;                /* device, shard_numel of state_dt, updated in place */
    const void* const* rank_grads;   /* host array [world] of device pointers, world*shard_numel each */
    const void* const* peer_shards;  /* host array [world] (entry `rank` ignored), or NULL without full_out */
    void* full_out;                  /* device, world*shard_numel of compute dtype, or NULL: no all-gather */
    void* compute_shard;             /* device, shard_numel of compute dtype, or NULL (must be NULL with
                                        16-bit state) */
    int64_t shard_numel;
} fsdp_unit;

/* Several units' steps in as few launches as possible: the optimizer step of
 * every flat unit of a model, as one fused multi-tensor update.  [P4]
 * "工作原理": each rank updates the optimizer state of its own shards only;
 * [TR] "Adoption paths for FSDP", concern 3: one hyper-parameter set per
 * flattened unit (here one set for the whole call).  Unit k is stepped exactly
 * as by fsdp_step_unit (when units[k].full_out is set: fused reduce-scatter,
 * AdamW, cast, all-gather) or as by fsdp_sharded_adamw (when it is NULL, with
 * compute_shard as the compute output); every unit of a call must take the
 * same form.  All units share world, rank, dtypes and hp.
 * state_dt: FSDP_F32 for an fp32 master with fp32 m / v (as above), or
 * FSDP_BF16 / FSDP_F16 for 16-bit parameters and m / v with no fp32 master
 * ([P3] "Mixed Precision and FSDP", pure bf16, 3P/N per worker; [TR] concern 4,
 * FP16 master weights): the update is the fp32 sequence above on the widened
 * values, and the new parameter, m and v are each rounded once to state_dt;
 * compute_dt must equal state_dt, the parameter shard is the compute shard
 * (compute_shard NULL), and with full_out the gather copies it.
 * Units are packed in order into launches of up to 40 (world <= 2), 24
 * (world 4) or 16 (world 8) units, other world sizes one unit per launch, and
 * at most 2^26 shard elements per launch (a larger unit is stepped in slices
 * of 2^26 elements, a launch each); fsdp_units_in_launch gives the plan.  With
 * full_out, a launch copies the peers' shards of its units in its own trip, or,
 * where fsdp_unit_gather_split says so for its units' shard elements, is
 * followed by one launch that copies them (up to 128 copies).  No output
 * of any unit may overlap an input or an output of any unit (FSDP_E_ALIAS): a
 * unit may appear only once per call. */
FSDP_API int fsdp_step_units(const fsdp_unit* units, int32_t n_units, int32_t world, int32_t rank,
                             fsdp_dtype grad_dt, int32_t fp32_reduce, fsdp_dtype state_dt,
                             fsdp_dtype compute_dt, const fsdp_adamw_hp* hp, void* stream);

/* ------------------------------------------------------------------------
 * Other pointwise optimizers.  [P4] "限制与兼容性说明": FSDP supports the
 * pointwise optimizers (Adam, AdamW, Adadelta, Adamax, SGD, ...), whose update
 * of an element needs only that element's gradient and state, and not
 * Adagrad, Adafactor or LAMB.  The pages write none of the updates; these are
 * the published algorithms in the form torch.optim documents them, weight
 * decay added to the gradient (d = g + wd*p, skipped when wd == 0) except for
 * AdamW's decoupled decay.  Host scalars: hyper-parameters as fp32, 1 - beta,
 * 1 - dampening and 1 - rho one fp32 operation, lr / (1 - beta1^t) in double
 * rounded once.  Per element, with t = step:
 *   SGD, momentum == 0:  p <- p - lr*d                       (no state)
 *   SGD, momentum mu:    b <- d if t == 1 else mu*b + (1 - dampening)*d;
 *                        d <- d + mu*b (nesterov) or b;  p <- p - lr*d
 *                        (state: exp_avg = momentum buffer)
 *   Adamax:              m <- beta1*m + (1 - beta1)*d;
 *                        u <- max(beta2*u, |d| + eps) (NaN if either is NaN);
 *                        p <- p - (lr / (1 - beta1^t)) * (m / u)
 *                        (state: exp_avg = m, exp_avg_sq = u)
 *   Adadelta:            v <- rho*v + (1 - rho)*(d*d);
 *                        delta = (sqrt(acc + eps) / sqrt(v + eps)) * d;
 *                        acc <- rho*acc + (1 - rho)*(delta*delta); p <- p - lr*delta
 *                        (state: exp_avg = v, exp_avg_sq = acc)
 *   AdamW:               as fsdp_sharded_adamw (exp_avg = m, exp_avg_sq = v)
 * ------------------------------------------------------------------------ */
/* A 32-bit integer for the same reason as fsdp_dtype (others: FSDP_E_INVAL). */
typedef int32_t fsdp_optimizer;
enum {
    FSDP_OPT_ADAMW = 0,
    FSDP_OPT_SGD = 1,
    FSDP_OPT_ADAMAX = 2,
    FSDP_OPT_ADADELTA = 3
};

typedef struct fsdp_optim_hp {
    fsdp_optimizer kind;
    float lr;             /* >= 0 */
    float weight_decay;   /* >= 0 */
    float beta1;          /* AdamW, Adamax: [0, 1) */
    float beta2;          /* AdamW, Adamax: [0, 1) */
    float eps;            /* AdamW, Adamax, Adadelta: >= 0 */
    float momentum;       /* SGD: >= 0 */
    float dampening;      /* SGD */
    float rho;            /* Adadelta: [0, 1] */
    int32_t nesterov;     /* SGD: needs momentum > 0 and dampening == 0 */
    int64_t step;         /* t >= 1, the step being taken */
} fsdp_optim_hp;

/* fsdp_step_units with the optimizer named by hp->kind.  The state buffers the
 * optimizer does not keep may be NULL (SGD without momentum: exp_avg and
 * exp_avg_sq; SGD with momentum: exp_avg_sq) and are never touched.  16-bit
 * state_dt only with FSDP_OPT_ADAMW (FSDP_E_DTYPE otherwise).  FSDP_E_INVAL for
 * hyper-parameters outside the ranges above. */
FSDP_API int fsdp_step_units_optim(const fsdp_unit* units, int32_t n_units, int32_t world, int32_t rank,
                                   fsdp_dtype grad_dt, int32_t fp32_reduce, fsdp_dtype state_dt,
                                   fsdp_dtype compute_dt, const fsdp_optim_hp* hp, void* stream);

/* Launch plan of the unit step, for tools that time or count its kernels
 * (host only).  1 when a step launch of fsdp_step_units / fsdp_step_units_optim
 * / fsdp_step_unit with full_out, whose units hold `shard_elements` shard
 * elements together, writes only the own slots and a second launch copies the
 * peers' shards; 0 when the step launch copies them in its own trip.  Measured
 * rule: 1 for fp32 state (state_dt FSDP_F32) with an optimizer that keeps
 * n_states >= 1 state buffers (AdamW, Adamax, Adadelta: 2; SGD with momentum: 1;
 * SGD without momentum: 0) and shard_elements >= 2^24.  FSDP_E_INVAL for
 * n_states outside [0, 2] or shard_elements < 0, FSDP_E_DTYPE for state_dt. */
FSDP_API int fsdp_unit_gather_split(fsdp_dtype state_dt, int32_t n_states, int64_t shard_elements);

/* Launch plan, continued (host only): how many of the units with shard sizes
 * shard_numels[0 .. n_units) the next step launch of fsdp_step_units /
 * fsdp_step_units_optim takes (at least 1 when n_units > 0; 0 when n_units is
 * 0), and in *shard_elements_out (may be NULL) the shard elements that launch
 * covers.  A launch covers at most 2^26 shard elements: units are packed up to
 * that, and a larger unit is stepped in slices of 2^26 elements, a launch each
 * (then the answer is 1 unit and 2^26 elements).  FSDP_E_INVAL for world outside
 * [1, FSDP_MAX_WORLD], n_units < 0, a NULL array with n_units > 0 or a
 * negative size. */
FSDP_API int fsdp_units_in_launch(int32_t world, const int64_t* shard_numels, int32_t n_units,
                                  int64_t* shard_elements_out);

/* Per-tensor views of the full buffer.  [P3] "The FSDP Unit" (use_orig_params):
 * tensor k is full[off_k : off_k + numel_k]; the padding belongs to no view.
 *   views_out[n_tensors]  host, receives {off_k, numel_k}
 *   padded_numel          length of the full buffer (>= sum numels)
 *   full, dsts            if dsts is NULL only the views are produced (no device
 *                         work; full may be NULL).  Otherwise dsts[k] (host
 *                         array of device pointers) receives a copy of tensor k. */
FSDP_API int fsdp_unflatten_views(const int64_t* numels, int32_t n_tensors, int64_t padded_numel,
                                  fsdp_view* views_out, const void* full, fsdp_dtype dt,
                                  void* const* dsts, void* stream);

/* ------------------------------------------------------------------------
 * CPU offload of the optimizer step.  [TR] "Adoption paths for FSDP"
 * (fairseq, --cpu-offload): the fp32 master copy and the optimizer state move
 * to host memory and the Adam update runs on the CPU; [P3] "CPU Offloading":
 * the cost is the PCIe transfer of every step; [P4] flag table and the
 * single-GPU example (--cpu-offload with the Adam step on the CPU).
 * The update is the one of fsdp_sharded_adamw, bit for bit.
 * ------------------------------------------------------------------------ */

/* AdamW on a host shard, on the calling thread plus up to n_threads - 1 worker
 * threads of the library (AVX2 + F16C when the CPU has them, same IEEE fp32
 * operation sequence either way; the caller's MXCSR is left as it was).
 *   master, exp_avg, exp_avg_sq  host fp32, n elements each, updated in place
 *   grad                         host, n elements of grad_dt (already averaged)
 *   compute                      host, n elements of compute_dt, or NULL (no cast)
 * Blocks until done.  FSDP_E_ALIAS if two buffers overlap. */
FSDP_API int fsdp_host_adamw(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                             fsdp_dtype grad_dt, void* compute, fsdp_dtype compute_dt, int64_t n,
                             const fsdp_adamw_hp* hp, int32_t n_threads);

/* One unit of an offloaded step (fsdp_offload_step_units).
 *   master, exp_avg, exp_avg_sq  host fp32, shard_numel each, updated in place
 *   rank_grads                   host array of `world` device pointers, as in
 *                                fsdp_reduce_scatter_local
 *   grad_shard_dev               device, shard_numel of the reduce-scatter output
 *                                dtype (fp32 when fp32_reduce or fp32 grads)
 *   grad_shard_host              host, same size and dtype
 *   compute_host                 host, shard_numel of compute_dt
 *   compute_dev                  device, shard_numel of compute_dt (e.g. the rank's
 *                                slot of the full buffer, or the shard that
 *                                fsdp_unshard_gather reads)
 * Host buffers should be pinned (hipHostMalloc) for the copies to be
 * asynchronous; pageable memory works, with copies that block. */
typedef struct fsdp_offload_unit {
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    const void* const* rank_grads;
    void* grad_shard_dev;
    void* grad_shard_host;
    void* compute_host;
    void* compute_dev;
    int64_t shard_numel;
} fsdp_offload_unit;

/* Offloaded step of n_units units of rank `rank`.  Enqueued on `stream`, in
 * unit order: each unit's device reduce-scatter of block `rank` (as
 * fsdp_reduce_scatter_local) into grad_shard_dev, then its device-to-host
 * copies into grad_shard_host in chunks of chunk_numel elements (<= 0: 4 Mi;
 * rounded up to a multiple of 8).  Then up to n_threads host threads run
 * fsdp_host_adamw over the chunks in order, each chunk once its copy has
 * landed; the thread that completes a chunk enqueues the copy of its compute
 * values to compute_dev, on copy_stream if it is not NULL (copy_stream first
 * waits for the work already on `stream`, and `stream` waits for copy_stream's
 * copies before the call returns, so later work on `stream` sees compute_dev),
 * else on `stream`.
 * Blocks until the host update of every unit is done; the copies to the device
 * are enqueued and not waited for (compute_host must stay untouched until
 * `stream` has passed them).  Every buffer of every unit is distinct
 * (FSDP_E_ALIAS otherwise), so a unit appears at most once per call.  After a
 * HIP error reported as FSDP_E_HIP, some units may have been stepped. */
FSDP_API int fsdp_offload_step_units(const fsdp_offload_unit* units, int32_t n_units, int32_t world,
                                     int32_t rank, fsdp_dtype grad_dt, int32_t fp32_reduce,
                                     fsdp_dtype compute_dt, int64_t chunk_numel,
                                     const fsdp_adamw_hp* hp, int32_t n_threads, void* stream,
                                     void* copy_stream);

/* fsdp_offload_step_units for callers that cannot allocate device memory
 * (harnesses that forbid hipMalloc during steps, serving loops with a fixed
 * memory budget), and which cannot spare a device gradient shard per unit.
 * Same arguments, results and blocking behaviour as fsdp_offload_step_units,
 * except that every unit's grad_shard_dev must be NULL: each chunk of a unit's
 * gradient shard is reduce-scattered into a device scratch array of
 * FSDP_OFFLOAD_SCRATCH_BYTES (32 MiB) that the library holds per device until
 * the process ends, and copied to grad_shard_host from there.  Limit: a chunk
 * must fit the scratch, chunk_numel * (4 bytes when fp32_reduce or fp32
 * gradients, else 2) <= FSDP_OFFLOAD_SCRATCH_BYTES after rounding chunk_numel
 * up to a multiple of 8 (<= 0 means 4 Mi elements, which fits); FSDP_E_SIZE
 * otherwise, before anything is enqueued.  Its first call on a device, with
 * that device current, looks up the scratch's device address and creates 258
 * events for that device; later calls call no hipMalloc, hipFree, event or
 * stream creation (host-side bookkeeping uses the C++ heap).  Every call on a
 * device uses that device's one scratch, which keeps the previous call's bytes
 * (each chunk is written whole before it is read, so nothing needs clearing);
 * calls that overlapped in time on one device would race on it, so the library
 * serializes them with a per-device lock held for the whole call (the call
 * returns only after every copy out of the scratch has landed).  Calls on
 * different devices run independently. */
FSDP_API int fsdp_offload_step_units_noalloc(const fsdp_offload_unit* units, int32_t n_units, int32_t world,
                                             int32_t rank, fsdp_dtype grad_dt, int32_t fp32_reduce,
                                             fsdp_dtype compute_dt, int64_t chunk_numel, const fsdp_adamw_hp* hp,
                                             int32_t n_threads, void* stream, void* copy_stream);

/* fsdp_offload_step_units for one unit, its fields passed one by one. */
FSDP_API int fsdp_offload_step(float* master, float* exp_avg, float* exp_avg_sq,
                               const void* const* rank_grads, int32_t world, int32_t rank,
                               fsdp_dtype grad_dt, int32_t fp32_reduce, void* grad_shard_dev,
                               void* grad_shard_host, void* compute_host, void* compute_dev,
                               fsdp_dtype compute_dt, int64_t shard_numel, int64_t chunk_numel,
                               const fsdp_adamw_hp* hp, int32_t n_threads, void* stream,
                               void* copy_stream);

/* ------------------------------------------------------------------------
 * Sharded-state checkpoints.  [P4] "工作原理", checkpoint paragraph: with
 * --use-sharded-state every rank saves its own local state to a file named
 * with the suffix -shard{rank} and loads it back the same way (all ranks save);
 * the default mode consolidates the full state instead, which is a gather of
 * the shards followed by the per-tensor views.  [P3] "FSDP Checkpointing".
 *
 * A shard file holds: a 256-byte header (the fields of fsdp_ckpt_info, the
 * hyper-parameters at save time, CRC32C checksums), the unit's tensor sizes,
 * and at a 4096-aligned offset the master, exp_avg and exp_avg_sq shards
 * (shard_numel elements each, state dtype).  Files are written to
 * "<path>.tmp", synced and renamed, so the final name never holds a partial
 * file.  Buffers live in host memory (on_device = 0) or device memory
 * (on_device = 1, copied through pinned staging on `stream`; the call returns
 * after the copies completed).  The calls block the calling thread.
 * ------------------------------------------------------------------------ */
typedef struct fsdp_ckpt_info {
    int32_t world;           /* N */
    int32_t rank;            /* r, 0 <= r < N */
    int64_t numel;           /* P: elements of the unit's tensors */
    int64_t padded_numel;    /* P_pad */
    int64_t shard_numel;     /* S = P_pad / N */
    fsdp_dtype state_dt;     /* FSDP_F32 master/m/v, or 16-bit parameter/m/v */
    fsdp_dtype compute_dt;
    int64_t step;            /* optimizer steps taken so far */
    fsdp_adamw_hp hp;        /* hyper-parameters (hp.step is not stored; read back as `step`) */
    int32_t n_tensors;
} fsdp_ckpt_info;

/* CRC32C (Castagnoli) of n bytes of host memory, as stored in shard files. */
FSDP_API uint32_t fsdp_crc32c(const void* data, int64_t n);

/* Save one rank's shard state.  numels[info->n_tensors]: the unit's tensor
 * sizes (host), summing to info->numel.  master/exp_avg/exp_avg_sq:
 * info->shard_numel elements of info->state_dt each. */
FSDP_API int fsdp_save_shard(const char* path, const fsdp_ckpt_info* info, const int64_t* numels,
                             const void* master, const void* exp_avg, const void* exp_avg_sq,
                             int32_t on_device, void* stream);

/* Read a shard file's header and size table (no payload).  numels_out may be
 * NULL; otherwise it must hold info_out->n_tensors entries (FSDP_E_SIZE). */
FSDP_API int fsdp_shard_info(const char* path, fsdp_ckpt_info* info_out, int64_t* numels_out,
                             int32_t numels_capacity);

/* Load a shard file into master/exp_avg/exp_avg_sq (shard_capacity elements
 * each at least).  FSDP_E_FORMAT on a bad header, truncation or checksum
 * mismatch; after a payload mismatch the destinations' contents are
 * unspecified.  info_out (may be NULL) receives the header. */
FSDP_API int fsdp_load_shard(const char* path, fsdp_ckpt_info* info_out, void* master, void* exp_avg,
                             void* exp_avg_sq, int64_t shard_capacity, int32_t on_device, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_SHARD_H */
