/*
 * zs.h -- C ABI of the ZeRO-3 shard-step library (libzs.so) for MI355X (gfx950).
 *
 * One data-parallel rank's ZeRO-3 / FSDP shard step, with the D ranks of a
 * data-parallel group simulated as D buffers in one GPU's memory:
 *
 *   zs_unit_layout   flat layout of one FSDP unit (host arithmetic only)
 *   zs_pack_flat     pack a unit's tensors into D contiguous shards
 *   zs_reduce_shard  reduce-scatter arithmetic for one shard
 *   zs_adamw_step    fused reduce + mixed-precision AdamW on one shard
 *   zs_reduce_shard_ex, zs_adamw_step_ex  the same under HYBRID_SHARD's
 *                    two-level reduce and/or reduce-dtype rounding
 *   zs_adamw_step_timed  zs_adamw_step_ex with the kernel's own start and
 *                    end recorded in two events (a measurement aid)
 *   zs_gather_unit   all-gather's local rebuild of a unit from its shards
 *   zs_step_pipelined  the step over a sequence of buckets, each bucket's
 *                    contribution transfer overlapped with the previous step
 *   zs_step_pipelined_static  the same with library-owned staging, for
 *                    callers that cannot allocate device memory
 *   zs_reshard       re-shard a unit from D to D2 shards on the device
 *   zs_shard_save, zs_shard_load, zs_shard_load_resharded, zs_shard_info_read
 *                    per-rank shard checkpoints, resumable at any D2
 *   zs_adamw_step_host, zs_offload_step
 *                    the step's AdamW on host cores (ZeRO-Offload)
 *   zs_stream_ceiling, zs_stream_ceiling_timed, zs_hbm_probe
 *                    measurement aids: the step's memory streams without its
 *                    arithmetic, and HBM's rate for one direction alone
 *
 * Sources (web pages, by title and section):
 *   [ZT]   "7.10 -- Fully-sharded data parallel (FSDP / ZeRO-3)", AI / ML
 *          Theory, chapter 7.
 *   [GPT8] "Building GPT from Scratch -- Part 8: FSDP -- When the Model
 *          Won't Fit".
 *   [RP]   "Distributed LLM Fine-Tuning at Scale: FSDP, ZeRO-3, and
 *          Multi-GPU Orchestration".
 *
 * Conventions shared by every entry point:
 *   - All data buffers are device memory owned by the caller. The library
 *     never allocates, frees or synchronizes; kernels are enqueued on the
 *     caller's stream (which must belong to the current HIP device) and the
 *     call returns as soon as they are enqueued.
 *   - Arrays of D pointers (shards, contributions) are HOST arrays of DEVICE
 *     pointers; they are copied into kernel arguments, so D <= ZS_MAX_D.
 *   - bf16 values are raw IEEE binary32 high halves stored as uint16.
 *   - Every argument is validated on the host before anything is enqueued.
 *     A failing call returns a nonzero status, enqueues nothing, and leaves
 *     a message for zs_last_error(). A launch failure reported by the HIP
 *     runtime returns ZS_EHIP. Faults of enqueued kernels surface at the
 *     caller's next synchronization, as for any HIP kernel.
 *   - Zero-length work (S == 0, T == 0) returns ZS_OK and enqueues nothing.
 *   - Calls are thread-safe; the error message is per calling thread.
 *   - Full-speed paths need 16-byte-aligned buffers; any other alignment
 *     allowed by the element size is correct but slower.
 */
#ifndef ZS_H_
#define ZS_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t zs_status;
#define ZS_OK            0  /* success                                       */
#define ZS_EINVAL        1  /* an argument is out of range or inconsistent   */
#define ZS_EALIAS        2  /* an output overlaps an input it may not        */
#define ZS_EHIP          3  /* the HIP runtime reported an error             */
#define ZS_EUNSUPPORTED  4  /* unknown dtype or a size beyond the limits     */
#define ZS_EIO           5  /* a checkpoint file could not be read or written,
                               or failed its format or checksum checks    */

/* Element types. */
#define ZS_BF16 1  /* bf16 as uint16 bit patterns (2 bytes)                   */
#define ZS_F32  2  /* IEEE binary32 (4 bytes)                                 */

#define ZS_MAX_D 64  /* most ranks (or contributions) one call handles       */

/* One tensor of an FSDP unit: its data and where it lands in the flat unit. */
typedef struct {
    const void* ptr;      /* device pointer to numel contiguous elements      */
    int64_t numel;        /* >= 0                                             */
    int64_t flat_offset;  /* start in the flat unit: prefix sum of numels     */
} zs_tensor_ref;

/* AdamW hyperparameters, in double; the library rounds each derived
 * constant to fp32 once (see zs_adamw_step). */
typedef struct {
    double lr;            /* >= 0                                             */
    double beta1;         /* in [0, 1)                                        */
    double beta2;         /* in [0, 1)                                        */
    double eps;           /* >= 0                                             */
    double weight_decay;  /* >= 0, decoupled, multiplied by lr               */
    int64_t step;         /* t >= 1, the step being taken                     */
} zs_adamw_hp;

/*
 * zs_unit_layout -- flat layout of one FSDP unit (host only, no GPU work).
 *
 * [ZT] section 3 gives each rank r a partition P_r of about 1/D of the
 * parameters; [ZT] section 6 and [GPT8] "PyTorch FSDP Implementation" make
 * each transformer block one unit. Layout: the T tensors end to end in the
 * given order, no per-tensor alignment, the flat length N padded up to
 * N_pad = D * ceil(N / D); rank r owns flat[r*S, (r+1)*S) with S = N_pad / D.
 *
 *   numels      host, T entries, each >= 0 (may be NULL when T == 0)
 *   T           number of tensors, >= 0
 *   D           ranks, 1..ZS_MAX_D
 *   offsets_out host, T + 1 entries: offsets_out[j] = start of tensor j,
 *               offsets_out[T] = N
 *   n_out, n_pad_out, shard_len_out  host scalars: N, N_pad, S
 * Errors: ZS_EINVAL for a negative count, a NULL output or D out of range;
 * ZS_EUNSUPPORTED if N_pad overflows int64.
 */
zs_status zs_unit_layout(const int64_t* numels, int32_t T, int32_t D,
                         int64_t* offsets_out, int64_t* n_out,
                         int64_t* n_pad_out, int64_t* shard_len_out);

/*
 * zs_pack_flat -- pack a unit's tensors into its D shards (bit copy).
 *
 * The flat unit (layout of zs_unit_layout) is split into D contiguous
 * shards, the rank-ordered blocks of the all-gather diagram in [GPT8]
 * "AllGather vs AllReduce" and the local shards of [ZT] section 5.1:
 * shards[r][i] = flat[r*S + i], with flat[N, N_pad) = +0 (all-zero bits).
 * Bytes are copied unchanged whatever they hold.
 *
 *   h_table  host array of T tensor refs, checked by the library: numel >= 0,
 *            ptr non-NULL when numel > 0 and aligned to the element size,
 *            flat_offset equal to the prefix sum of the numels
 *   d_table  device array holding the same T refs byte for byte (the kernel
 *            reads this copy; the caller keeps it alive until the work is done)
 *   T        tensors, >= 0
 *   dtype    ZS_BF16 or ZS_F32 (element size of every tensor and shard)
 *   D        ranks, 1..ZS_MAX_D
 *   shards   host array of D device pointers, each to S elements
 *   S        shard length; must equal ceil(N / D) for N = sum of numels
 * Errors: ZS_EINVAL (inconsistent table, S, NULLs, alignment), ZS_EALIAS
 * (a shard overlaps a tensor or another shard), ZS_EUNSUPPORTED (dtype).
 */
zs_status zs_pack_flat(const zs_tensor_ref* h_table, const zs_tensor_ref* d_table,
                       int32_t T, int32_t dtype, int32_t D,
                       void* const* shards, int64_t S, hipStream_t stream);

/*
 * zs_reduce_shard -- reduce-scatter arithmetic for one rank's shard.
 *
 * [GPT8] "AllGather vs AllReduce": rank r receives the sum over ranks of
 * their gradients restricted to its shard; [ZT] section 4: this is the
 * all-reduce's result, scattered; DDP's all-reduce averages. For i < S:
 *   grad_out[i] = (((c_0[i] + c_1[i]) + ...) + c_{D-1}[i]) * float(1/D)
 * in fp32, contributions widened exactly from the reduce dtype (bf16 as in
 * [RP] section 2, or fp32 as in [GPT8] "Mixed Precision"), folded left to
 * right in rank order starting from c_0, one rounding per add, then one
 * multiply by 1/D rounded to fp32. The result stays fp32.
 *
 *   contribs  host array of D device pointers, each to S elements of dtype
 *   D         contributions, 1..ZS_MAX_D
 *   dtype     ZS_BF16 or ZS_F32
 *   S         >= 0
 *   grad_out  device, S floats
 * Errors: ZS_EINVAL, ZS_EALIAS (grad_out overlaps a contribution),
 * ZS_EUNSUPPORTED.
 */
zs_status zs_reduce_shard(const void* const* contribs, int32_t D, int32_t dtype,
                          int64_t S, float* grad_out, hipStream_t stream);

/*
 * zs_adamw_step -- fused reduce + mixed-precision AdamW on one shard.
 *
 * [ZT] section 3: a rank updates only its partition, from its fp32 master
 * copy, its m and v and its slice of the gradient; [ZT] section 6 and
 * [GPT8] "Mixed Precision": master and moments stay fp32, the working
 * weights are bf16. Per element, g is the zs_reduce_shard value of the
 * n_contrib contributions (their mean, folded in order), never stored; then
 * in fp32, each operation rounded on its own, no fused multiply-add:
 *   p1  = p * DEC
 *   m'  = B1 * m + B1c * g
 *   v'  = B2 * v + B2c * (g * g)
 *   den = sqrt(v') / BC2S + EPS
 *   p'  = p1 - SS * (m' / den)
 *   w   = bf16 round-to-nearest-even of p'
 * with constants rounded to fp32 once from double: B1 = beta1,
 * B1c = 1 - beta1, B2 = beta2, B2c = 1 - beta2, SS = lr / (1 - beta1^t),
 * BC2S = sqrt(1 - beta2^t), DEC = 1 - lr * weight_decay, EPS = eps, where
 * beta^t is t successive double multiplications starting from 1.0.
 * An unfused step (zs_reduce_shard, then this call with its output as the
 * single fp32 contribution) gives the same bits.
 *
 *   p, m, v   device, S floats each, updated in place (pairwise disjoint)
 *   w_out     device, S uint16 (bf16 working shard), written
 *   S         >= 0
 *   contribs  host array of n_contrib device pointers, S elements of dtype
 *   n_contrib 1..ZS_MAX_D
 *   dtype     ZS_BF16 or ZS_F32
 *   hp        host pointer to the hyperparameters
 * Errors: ZS_EINVAL (NULLs, alignment, hyperparameters out of range),
 * ZS_EALIAS (p, m, v, w_out overlap each other or a contribution),
 * ZS_EUNSUPPORTED.
 */
zs_status zs_adamw_step(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                        const void* const* contribs, int32_t n_contrib, int32_t dtype,
                        const zs_adamw_hp* hp, hipStream_t stream);

/* How the contributions of one shard are reduced (zs_reduce_shard_ex,
 * zs_adamw_step_ex), and how the step's bf16 working shard is stored.
 * All fields 0 except replicas = 1 is the flat reduce of zs_reduce_shard /
 * zs_adamw_step, which always multiply by 1/D (the averaged gradient); a
 * caller that wants another multiplier (1 for the plain sum of the
 * reduce-scatter diagram in [GPT8] "AllGather vs AllReduce", or a
 * loss-scale factor) sets scale here.
 *
 * working_shard_hint (zs_adamw_step_ex only; zs_reduce_shard_ex ignores it):
 *   ZS_W_STREAM  non-temporal stores, as every other stream of the step: the
 *                default, for a working shard read much later;
 *   ZS_W_KEEP    ordinary stores that allocate in the caches (L2 and the
 *                memory-side Infinity Cache), for a caller that reads the
 *                working shard right after -- the all-gather of the same unit,
 *                [ZT] section 5.1 / [GPT8] "The Lifecycle of a Parameter".
 *                The gather then reads it from the cache, so the shard crosses
 *                HBM once (written back later) instead of twice (written, then
 *                read). The values are the same bits either way. */
#define ZS_W_STREAM 0
#define ZS_W_KEEP   1
typedef struct {
    int32_t replicas;               /* R >= 1 replica groups (HYBRID_SHARD nodes) */
    int32_t round_to_reduce_dtype;  /* 0 or 1: each collective's output is held
                                       in the reduce dtype                        */
    double scale;                   /* finite, and finite once rounded to fp32;
                                       the one multiplier of the reduced sum,
                                       rounded to fp32 once; 0 means 1 / (R * D)  */
    int32_t working_shard_hint;     /* ZS_W_STREAM or ZS_W_KEEP                   */
    int32_t reserved;               /* must be 0                                  */
} zs_reduce_opts;

/*
 * zs_reduce_shard_ex -- reduce-scatter arithmetic under HYBRID_SHARD and/or
 * with the collectives' outputs rounded to the reduce dtype.
 *
 * [GPT8] "Sharding Strategies" and "HYBRID_SHARD: The Multi-Node Strategy":
 * parameters are fully sharded over the D GPUs of a node and replicated
 * over R nodes; each node reduce-scatters over its local ranks, then the
 * nodes all-reduce their shards. [RP] section 2 (reduce_dtype bf16) and
 * [GPT8] "Mixed Precision" (reduce_dtype fp32) give the dtype the
 * collectives communicate in. For i < S, with contributions replica-major
 * (contribs[j*D + k] = local rank k of node j):
 *   s_j = ((c_{j,0} + c_{j,1}) + ...) + c_{j,D-1}      fp32, per node j
 *   s_j = round_to_reduce_dtype(s_j)                   if opts->round...
 *   t   = ((s_0 + s_1) + ...) + s_{R-1}                fp32
 *   t   = round_to_reduce_dtype(t)                     if opts->round...
 *   grad_out[i] = t * float(1 / (R * D))
 * where round_to_reduce_dtype is bf16 round-to-nearest-even widened back
 * (exact identity for fp32); with opts->scale != 0 the last line multiplies
 * by float(opts->scale) instead. opts == NULL means R = 1, no rounding,
 * scale 1 / D.
 *
 *   contribs  host array of R * D device pointers (R * D <= ZS_MAX_D), each
 *             to S elements of dtype
 *   D         contributions per node, >= 1
 *   opts      host pointer or NULL
 * Other arguments and errors as zs_reduce_shard; ZS_EINVAL also for
 * replicas < 1, round_to_reduce_dtype not 0/1, R * D > ZS_MAX_D, a scale
 * that is not finite, an unknown working_shard_hint or reserved != 0.
 */
zs_status zs_reduce_shard_ex(const void* const* contribs, int32_t D, const zs_reduce_opts* opts,
                             int32_t dtype, int64_t S, float* grad_out, hipStream_t stream);

/*
 * zs_adamw_step_ex -- zs_adamw_step with the reduce of zs_reduce_shard_ex:
 * the gradient is the grad_out value of zs_reduce_shard_ex for these
 * contributions and opts (never stored, scale included), then the AdamW
 * update of zs_adamw_step; the working shard is stored as
 * opts->working_shard_hint asks.
 * Arguments and errors as zs_adamw_step and zs_reduce_shard_ex.
 */
zs_status zs_adamw_step_ex(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                           const void* const* contribs, int32_t D, const zs_reduce_opts* opts,
                           int32_t dtype, const zs_adamw_hp* hp, hipStream_t stream);

/*
 * zs_adamw_step_timed -- zs_adamw_step_ex whose kernel carries two timing
 * events: a measurement aid for benchmarks and profilers, same arithmetic,
 * same results bit for bit.
 *
 * A step with S > 0 is exactly one kernel launch. This call makes it with
 * hipExtLaunchKernel, which has the runtime record `start` at that kernel's
 * start and `stop` at its end, with no marker packets enqueued around it, so
 * hipEventElapsedTime(start, stop) times the kernel itself. (On MI355X, over
 * the 70B shard's 0.7 ms launches, these events read 0.7% above a kernel
 * trace's durations; events recorded with hipEventRecord before and after
 * each launch read 0.9% above.)
 *
 *   start, stop  distinct events created by the caller on the current device
 *                with timing enabled (hipEventCreate); each is re-recorded by
 *                this call, as by hipEventRecord, and stays the caller's
 * Other arguments and errors as zs_adamw_step_ex; ZS_EINVAL also when start
 * or stop is NULL or they are the same event. With S == 0 nothing is
 * launched and the events are not touched.
 */
zs_status zs_adamw_step_timed(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                              const void* const* contribs, int32_t D, const zs_reduce_opts* opts,
                              int32_t dtype, const zs_adamw_hp* hp, hipEvent_t start,
                              hipEvent_t stop, hipStream_t stream);

/*
 * zs_gather_unit -- the local data movement of all-gather.
 *
 * [GPT8] "AllGather vs AllReduce": afterwards every rank holds all blocks in
 * rank order; [ZT] section 5.1 gathers a block's shards into its full
 * parameters before each forward and backward. For r < D, i < S:
 *   flat_out[r*S + i] = shards[r][i]   (bit copy, padding included)
 * Tensor j of the unit is then the view flat_out[off_j, off_j + numel_j).
 *
 *   shards    host array of D device pointers, each to S elements
 *   D         1..ZS_MAX_D
 *   S         >= 0
 *   dtype     ZS_BF16 or ZS_F32
 *   flat_out  device, D * S elements
 * In place: a shard whose pointer is exactly flat_out + r * S (its own slot,
 * as in an in-place all-gather, where each rank's shard lives inside the
 * unit buffer) is already where it belongs and is not copied.
 * Errors: ZS_EINVAL, ZS_EALIAS (a shard overlaps flat_out anywhere but
 * exactly in its own slot), ZS_EUNSUPPORTED.
 */
zs_status zs_gather_unit(const void* const* shards, int32_t D, int64_t S,
                         int32_t dtype, void* flat_out, hipStream_t stream);

/* One bucket of a rank's shard (one FSDP unit's slice) for the pipelined step. */
typedef struct {
    float* p;                    /* device, S floats: fp32 master, updated in place */
    float* m;                    /* device, S floats: first moment, in place        */
    float* v;                    /* device, S floats: second moment, in place       */
    uint16_t* w_out;             /* device, S bf16: working shard, written          */
    int64_t S;                   /* >= 0; 0 skips the bucket                        */
    const void* const* sources;  /* host array of n_contrib pointers, each to S
                                    elements of the reduce dtype, in device memory
                                    or pinned host memory; read only            */
} zs_bucket;

/*
 * zs_step_pipelined -- the shard step over a sequence of buckets, with the
 * arrival of each bucket's contributions overlapped with the previous
 * bucket's fused step.
 *
 * [ZT] section 5.4 and [GPT8] "Prefetching: Hiding the Cost": FSDP issues
 * the collective of the next block while the current block computes, so
 * communication hides behind compute. Here the reduce-scatter's transfer is
 * stood in for by copies of the n_contrib contributions of bucket b from
 * `sources` into a device staging slot (slots alternate between staging0
 * and staging1), enqueued on `transfer`; the fused step of bucket b (the
 * exact arithmetic of zs_adamw_step with these contributions) runs on
 * `compute` once its copies have landed, and the copies of the bucket after
 * next wait until that step has released the slot. The first copies wait
 * for all work already enqueued on `compute`. Results are bit-identical to
 * calling zs_adamw_step on every bucket in order.
 *
 *   buckets      host array of n_buckets bucket descriptors
 *   n_buckets    >= 0
 *   n_contrib    1..ZS_MAX_D contributions per bucket
 *   dtype        ZS_BF16 or ZS_F32: element type of sources and staging
 *   staging0/1   device, n_contrib * staging_len elements each; contribution
 *                q of a bucket lands at element q * staging_len of its slot
 *   staging_len  >= every bucket's S (a multiple of 8 keeps the full-speed
 *                kernel)
 *   hp           host pointer to the hyperparameters (one step for all buckets)
 *   compute      stream that runs the steps; when all work enqueued on it by
 *                this call has completed, every copy has completed too
 *   transfer     stream that runs the copies (may equal compute: no overlap)
 * Returns after enqueuing; nothing is synchronized and no device memory is
 * allocated. The five events that order the two streams come from a
 * per-device pool in the library (created on first use, reused by later
 * calls), so a call creates no runtime object once the pool holds them.
 * Errors: ZS_EINVAL (NULLs, misalignment, a bucket larger than staging_len,
 * hyperparameters), ZS_EALIAS (any two of the buckets' p, m, v, w_out and the
 * staging slots overlap, or a source overlaps one of them), ZS_EUNSUPPORTED,
 * ZS_EHIP (a runtime call failed; buckets before the failing one may already
 * be enqueued).
 */
zs_status zs_step_pipelined(const zs_bucket* buckets, int32_t n_buckets, int32_t n_contrib,
                            int32_t dtype, void* staging0, void* staging1, int64_t staging_len,
                            const zs_adamw_hp* hp, hipStream_t compute, hipStream_t transfer);

/*
 * zs_step_pipelined_static -- zs_step_pipelined for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The caller passes the buckets (inputs and
 * outputs) only; the staging slots live in a device array of the library
 * (two slots of 64 MiB, 128 MiB in all on each device that runs this call,
 * held until the process ends). A bucket whose n_contrib contributions do
 * not fit one slot is staged and stepped in pieces of at most
 * P = floor(64 MiB / (n_contrib * element size) / 1024) * 1024 elements
 * (P >= 262,144), so there is no limit on a bucket's size; the results are
 * bit-identical to zs_step_pipelined (and to zs_adamw_step on every bucket),
 * the step being elementwise. Sources may be device or pinned host memory.
 *
 * The first call on a device sets up that device's staging array address and
 * five events; no call allocates device memory or calls an allocating
 * library routine. Every call on one device shares the same staging array:
 * calls whose work overlaps in time on one device (enqueued on different
 * compute streams, or from several threads) race on it and on its events;
 * calls enqueued one after another on the same compute stream are ordered
 * (each call's first copies wait for all work already on `compute`).
 *
 *   buckets, n_buckets, n_contrib, dtype, hp, compute, transfer
 *                as zs_step_pipelined (no staging arguments)
 * Errors: as zs_step_pipelined; ZS_EHIP also when the staging array's
 * set-up fails.
 */
zs_status zs_step_pipelined_static(const zs_bucket* buckets, int32_t n_buckets,
                                   int32_t n_contrib, int32_t dtype, const zs_adamw_hp* hp,
                                   hipStream_t compute, hipStream_t transfer);

/*
 * zs_reshard -- re-shard one unit from D shards to D2 shards, on the device.
 *
 * [GPT8] "Checkpointing with FSDP": a sharded state dict resumes only on
 * the same GPU count, while the full (gathered) state dict loads on any
 * count. This is the full state dict's gather followed by a fresh split,
 * in one pass with no flat buffer: for new rank r2 and j < S2, with
 * i = r2 * S2 + j,
 *   dst[r2][j] = src[i / S][i % S]   if i < N   (bit copy)
 *   dst[r2][j] = +0                  if i >= N  (the new padding)
 *
 *   src   host array of D device pointers, each to S = ceil(N / D) elements
 *   dst   host array of D2 device pointers, each to S2 = ceil(N / D2)
 *   N     real (unpadded) elements of the unit, >= 0
 *   dtype ZS_BF16 or ZS_F32 (2- or 4-byte elements; p, m, v and w are
 *         re-sharded one array at a time)
 * Errors: ZS_EINVAL (counts out of range, S or S2 not the layout's, NULLs,
 * misalignment), ZS_EALIAS (a dst shard overlaps another dst or any src),
 * ZS_EUNSUPPORTED.
 */
zs_status zs_reshard(const void* const* src, int32_t D, int64_t S, int64_t N, int32_t dtype,
                     void* const* dst, int32_t D2, int64_t S2, hipStream_t stream);

/* Layout and step of one rank's shard checkpoint. S = ceil(N / D). */
typedef struct {
    int32_t rank;   /* 0 <= rank < D                      */
    int32_t D;      /* ranks the state was sharded over   */
    int64_t N;      /* real elements of the sharded state */
    int64_t S;      /* elements per rank shard            */
    int64_t step;   /* optimizer steps taken, >= 0        */
} zs_shard_info;

/*
 * Shard checkpoints: each rank saves its own shard (p, m, v fp32 and w
 * bf16, S elements each) to its own file -- [GPT8] "Checkpointing with
 * FSDP", sharded state dict, and "Shared Storage for Checkpoints": every
 * rank writes its own shard file concurrently. A checkpoint taken at D
 * ranks loads back at D (zs_shard_load) or at any D2
 * (zs_shard_load_resharded), each new rank reading only the byte ranges it
 * owns from the old files.
 *
 * File format (little-endian). Header page, bytes [0, 4096):
 *   0 char[8] "ZSSHARD1"   8 uint32 version (1)   12 uint32 header bytes (4096)
 *   16 int32 rank   20 int32 D   24 int64 N   32 int64 S   40 int64 step
 *   48 int64 CRC block bytes (16 MiB)
 *   56 + 48 i, i = 0..3 (p, m, v, w): char[8] name, int32 dtype (ZS_F32 or
 *      ZS_BF16), uint32 0, uint64 data offset, uint64 data bytes, uint64 CRC
 *      table offset, uint64 CRC blocks
 *   4092 uint32 CRC-32C of bytes [0, 4092)
 * then the four arrays at 4096-aligned offsets, then per array one uint32
 * CRC-32C (Castagnoli: reflected polynomial 0x82F63B78, initial value and
 * final xor 0xFFFFFFFF) per 16 MiB block of its data. A file is written as
 * path + ".tmp" and
 * renamed into place when complete.
 *
 * Unlike the kernel entry points these calls SYNCHRONIZE `stream` (the
 * state must be final before it is saved, and loaded data is complete
 * when they return), move data through a 64 MiB pinned host buffer they
 * allocate and free, and do file IO. The state pointers are device memory.
 * Errors: ZS_EINVAL (arguments), ZS_EALIAS (state arrays overlap), ZS_EIO
 * (open/read/write failure, bad magic, version or header, a checksum
 * mismatch, files that are not ranks 0..D-1 of one checkpoint), ZS_EHIP.
 */
zs_status zs_shard_save(const char* path, const zs_shard_info* info, const float* p,
                        const float* m, const float* v, const uint16_t* w, hipStream_t stream);
zs_status zs_shard_info_read(const char* path, zs_shard_info* info);
zs_status zs_shard_load(const char* path, float* p, float* m, float* v, uint16_t* w, int64_t S,
                        zs_shard_info* info_out, hipStream_t stream);
/* paths: host array of D file names, paths[r] = rank r's file of one
 * checkpoint; fills rank `rank` of a D2-way sharding (S2 = ceil(N / D2)),
 * the new padding +0; info_out (may be NULL) gets rank, D2, N, S2, step. */
zs_status zs_shard_load_resharded(const char* const* paths, int32_t D, int32_t rank, int32_t D2,
                                  float* p, float* m, float* v, uint16_t* w, int64_t S2,
                                  zs_shard_info* info_out, hipStream_t stream);

/*
 * zs_adamw_step_host -- the AdamW update of zs_adamw_step on HOST memory,
 * on host cores (ZeRO-Offload's optimizer step).
 *
 * [ZT] section 8: the Adam optimizer state moves to CPU memory; each step
 * the gradients go to the CPU and the updated weights come back. This is
 * that CPU step: for i < S, with g = grad[i] (the reduced fp32 gradient, as
 * zs_reduce_shard writes it), exactly the operations of zs_adamw_step with
 * one fp32 contribution, in the same order and rounding, so the results are
 * bit-identical to the device step. Runs synchronously on `threads` host
 * threads (the calling thread is one of them), vectorized with AVX2 where
 * the CPU has it; denormals are kept whatever the caller's MXCSR.
 *
 *   p, m, v  host, S floats, updated in place;  w_out host, S bf16, written
 *   grad     host, S floats, read
 *   threads  1..1024
 * Errors: ZS_EINVAL (NULLs, misalignment, threads, hyperparameters),
 * ZS_EALIAS (any two of p, m, v, w_out, grad overlap).
 */
zs_status zs_adamw_step_host(float* p, float* m, float* v, uint16_t* w_out, int64_t S,
                             const float* grad, const zs_adamw_hp* hp, int32_t threads);

/*
 * zs_offload_step -- one ZeRO-Offload shard step: reduce on the device,
 * gradient down, AdamW on host cores, working shard up.
 *
 * [ZT] section 8 (cost: gradients to the CPU and weights back over PCIe
 * every step). Enqueues the zs_reduce_shard reduce of the D device
 * contributions into grad_dev on `stream`, then copies grad_dev to
 * grad_host in chunks of `chunk` elements on `stream`; as each chunk lands
 * the host steps it (zs_adamw_step_host arithmetic on p, m, v, w_host) and
 * enqueues its copy w_host -> w_dev on `h2d_stream`. Returns when the host
 * work is done; the last working-shard copies may still be in flight on
 * h2d_stream (synchronize it before reading w_dev or rewriting w_host).
 * Results are bit-identical to zs_adamw_step on the same contributions.
 *
 *   contribs   host array of D device pointers, S elements of dtype each
 *   grad_dev   device, S floats (scratch, written)
 *   grad_host  host, S floats (written; pinned memory makes the copies async)
 *   p, m, v    host, S floats, updated in place
 *   w_host     host, S bf16 (written; pinned for async copies)
 *   w_dev      device, S bf16 (written by the copies)
 *   threads    1..1024 host threads;  chunk  >= 1 elements per pipeline chunk
 * Errors: as zs_reduce_shard and zs_adamw_step_host; ZS_EALIAS also when
 * grad_dev and w_dev overlap each other or a contribution.
 */
zs_status zs_offload_step(const void* const* contribs, int32_t D, int32_t dtype, int64_t S,
                          float* grad_dev, float* grad_host, float* p, float* m, float* v,
                          uint16_t* w_host, uint16_t* w_dev, const zs_adamw_hp* hp,
                          int32_t threads, int64_t chunk, hipStream_t stream,
                          hipStream_t h2d_stream);

/*
 * zs_stream_ceiling -- a measurement aid, not part of the step: moves the
 * fused step's exact memory streams with none of its arithmetic (reads n
 * contributions and p, m, v; writes p, m, v and w), with the fused kernel's
 * launch shape, lane map and cache hints, so that the step kernel can be
 * read against what HBM delivers for its own mix of streams. The values it
 * writes are placeholders: p, m, v and w are garbage afterwards. Processes
 * the first 1024 * floor(S / 1024) elements; every buffer 16-byte aligned.
 * Errors: ZS_EINVAL, ZS_EALIAS, ZS_EUNSUPPORTED as zs_adamw_step.
 */
zs_status zs_stream_ceiling(float* p, float* m, float* v, uint16_t* w, int64_t S,
                            const void* const* contribs, int32_t n, int32_t dtype,
                            hipStream_t stream);

/*
 * zs_stream_ceiling_timed -- zs_stream_ceiling whose one kernel launch records
 * `start` and `stop` at its own start and end, as zs_adamw_step_timed does
 * for the step, so that the two are timed alike.
 *   start, stop  as zs_adamw_step_timed
 * Errors: as zs_stream_ceiling; ZS_EINVAL also when start or stop is NULL or
 * they are the same event. With S < 1024 nothing is launched and the events
 * are not touched.
 */
zs_status zs_stream_ceiling_timed(float* p, float* m, float* v, uint16_t* w, int64_t S,
                                  const void* const* contribs, int32_t n, int32_t dtype,
                                  hipEvent_t start, hipEvent_t stop, hipStream_t stream);

/*
 * zs_hbm_probe -- a measurement aid, not part of the step: the memory
 * system's own rate for one stream direction, a copy or a triad, so that the
 * step kernel's mix of reads and writes can be read against what HBM gives
 * each direction alone and a plain mix with the same ratio. Non-temporal 16-byte vector accesses in grid-stride order, on a
 * grid of 256-thread workgroups that covers the buffer (blocks_per_cu = 0)
 * or on a persistent grid of blocks_per_cu workgroups per CU:
 *
 *   ZS_PROBE_READ   reads bytes of buf (two vectors per lane in flight); may
 *                   write 16 bytes at buf2 (a sink that keeps the loads)
 *   ZS_PROBE_WRITE  writes bytes of buf (element i of each 16-byte vector v:
 *                   {v mod 2^32, v >> 32, 0x5a5a5a5a, 0} as uint32 words)
 *   ZS_PROBE_COPY   copies bytes of buf to buf2
 *   ZS_PROBE_TRIAD  two reads per write, the fused step's ratio in three
 *                   streams: buf holds 2 * bytes, buf2[i] = buf[i] ^
 *                   buf[bytes + i] for the bytes of buf2 (XOR of 32-bit words)
 *
 *   bytes           a multiple of 16 (per stream); 0 returns ZS_OK with no launch
 *   buf, buf2       16-byte aligned device pointers; buf2 unused for WRITE;
 *                   for READ, COPY and TRIAD buf2 must not overlap buf
 *   blocks_per_cu   0..16
 * Errors: ZS_EINVAL (kind, sizes, alignment, NULL), ZS_EALIAS, ZS_EHIP.
 */
enum { ZS_PROBE_READ = 0, ZS_PROBE_WRITE = 1, ZS_PROBE_COPY = 2, ZS_PROBE_TRIAD = 3 };
zs_status zs_hbm_probe(int32_t kind, void* buf, void* buf2, int64_t bytes,
                       int32_t blocks_per_cu, hipStream_t stream);

/* Text of the calling thread's most recent failure ("" if none). The pointer
 * stays valid until the thread's next call into the library. */
const char* zs_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t zs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H_ */
