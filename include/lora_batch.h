/*
 * lora_batch.h -- C ABI of the multi-LoRA batched adapter library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method.  LoRA replaces the update of a frozen weight W in R^{d x k} by a
 * low-rank product Delta W = B A with A in R^{r x k} and B in R^{d x r}
 * (DeltaServe, section 2.2), so a layer computes h(x) = W x + B A x (MOLT,
 * section 2.1, displayed equation).  Multi-LoRA batching lets rows that use
 * different adapters share one base pass while each row applies the low-rank
 * weights of its own adapter (DeltaServe, section 2.2; the adapter-caching page
 * on kernel-level batching of several adapters).  A fine-tuning sample is an
 * ordinary batch entry routed to a reserved adapter (DeltaServe, section 3.2,
 * "Mixed forward batch"), and the fine-tuning backward computes the LoRA
 * gradients from the saved layer input (DeltaServe, section 3.2, "Backward
 * subprocess").  The caller computes the base output y0 = W x; this library
 * adds, for every row t bound to adapter a = a(t),
 *
 *     v_t = A_a x_t                      (lora_shrink,    fp32 [r_a])
 *     y_t += s_a * B_a v_t               (lora_expand_add)
 *
 * and for fine-tuning rows, given dY = dL/dy,
 *
 *     g_t = B_a^T dy_t,  dX_t += s_a A_a^T g_t,
 *     dA_a += s_a sum_t g_t x_t^T,  dB_a += s_a sum_t dy_t v_t^T   (lora_backward)
 *
 * s_a is a per-adapter multiplier (alpha / r; DeltaServe section 4.1 uses
 * alpha = 32 at r = 16, i.e. s = 2).
 *
 * Conventions shared by every call
 *   - Matrices are row-major.  d_in = k and d_out = d in the pages' notation.
 *     A_a is [r_a, d_in], B_a is [d_out, r_a]; x is [T, d_in] with row pitch
 *     ldx elements; y is [T, d_out] with pitch ldy.
 *   - Element type (lora_dtype) applies to x, y, dY, dX, A_a and B_a.  v, g,
 *     dA and dB are always fp32.  bf16 results (y, dX) are formed in fp32 and
 *     rounded once, to nearest even.
 *   - All data pointers are DEVICE pointers unless stated; the lora_segments
 *     struct itself is passed by value from the host and holds device
 *     pointers.  `stream` is a hipStream_t (NULL = the null stream).  Every
 *     compute call only enqueues work on `stream`; none synchronizes.
 *   - Ownership: the caller allocates and owns every buffer, including
 *     workspaces (sized by the *_workspace_bytes queries) and the
 *     device-resident adapter and gradient tables.  The library allocates no
 *     memory and keeps no mutable global state (the one exception is the
 *     static scratch of lora_shrink_noalloc); calls on different streams are
 *     independent when they use different output and workspace buffers.
 *   - Requirements checked on the host before anything is enqueued (a failing
 *     check returns a negative status and enqueues nothing):
 *       non-NULL required pointers; T >= 0; d_in, d_out >= 1; num_adapters >= 1;
 *       1 <= r_max <= LORA_MAX_RANK; leading dimensions >= the row length;
 *       x, y, dY, dX, v pointers 16-byte aligned; d_in, d_out and every
 *       element-matrix pitch a multiple of 8 (else LORA_ERR_UNSUPPORTED);
 *       fp32 pitches ldv a multiple of 8 and >= r_max; workspace large enough.
 *     T == 0 returns LORA_OK and enqueues nothing.
 *   - Data checked on the device: adapter ids outside [-1, num_adapters) and
 *     table entries with rank outside [1, r_max], a NULL or non-16-byte-aligned
 *     A/B pointer, or a NULL gradient entry for a trained adapter.  Such rows
 *     are skipped (never read or written out of bounds) and *seg.err is
 *     increased; a nonzero *seg.err after the stream completes means the call
 *     met bad data.  lora_segments_build sets *err to the number of bad ids;
 *     later calls on the same segments only add to it.
 *   - Rows with adapter id -1 carry no adapter: y and v rows are left as they
 *     are.
 *   - Results are deterministic: every reduction runs in a fixed order and no
 *     floating-point atomics are used, so repeated calls give identical bits.
 */
#ifndef LORA_BATCH_H
#define LORA_BATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 1
#define LORA_MAX_RANK 128

/* Status codes returned by every entry point. */
enum {
    LORA_OK = 0,
    LORA_ERR_INVALID_ARG = -1, /* bad pointer, size, pitch or enum */
    LORA_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels cover */
    LORA_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    LORA_ERR_HIP = -4,         /* a HIP launch failed */
    LORA_ERR_TOO_LARGE = -5    /* needs more than a no-allocation entry point's static scratch */
};

/* Element type of x, y, dY, dX, A and B. */
enum { LORA_BF16 = 0, LORA_F32 = 1 };

/* One adapter of the device-resident table (24 bytes).
 * A: [rank, d_in] and B: [d_out, rank], row-major, 16-byte aligned, element
 * type of the call.  scale multiplies the adapter's delta. */
typedef struct lora_adapter {
    const void* A;
    const void* B;
    int32_t rank;
    float scale;
} lora_adapter;

/* Gradient targets of one adapter (device table, 16 bytes).  dA: [rank, d_in]
 * and dB: [d_out, rank], fp32 row-major, accumulated into ("+=").  Entries of
 * adapters without fine-tuning rows may be NULL. */
typedef struct lora_adapter_grad {
    float* dA;
    float* dB;
} lora_adapter_grad;

/* Rows grouped by adapter (all device pointers, filled by lora_segments_build).
 *   counts [A]     rows per adapter
 *   offsets[A+1]   exclusive prefix sum of counts; offsets[A] = rows with a valid id
 *   perm   [T]     row indices grouped by adapter, ascending inside a group
 *                  (entries past offsets[A] are unspecified)
 *   err    [1]     device-side error count (see the conventions above)
 *   sched  [lora_segments_sched_elems(T, A)]  scheduling metadata read by the
 *                  compute kernels (tile prefix sums, active-adapter list);
 *                  opaque to the caller. */
typedef struct lora_segments {
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* err;
    int32_t* sched;
} lora_segments;

/* LORA_ABI_VERSION of the built library. */
int lora_abi_version(void);

/* Static, NUL-terminated description of a status code (host). */
const char* lora_status_string(int status);

/* Number of int32 elements of lora_segments.sched for T rows and
 * num_adapters adapters (host, pure).  sched must be 16-byte aligned. */
size_t lora_segments_sched_elems(int32_t T, int32_t num_adapters);

/* Workspace bytes of lora_segments_build (host, pure). */
size_t lora_segments_workspace_bytes(int32_t T, int32_t num_adapters);

/* Workspace bytes of lora_shrink (host, pure). */
size_t lora_shrink_workspace_bytes(int dtype, int32_t T, int32_t d_in, int32_t r_max);

/* Workspace bytes of lora_backward for T_ft rows (host, pure). */
size_t lora_backward_workspace_bytes(int dtype, int32_t T_ft, int32_t d_in, int32_t d_out, int32_t r_max);

/*
 * Group the rows of a batch by adapter: which weights each row applies
 * (DeltaServe, section 2.2, multi-LoRA batching; the reserved fine-tuning
 * adapter of section 3.2 is an ordinary id).
 *   adapter_ids [T] int32 device: a(t) in [0, num_adapters), or -1 for none.
 *   seg: output buffers (see lora_segments).  ws: device workspace of
 *   lora_segments_workspace_bytes(T, num_adapters) bytes; its contents on
 *   entry do not matter.
 * Integer outputs are exact and unique (stable grouping).  Three kernels.
 */
int lora_segments_build(const int32_t* adapter_ids, int32_t T, int32_t num_adapters,
                        lora_segments seg, void* ws, size_t ws_bytes, void* stream);

/* One build of lora_segments_build_batch (all pointers device, as in
 * lora_segments_build; the struct array itself lives in host memory). */
typedef struct lora_segments_job {
    const int32_t* adapter_ids; /* [T] */
    int32_t T;
    lora_segments seg;
    void* ws;                   /* lora_segments_workspace_bytes(T, num_adapters) bytes */
    size_t ws_bytes;
} lora_segments_job;

/* Builds per launch of lora_segments_build_batch's one-workgroup path. */
#define LORA_SEG_BATCH_MAX 8

/*
 * Several independent lora_segments_build calls over the same adapter table
 * size, enqueued together: builds of up to 65536 rows (and num_adapters <=
 * 1024) share one launch, one workgroup each, LORA_SEG_BATCH_MAX per launch;
 * larger ones take the three-kernel path one after the other.  Typical use:
 * the whole mixed batch and its fine-tuning rows (the rows the backward
 * reads), which multi-LoRA co-serving groups separately (DeltaServe, sections
 * 2.2 and 3.2).  Outputs are identical to one lora_segments_build per job.
 * Every job is checked on the host first; if any check fails nothing is
 * enqueued and its status is returned.  jobs: host array of n_jobs >= 0
 * entries (NULL allowed when n_jobs == 0); jobs with T == 0 are skipped.
 * The jobs must not share output or workspace buffers.
 */
int lora_segments_build_batch(const lora_segments_job* jobs, int32_t n_jobs, int32_t num_adapters, void* stream);

/*
 * Shrink: v_t = A_{a(t)} x_t with fp32 accumulation, for every row with an
 * adapter (the "A x" of h(x) = W x + B A x, MOLT section 2.1).
 *   x [T, ldx] (dtype), adapters [num_adapters] device table, seg from
 *   lora_segments_build over the same T rows, v [T, ldv] fp32 output
 *   (ldv >= r_max, multiple of 8).  Row t of v receives columns 0..r_a-1
 *   and zeros in columns r_a..round_up(r_a, 8)-1; rows without an adapter
 *   are left unchanged.  ws: lora_shrink_workspace_bytes(dtype, T, d_in, r_max)
 *   bytes of device memory (the sum over d_in is split into slices of 512
 *   (bf16) or 256 (fp32) elements whose partials are added in slice order:
 *   two kernels).  bf16 batches with at most 32 rows per adapter on average,
 *   or with r_max <= 16, take one kernel on 16-row tiles that sums all of
 *   d_in per tile in a fixed order and writes v directly (ws is checked but
 *   not used).  Either way the sum order is fixed: results are
 *   bit-reproducible.
 */
int lora_shrink(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                const lora_adapter* adapters, int32_t num_adapters, int32_t r_max,
                lora_segments seg, float* v, int64_t ldv, void* ws, size_t ws_bytes, void* stream);

/*
 * lora_shrink without a workspace argument, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses that
 * forbid allocation.  The split-K partials live in a static device array of
 * the library, LORA_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs
 * on, held until the process ends; its device address is looked up once per
 * device (on the first call that runs on it, that device made current and the
 * caller's current device restored afterwards).  This call allocates nothing.
 *   Arguments, results and errors as for lora_shrink (the kernels are the
 *   same, so results are bit-identical to lora_shrink's); additionally
 *   LORA_ERR_TOO_LARGE when lora_shrink_workspace_bytes(dtype, T, d_in, r_max)
 *   exceeds LORA_NOALLOC_SCRATCH_BYTES, before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (other streams, other threads) race on it and must be ordered by
 * the caller.  Nothing in the scratch needs to start at zero (every partial
 * is written before it is read); it keeps the last call's contents.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (32u << 20)

int lora_shrink_noalloc(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                        const lora_adapter* adapters, int32_t num_adapters, int32_t r_max,
                        lora_segments seg, float* v, int64_t ldv, void* stream);

/*
 * Expand-add: y_t += s_{a(t)} B_{a(t)} v_t, computed in fp32 and rounded once to
 * the element type; the delta is added to the caller's base output (the
 * adapter-caching page: the adapter's activations are added to the backbone
 * layer's outputs).
 *   v [T, ldv] fp32 from lora_shrink; y [T, ldy] (dtype) in/out.
 *   Only columns 0..r_a-1 of each v row are read.
 */
int lora_expand_add(int dtype, const float* v, int64_t ldv, int32_t T, int32_t d_out,
                    const lora_adapter* adapters, int32_t num_adapters, int32_t r_max,
                    lora_segments seg, void* y, int64_t ldy, void* stream);

/*
 * Forward in one call: y_t += s_{a(t)} B_{a(t)} (A_{a(t)} x_t), the whole
 * h(x) = W x + B A x delta of MOLT section 2.1 for every row with an adapter,
 * without a workspace.  The call takes the fastest kernel sequence its
 * arguments allow (decode batch: bf16 with at most 32 rows per adapter on
 * average):
 *   - decode batch, r_max <= 16: one launch, 16-row tiles, one workgroup per
 *     (tile, column range) with every load of the tile in flight at once, v
 *     kept in LDS (256 decode rows over 64 rank-16 adapters, 4096 -> 4096:
 *     12.9 us against 18.3 us for lora_shrink + lora_expand_add);
 *   - otherwise, with v given, on a decode batch or at r_max <= 16 (bf16):
 *     the split calls' kernels that need no workspace, the 16-row-tile shrink
 *     into v, then the expand; results equal lora_shrink + lora_expand_add
 *     bit for bit;
 *   - otherwise: one launch, 64-row tiles (v = A x over all of d_in in LDS,
 *     then a range of d_out's columns).  On long row groups with r_max > 16
 *     this is slower than the split calls (2.2x on the mixed prefill / decode
 *     / fine-tuning batch at 4096 -> 14336, whose split-K shrink spreads x
 *     over the whole chip), as it is wherever the other routes apply and v
 *     is not given (1.6x on 4096 fine-tuning rows at rank 16, 2.8x on 2048
 *     decode rows over 320 adapters of ranks 8..128).
 * The one-launch routes equal lora_shrink + lora_expand_add up to the order
 * of the fp32 sum over d_in (a fixed order: bit-reproducible).
 *   x [T, ldx], y [T, ldy] in/out (dtype); adapters, seg as for lora_shrink.
 *   v: optional [T, ldv] fp32 output (ldv >= r_max, multiple of 8), written as
 *   lora_shrink writes it (columns r_a..round_up(r_a, 8)-1 zero; rows without
 *   an adapter unchanged), e.g. for a later lora_backward; NULL skips it.
 * Errors and device-side data checks as for lora_shrink / lora_expand_add
 * (a bad table entry is counted once per tile by each kernel that meets it).
 */
int lora_forward(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, int32_t d_out,
                 const lora_adapter* adapters, int32_t num_adapters, int32_t r_max, lora_segments seg,
                 void* y, int64_t ldy, float* v, int64_t ldv, void* stream);

/*
 * Multi-slice fused forward: several projections that read the same x, each
 * with its own adapters.  DeltaServe (section 4.1) adapts all attention
 * projections of a layer; the q, k and v projections (or the gate and up
 * projections of an MLP) read one input, so the one-launch kernels read x
 * once per tile for all of them and keep v = A x of every slice in LDS.  For
 * each slice q and each row t with adapter a = a(t) (the same adapter index
 * in every slice):
 *     y_q[t] += s_{q,a} B_{q,a} (A_{q,a} x_t),
 * exactly what lora_forward computes for that slice alone with the same
 * arguments (bit for bit).  The slices take lora_forward's routes: on a
 * decode batch with r_max <= 16 all of them run in one 16-row-tile launch;
 * otherwise each slice given v runs the split kernels where lora_forward
 * would (decode batch or r_max <= 16), and the remaining slices run in one
 * 64-row-tile launch.
 *   slices: HOST array of n_slices (1..LORA_MAX_SLICES) entries:
 *     adapters  device table [num_adapters] of the slice (A [r, d_in],
 *               B [d_out, r]; ranks may differ between slices);
 *     y [T, ldy] in/out (dtype) with d_out columns; v optional as in
 *     lora_forward; d_out >= 1; reserved must be 0.
 *   r_max: the largest rank over every slice's adapters.
 * Errors as for lora_forward; LORA_ERR_UNSUPPORTED for n_slices > 1 with
 * r_max > 64 (the slices' v rows and fragments would not fit the LDS).
 * Bad table entries are counted in seg.err as lora_forward counts them for
 * each slice (once per slice, tile and kernel that meets them), and only
 * that slice's rows are skipped.
 */
#define LORA_MAX_SLICES 3

typedef struct {
    const lora_adapter* adapters;
    void* y;
    int64_t ldy;
    float* v;
    int64_t ldv;
    int32_t d_out;
    int32_t reserved;
} lora_slice;

int lora_forward_multi(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                       const lora_slice* slices, int32_t n_slices, int32_t num_adapters, int32_t r_max,
                       lora_segments seg, void* stream);

/*
 * LoRA backward over T_ft fine-tuning rows (DeltaServe, section 3.2: the
 * backward computes the LoRA gradients from the saved layer input).
 *   x  [T_ft, ldx]  layer input of the fine-tuning rows (dtype)
 *   dy [T_ft, lddy] dL/dy of those rows (dtype)
 *   dx [T_ft, lddx] in/out, dX += s A^T B^T dy (dtype); NULL skips dX
 *   grads [num_adapters] device table; dA_a += s (B_a^T dy) x^T and
 *         dB_a += s dy (A_a x)^T, summed over the rows of adapter a (fp32)
 *   seg_ft: lora_segments_build over the fine-tuning rows' ids (row indices
 *         0..T_ft-1 refer to x, dy, dx)
 *   v_saved [T_ft, ldv] fp32: v = A x of these rows as lora_shrink wrote it,
 *         or NULL to recompute it from x
 *   ws: lora_backward_workspace_bytes(dtype, T_ft, d_in, d_out, r_max) bytes
 *         of device memory.
 * The caller passes a compact view of the fine-tuning rows; a contiguous
 * fine-tuning tail of a mixed batch is passed by pointer offset, no copy.
 */
int lora_backward(int dtype, const void* x, int64_t ldx, const void* dy, int64_t lddy,
                  void* dx, int64_t lddx, int32_t T_ft, int32_t d_in, int32_t d_out,
                  const lora_adapter* adapters, const lora_adapter_grad* grads,
                  int32_t num_adapters, int32_t r_max, lora_segments seg_ft,
                  const float* v_saved, int64_t ldv, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * lora_backward that yields to inference.  DeltaServe (section 3.4, backward
 * preemption) lets its backward run next to decode steps and preempts it for
 * prefill through a shared GPU-grant flag that the backward checks at every
 * layer boundary: the inference side clears the flag before a step with
 * prefill rows and sets it again afterwards.  Here the flag is checked on the
 * device at the start of the call and, when v_saved is NULL, again after the
 * recompute of v; every kernel that writes dA, dB or dX runs after the last
 * check.
 *   grant: int32 readable by the device (device memory, or host memory mapped
 *          for the device), read with system-scope loads; nonzero = granted.
 *   status: device int32, written by the call: 0 = the backward ran to the
 *          end; 1 = it yielded: the grant was zero at a check, and dA, dB and
 *          dX are left exactly as they were (the kernels after a check that
 *          yielded skip their work, so the outputs are written completely or
 *          not at all).  The caller re-issues the call once granted again.
 *          Read it after the call has completed on the stream.
 * Other arguments, results and errors as for lora_backward; additionally
 * LORA_ERR_INVALID_ARG for a NULL or misaligned grant / status.  With
 * T_ft == 0 nothing is enqueued and status is not written.
 */
int lora_backward_preemptible(int dtype, const void* x, int64_t ldx, const void* dy, int64_t lddy,
                              void* dx, int64_t lddx, int32_t T_ft, int32_t d_in, int32_t d_out,
                              const lora_adapter* adapters, const lora_adapter_grad* grads,
                              int32_t num_adapters, int32_t r_max, lora_segments seg_ft,
                              const float* v_saved, int64_t ldv, void* ws, size_t ws_bytes,
                              const int32_t* grant, int32_t* status, void* stream);

/*
 * AdamW step on adapter weights.  The fine-tuning applies its optimizer to the
 * shared adapter weights in place once the gradients of a backward batch have
 * been accumulated (DeltaServe, section 3.2, "Backward subprocess"); the
 * optimizer is AdamW with learning rate 1e-3 and weight decay 0.01 (DeltaServe,
 * section 4.1), i.e. Adam with decoupled weight decay.  For step t >= 1, for
 * every element of every listed tensor, in fp32:
 *     g = grad_scale * grad
 *     m = beta1 m + (1 - beta1) g
 *     v = beta2 v + (1 - beta2) g^2
 *     w = w (1 - lr weight_decay) - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * (the bias corrections are computed in double on the host).
 *   tensors: HOST array of n_tensors (0..LORA_ADAMW_MAX_TENSORS) entries, e.g.
 *     dA and dB of each trained adapter (one launch for all of them):
 *     w      [n] dtype, the weights (A_a or B_a), updated in place;
 *     master [n] fp32 master copy or NULL.  With a master, the update reads
 *            and writes the master and w receives its rounding (bf16: round
 *            to nearest even); without one, w itself is read and rounded;
 *     grad   [n] fp32 accumulated gradient (dA_a or dB_a from lora_backward);
 *            set to zero after it is read when hp.zero_grad != 0;
 *     m, v   [n] fp32 moments (zero before step 1), updated in place;
 *     n      element count (n = 0 entries are skipped).
 *   Every non-NULL pointer 16-byte aligned; the arrays of one entry must not
 *   overlap each other or those of another entry.
 *   hp: lr >= 0, 0 <= beta1, beta2 < 1, eps > 0, weight_decay >= 0, all
 *   finite; step >= 1.  Defaults of the pages' fine-tuning: lr 1e-3,
 *   weight_decay 0.01; beta1 0.9, beta2 0.999, eps 1e-8 (not stated there).
 * Errors: LORA_ERR_INVALID_ARG for a bad dtype, count, pointer, alignment or
 * hyper-parameter, before anything is enqueued.  One kernel.
 */
#define LORA_ADAMW_MAX_TENSORS 32

typedef struct {
    void* w;
    float* master;
    float* grad;
    float* m;
    float* v;
    int64_t n;
} lora_adamw_tensor;

typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    float grad_scale;
    int32_t step;
    int32_t zero_grad;
} lora_adamw_params;

int lora_adamw_step(int dtype, const lora_adamw_tensor* tensors, int32_t n_tensors, lora_adamw_params hp,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_BATCH_H */
